"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Masks are compared bit for bit on every row, near-tie rows included (see
parity.py); outputs within max-abs 2e-2 and mean-abs 2e-3 of the float64
oracle. Small shapes are compared in full (several tiles and a ragged tail in
both the query and the key direction); the full-size workloads compare every
mask row and a seeded sample of query blocks of the output (heads from every
group of the workload), in the launch configuration the benchmark times, and
check that every element of every head's output was written (outputs are
pre-filled with NaN).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_softmax_amd import binding as S
from block_sparse_attention_softmax_amd.workloads import WORKLOADS, generate
from oracle import sparge_oracle as O
from parity import (assert_all_written, check_bit_padding, check_index_list, compare_masks,
                    compare_outputs, gpu_bits_to_bool, nan_like, sentinel_mask_outputs, to_gpu)

pytestmark = pytest.mark.gpu

_CACHE = {}


def workload_tensors(name):
    if name not in _CACHE:
        _CACHE.clear()
        wl = WORKLOADS[name]
        Q, K, V = generate(wl)
        _CACHE[name] = (wl, Q, K, V, to_gpu(Q), to_gpu(K), to_gpu(V))
    return _CACHE[name]


def run_mask(wl, q, k, k_frac=None, p_mass=None):
    k_frac = wl.k_frac if k_frac is None else k_frac
    p_mass = wl.p_mass if p_mass is None else p_mass
    out = sentinel_mask_outputs(wl.B, wl.H, wl.n_q, wl.n_k, q.device)
    bits, idx, cnt, logits = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, k_frac, p_mass,
                                                   wl.scale, return_logits=True, out=out)
    torch.cuda.synchronize()
    n_k = wl.n_k
    check_bit_padding(bits, n_k)
    kept = gpu_bits_to_bool(bits, n_k)
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    check_index_list(kept, idx_np, cnt_np)
    return kept, idx, cnt, logits.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "wan1.3b", "wan1.3b_s95", "wan14b_720p"])
def test_mask_matches_oracle(name):
    wl, Q, K, V, q, k, v = workload_tensors(name)
    print(f"\n[mask] {name} B={wl.B} H={wl.H} N={wl.N} d={wl.d}", flush=True)
    kept, idx, cnt, logits = run_mask(wl, q, k)
    m = O.predict_mask(Q, K, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass, wl.scale)
    np.testing.assert_allclose(logits, m.logits, rtol=1e-12, atol=1e-12)
    ties, differ = compare_masks(m, kept, wl.k_frac, wl.p_mass)
    sparsity = 1 - kept.sum() / kept.size
    print(f"[mask] {name}: sparsity {sparsity:.4f} near-tie rows {ties} differing {differ}",
          flush=True)


@pytest.mark.parametrize("B,H,N,d,bq,k_frac,p_mass", [
    (1, 2, 5000, 128, 128, 0.1, 0.5),      # n_k 79   -> sort width 128
    (2, 1, 12345, 64, 64, 0.02, 0.95),     # n_k 193  -> 256
    (1, 1, 60000, 64, 128, 0.05, 0.0),     # n_k 938  -> 1024, Top-k alone (469 rows: LDS sort)
    (1, 2, 40000, 64, 64, 0.05, 0.9),      # n_k 625  -> 1024, 1250 rows: register sort
    (2, 1, 70000, 64, 128, 0.03, 0.8),     # n_k 1094 -> 2048, 1094 rows: register sort
    (1, 1, 100000, 64, 128, 0.02, 0.9),    # n_k 1563 -> 2048, 782 rows: LDS sort
    (1, 1, 200000, 64, 128, 0.01, 0.7),    # n_k 3125 -> 4096 (the largest supported width)
    (1, 3, 777, 128, 64, 1.0, 0.9),        # k = 100% keeps everything
    (1, 2, 3000, 64, 64, 0.2, 1.0)])       # p >= 1 keeps everything
def test_mask_matches_oracle_across_sort_widths(B, H, N, d, bq, k_frac, p_mass):
    rng = np.random.default_rng(N)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    # a smooth trend along the sequence makes the rows far from uniform
    trend = np.sin(np.arange(N) / 700.0)[None, None, :, None] * rng.standard_normal(d)
    Q, K = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d)) + 3 * trend) for _ in range(2))
    scale = S.default_scale(d)
    print(f"\n[mask] B={B} H={H} N={N} d={d} bq={bq} k={k_frac} p={p_mass}", flush=True)
    n_k = -(-N // 64)
    out = sentinel_mask_outputs(B, H, -(-N // bq), n_k, "cuda")
    bits, idx, cnt, logits = S.sparge_mask_predict(to_gpu(Q), to_gpu(K), bq, 64, k_frac, p_mass,
                                                   scale, return_logits=True, out=out)
    torch.cuda.synchronize()
    check_bit_padding(bits, n_k)
    kept = gpu_bits_to_bool(bits, n_k)
    check_index_list(kept, idx.cpu().numpy(), cnt.cpu().numpy())
    m = O.predict_mask(Q, K, bq, 64, k_frac, p_mass, scale)
    np.testing.assert_allclose(logits.cpu().numpy(), m.logits, rtol=1e-12, atol=1e-12)
    ties, differ = compare_masks(m, kept, k_frac, p_mass)
    print(f"[mask] kept {kept.mean():.4f} near-tie rows {ties} differing {differ}", flush=True)


@pytest.mark.parametrize("k_frac", [0.10, 0.05])
def test_mask_topk_only_operating_points(k_frac):
    """p = 0 (Top-k alone): the 90% and 95% block-sparsity points on wan1.3b inputs."""
    wl, Q, K, V, q, k, v = workload_tensors("wan1.3b")
    kept, idx, cnt, logits = run_mask(wl, q, k, k_frac=k_frac, p_mass=0.0)
    m = O.predict_mask(Q, K, wl.block_q, wl.block_k, k_frac, 0.0, wl.scale)
    compare_masks(m, kept, k_frac, 0.0)
    assert (cnt.cpu().numpy() == O.topk_size(k_frac, wl.n_k)).all()


def test_uniform_rows_keep_lowest_indices():
    """Q = 0 gives exactly equal block scores: Top-p(0.9) keeps 15 of 16 blocks, ties to the
    lower index (the uniform-row case of the SpargeAttention2 page, section 1)."""
    B, H, N, d = 1, 2, 1024, 64
    g = torch.Generator().manual_seed(0)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16).cuda()
    k = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).cuda()
    bits, idx, cnt = S.sparge_mask_predict(q, k, 64, 64, 0.1, 0.9)
    assert (cnt.cpu() == 15).all()
    assert (idx.cpu()[..., :15] == torch.arange(15, dtype=torch.int32)).all()
    bits, idx, cnt = S.sparge_mask_predict(q, k, 64, 64, 0.1, 0.0)
    assert (cnt.cpu() == 2).all()
    assert (idx.cpu()[..., :2] == torch.tensor([0, 1], dtype=torch.int32)).all()


# ------------------------------------------------- routed mask (SLA2 router)
@pytest.mark.parametrize("name,k_frac,p_mass", [("tiny", None, None), ("wan1.3b", None, None),
                                                ("wan1.3b", 0.10, 0.0)])
def test_routed_mask_matches_oracle(name, k_frac, p_mass):
    from block_sparse_attention_softmax_amd.workloads import router_weights
    wl, Q, K, V, q, k, v = workload_tensors(name)
    k_frac = wl.k_frac if k_frac is None else k_frac
    p_mass = wl.p_mass if p_mass is None else p_mass
    wq, wk = router_weights(wl.H, wl.d, 77)
    bits, idx, cnt, logits = S.sparge_mask_predict_routed(
        q, k, torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda(), wl.block_q, wl.block_k,
        k_frac, p_mass, wl.scale, return_logits=True,
        out=sentinel_mask_outputs(wl.B, wl.H, wl.n_q, wl.n_k, q.device))
    torch.cuda.synchronize()
    check_bit_padding(bits, wl.n_k)
    kept = gpu_bits_to_bool(bits, wl.n_k)
    check_index_list(kept, idx.cpu().numpy(), cnt.cpu().numpy())
    m = O.predict_mask_routed(Q, K, wq, wk, wl.block_q, wl.block_k, k_frac, p_mass, wl.scale)
    np.testing.assert_allclose(logits.cpu().numpy(), m.logits, rtol=1e-12, atol=1e-12)
    ties, differ = compare_masks(m, kept, k_frac, p_mass)
    print(f"\n[routed mask] {name} k={k_frac} p={p_mass}: sparsity {1 - kept.mean():.4f} "
          f"near-tie rows {ties} differing {differ}", flush=True)


def test_routed_mask_with_identity_weights_is_the_plain_mask():
    wl, Q, K, V, q, k, v = workload_tensors("wan1.3b")
    eye = torch.eye(wl.d, dtype=torch.float32, device="cuda").expand(wl.H, wl.d, wl.d)
    r = S.sparge_mask_predict_routed(q, k, eye.contiguous(), eye.contiguous(), wl.block_q,
                                     wl.block_k, wl.k_frac, wl.p_mass, wl.scale)
    p = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(r[0], p[0]) and torch.equal(r[2], p[2])


# --------------------------------------------------------------- attention
def _random_lists(rng, B, H, n_q, n_k):
    kept = rng.random((B, H, n_q, n_k)) < rng.uniform(0.05, 0.7)
    flat = kept.reshape(-1, n_k)
    flat[0] = False                      # an empty row -> zeros
    if flat.shape[0] > 1:
        flat[1] = True                   # a dense row
    if flat.shape[0] > 2:
        flat[2] = False
        flat[2, n_k - 1] = True          # only the short last block
    return kept


@pytest.mark.parametrize("B,H,N,d,bq", [
    (1, 2, 1000, 128, 128), (2, 1, 1000, 64, 64), (1, 3, 777, 128, 64),
    (1, 2, 300, 64, 128), (1, 1, 50, 128, 128), (2, 2, 1, 64, 64), (1, 1, 4096, 128, 128)])
def test_attention_small_shapes_in_full(B, H, N, d, bq):
    rng = np.random.default_rng(N + d + bq)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d)) * 1.5) for _ in range(3))
    n_q, n_k = -(-N // bq), -(-N // 64)
    kept = _random_lists(rng, B, H, n_q, n_k)
    idx, cnt = O.kept_to_index_list(kept)
    print(f"\n[attn] B={B} H={H} N={N} d={d} bq={bq}", flush=True)
    o = S.sparge_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), bq, 64, None)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref = O.masked_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                          O.bf16_to_f64(V[b, h]), kept[b, h], bq, 64, scale)
            compare_outputs(got[b, h], ref)


@pytest.mark.parametrize("N,d,bq,k_frac,p_mass", [
    (1, 64, 64, 0.1, 0.9), (37, 128, 128, 0.5, 0.0), (64, 64, 64, 0.3, 0.5),
    (65, 128, 64, 0.2, 0.9), (129, 64, 128, 0.05, 1.0), (200, 128, 128, 1.0, 0.0)])
def test_mask_and_attention_at_tiny_lengths(N, d, bq, k_frac, p_mass):
    """The whole path where the sequence is at most a few blocks: one block,
    a short only block, exact multiples and a one-token last block."""
    rng = np.random.default_rng(7 * N + d)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    B, H = 2, 2
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    scale = S.default_scale(d)
    q, k, v = to_gpu(Q), to_gpu(K), to_gpu(V)
    n_k = -(-N // 64)
    out = sentinel_mask_outputs(B, H, -(-N // bq), n_k, q.device)[:3]
    bits, idx, cnt = S.sparge_mask_predict(q, k, bq, 64, k_frac, p_mass, scale, out=out)
    o = S.sparge_attn_fwd(q, k, v, idx, cnt, bq, 64, scale, out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(o)
    check_bit_padding(bits, n_k)
    kept = gpu_bits_to_bool(bits, n_k)
    check_index_list(kept, idx.cpu().numpy(), cnt.cpu().numpy())
    m = O.predict_mask(Q, K, bq, 64, k_frac, p_mass, scale)
    ties, differ = compare_masks(m, kept, k_frac, p_mass)
    print(f"\n[tiny] N={N} d={d} bq={bq} k={k_frac} p={p_mass}: near-tie rows {ties} "
          f"differing {differ}", flush=True)
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    for b in range(B):
        for h in range(H):
            ref = O.masked_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                          O.bf16_to_f64(V[b, h]), kept[b, h], bq, 64, scale)
            compare_outputs(got[b, h], ref)


def test_pack_then_packed_equals_one_call():
    wl, Q, K, V, q, k, v = workload_tensors("tiny")
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass)
    o1 = S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q, wl.block_k)
    ws = S.sparge_attn_pack(v)
    o2 = S.sparge_attn_fwd_packed(q, k, idx, cnt, ws, wl.block_q, wl.block_k)
    o3 = S.sparge_attn_fwd_packed(q, k, idx, cnt, ws, wl.block_q, wl.block_k)  # reuse
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_attention_is_deterministic():
    wl, Q, K, V, q, k, v = workload_tensors("tiny")
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass)
    o1 = S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q, wl.block_k)
    o2 = S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q, wl.block_k)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def sample_heads(name, H, rng, n=4):
    """Heads to compare on a workload: wan1.3b_s95 takes half from its
    near-uniform heads (0-5) and half from its sink heads (6-11)."""
    if name == "wan1.3b_s95":
        half = H // 2
        return sorted([*rng.choice(half, n // 2, replace=False),
                       *(half + rng.choice(H - half, n - n // 2, replace=False))])
    return sorted(rng.choice(H, size=min(n, H), replace=False))


@pytest.mark.parametrize("name,samples", [("tiny", None), ("wan1.3b", 8), ("wan1.3b_s95", 8),
                                          ("wan14b_720p", 6)])
def test_attention_matches_oracle_on_workloads(name, samples):
    """Mask and attention as the benchmark runs them; the oracle uses the GPU's mask.
    Every element of every head is checked to have been written."""
    wl, Q, K, V, q, k, v = workload_tensors(name)
    print(f"\n[attn] {name}", flush=True)
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass)
    o = S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q, wl.block_k, out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(o)
    kept = gpu_bits_to_bool(bits, wl.n_k)
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    rng = np.random.default_rng(2024)
    for b in range(wl.B):
        heads = range(wl.H) if samples is None else sample_heads(name, wl.H, rng)
        for h in heads:
            if samples is None:
                blocks = None
            else:  # always the first and the short last block, plus a seeded sample
                blocks = sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, samples - 2, replace=False)})
            ref = O.masked_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                          O.bf16_to_f64(V[b, h]), kept[b, h], wl.block_q,
                                          wl.block_k, wl.scale, q_blocks=blocks)
            rows = ~np.isnan(ref[:, 0])
            mx, mean = compare_outputs(got[b, h][rows], ref[rows])
            print(f"[attn] {name} b={b} h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("k_frac", [0.10, 0.05])
def test_attention_matches_oracle_at_topk_operating_points(k_frac):
    """The 90% / 95% block-sparsity points the benchmark times (p = 0, Top-k alone),
    sampled query blocks of two heads against the oracle."""
    wl, Q, K, V, q, k, v = workload_tensors("wan1.3b")
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, k_frac, 0.0)
    ws = S.sparge_attn_pack(v)
    o = S.sparge_attn_fwd_packed(q, k, idx, cnt, ws, wl.block_q, wl.block_k, out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(o)
    kept = gpu_bits_to_bool(bits, wl.n_k)
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    rng = np.random.default_rng(int(k_frac * 1000))
    for h in sample_heads("wan1.3b", wl.H, rng):
        blocks = sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, 6, replace=False)})
        ref = O.masked_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                      O.bf16_to_f64(V[0, h]), kept[0, h], wl.block_q,
                                      wl.block_k, wl.scale, q_blocks=blocks)
        rows = ~np.isnan(ref[:, 0])
        mx, mean = compare_outputs(got[0, h][rows], ref[rows])
        print(f"[attn k={k_frac}] h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


def test_attention_accepts_lists_in_any_order():
    """kv_idx rows need not be sorted: a permuted list gives the oracle's result."""
    B, H, N, d, bq = 1, 2, 2000, 128, 128
    rng = np.random.default_rng(99)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d)) * 1.5) for _ in range(3))
    n_q, n_k = -(-N // bq), -(-N // 64)
    kept = _random_lists(rng, B, H, n_q, n_k)
    idx, cnt = O.kept_to_index_list(kept)
    for row in np.ndindex(B, H, n_q):
        idx[row][: cnt[row]] = rng.permutation(idx[row][: cnt[row]])
    o = S.sparge_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), bq, 64, None)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    for h in range(H):
        ref = O.masked_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                      O.bf16_to_f64(V[0, h]), kept[0, h], bq, 64,
                                      S.default_scale(d))
        compare_outputs(got[0, h], ref)


def test_attention_long_rows_sampled():
    """N = 200000 (3125 key blocks): rows listing up to every block, so the kernel
    walks lists far longer than its 128-entry index windows; sampled query
    blocks against the oracle."""
    B, H, N, d, bq = 1, 1, 200000, 128, 128
    rng = np.random.default_rng(200000)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // bq), -(-N // 64)
    kept = rng.random((B, H, n_q, n_k)) < 0.3
    kept[0, 0, 0] = True                   # every block
    kept[0, 0, n_q - 1] = False
    kept[0, 0, n_q - 1, n_k - 1] = True    # only the short last key block
    idx, cnt = O.kept_to_index_list(kept)
    qg = to_gpu(Q)
    o = S.sparge_attn_fwd(qg, to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), bq, 64, None, out=nan_like(qg))
    torch.cuda.synchronize()
    assert_all_written(o)
    got = O.bf16_to_f64(o[0, 0].cpu().view(torch.uint16).numpy())
    blocks = sorted({0, 1, n_q // 2, n_q - 1})
    ref = O.masked_attention_head(O.bf16_to_f64(Q[0, 0]), O.bf16_to_f64(K[0, 0]),
                                  O.bf16_to_f64(V[0, 0]), kept[0, 0], bq, 64,
                                  S.default_scale(d), q_blocks=blocks)
    rows = ~np.isnan(ref[:, 0])
    mx, mean = compare_outputs(got[rows], ref[rows])
    print(f"[attn long rows] max {mx:.2e} mean {mean:.2e}", flush=True)


# ------------------------------------------------------------ linear branch
@pytest.mark.parametrize("B,H,N,d,bq", [(1, 2, 1000, 128, 128), (2, 1, 777, 64, 64),
                                         (1, 3, 300, 128, 128), (1, 1, 64, 64, 64),
                                         (2, 2, 700, 128, 128)])
def test_sparse_linear_small_shapes_in_full(B, H, N, d, bq):
    rng = np.random.default_rng(7 * N + d)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // bq), -(-N // 64)
    kept = _random_lists(rng, B, H, n_q, n_k)  # includes an empty and a full row
    idx, cnt = O.kept_to_index_list(kept)
    alpha = rng.uniform(0.05, 0.8, size=H).astype(np.float32)
    print(f"\n[linear] B={B} H={H} N={N} d={d} bq={bq}", flush=True)
    o = S.sparse_linear_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(cnt).cuda(), torch.from_numpy(alpha).cuda(),
                                 bq, 64)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref = O.sparse_linear_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                                 O.bf16_to_f64(V[b, h]), kept[b, h], bq, 64,
                                                 scale, float(alpha[h]))
            mx, mean = compare_outputs(got[b, h], ref)
            print(f"[linear] b={b} h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("N,d,sampled", [(4480, 64, False), (19217, 64, True), (38405, 128, True)])
def test_sparse_linear_long_rows_and_many_query_blocks(N, d, sampled):
    """Key-block counts that are not a multiple of 32 and span several stages of
    the dropped-block product (70, 301 and 601 blocks: the last bit word is
    partial), and 301 query blocks, so the product runs a second tile of
    query blocks holding 45 of them. Sampled query blocks include the first and
    last of each tile and the ragged last block."""
    rng = np.random.default_rng(N + 3 * d)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    H = 2 if N < 10000 else 1
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((1, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // d), -(-N // 64)
    kept = _random_lists(rng, 1, H, n_q, n_k)
    idx, cnt = O.kept_to_index_list(kept)
    alpha = rng.uniform(0.05, 0.8, size=H).astype(np.float32)
    print(f"\n[linear long] N={N} d={d} n_q={n_q} n_k={n_k}", flush=True)
    q = to_gpu(Q)
    o = S.sparse_linear_attn_fwd(q, to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(cnt).cuda(), torch.from_numpy(alpha).cuda(),
                                 d, 64, out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(o)
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    blocks = None
    if sampled:
        blocks = sorted({0, 1, 2, 255, 256, n_q - 1, *rng.choice(n_q, 3, replace=False)})
    for h in range(H):
        ref = O.sparse_linear_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                             O.bf16_to_f64(V[0, h]), kept[0, h], d, 64,
                                             S.default_scale(d), float(alpha[h]),
                                             q_blocks=blocks)
        rows = ~np.isnan(ref[:, 0])
        mx, mean = compare_outputs(got[0, h][rows], ref[rows])
        print(f"[linear long] h={h} blocks={blocks}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("B,H,N,d", [(1, 2, 1000, 128), (2, 1, 1500, 64)])
def test_sparse_linear_dense_lists_sum_the_dropped_blocks(B, H, N, d):
    """Rows listing more than half of the key blocks take the branch's other
    route (the dropped blocks summed directly); every row here does, except a
    full one (no linear part) and an empty one."""
    rng = np.random.default_rng(11 * N + d)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // d), -(-N // 64)
    kept = rng.random((B, H, n_q, n_k)) < 0.8
    flat = kept.reshape(-1, n_k)
    flat[0] = True
    flat[1] = False
    idx, cnt = O.kept_to_index_list(kept)
    alpha = rng.uniform(0.05, 0.8, size=H).astype(np.float32)
    o = S.sparse_linear_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(cnt).cuda(), torch.from_numpy(alpha).cuda(),
                                 d, 64)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref = O.sparse_linear_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                                 O.bf16_to_f64(V[b, h]), kept[b, h], d, 64,
                                                 scale, float(alpha[h]))
            mx, mean = compare_outputs(got[b, h], ref)
            print(f"[linear dense lists] b={b} h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


def test_sparse_linear_matches_oracle_on_workload():
    """The sparse-linear workload: wan1.3b inputs and mask, alpha = 0.1 per head."""
    wl, Q, K, V, q, k, v = workload_tensors("wan1.3b_linear")
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass)
    alpha = torch.full((wl.H,), wl.linear_alpha, dtype=torch.float32, device="cuda")
    o = S.sparse_linear_attn_fwd(q, k, v, idx, cnt, alpha, wl.block_q, wl.block_k,
                                 out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(o)
    kept = gpu_bits_to_bool(bits, wl.n_k)
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    rng = np.random.default_rng(99)
    for h in sample_heads("wan1.3b_linear", wl.H, rng):
        blocks = sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, 4, replace=False)})
        ref = O.sparse_linear_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                             O.bf16_to_f64(V[0, h]), kept[0, h], wl.block_q,
                                             wl.block_k, wl.scale, wl.linear_alpha,
                                             q_blocks=blocks)
        rows = ~np.isnan(ref[:, 0])
        mx, mean = compare_outputs(got[0, h][rows], ref[rows])
        print(f"[linear] wan1.3b_linear h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


def test_sparse_linear_branch_contributes():
    """The linear term is really added: with alpha = 0 the output equals sparse attention,
    and with alpha > 0 it differs exactly on rows that dropped blocks."""
    rng = np.random.default_rng(5)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    B, H, N, d = 1, 2, 512, 128
    Q, K, V = (to_gpu(f64_to_bf16_bits(rng.standard_normal((B, H, N, d)))) for _ in range(3))
    kept = np.zeros((B, H, 4, 8), bool)
    kept[..., :3] = True
    kept[:, :, 2, :] = True  # query block 2 keeps everything -> no linear term
    idx, cnt = (torch.from_numpy(x).cuda() for x in O.kept_to_index_list(kept))
    o_s = S.sparge_attn_fwd(Q, K, V, idx, cnt, 128, 64)
    zero = S.sparse_linear_attn_fwd(Q, K, V, idx, cnt, torch.zeros(H, device="cuda"), 128, 64)
    half = S.sparse_linear_attn_fwd(Q, K, V, idx, cnt, torch.full((H,), 0.5, device="cuda"),
                                    128, 64)
    torch.cuda.synchronize()
    assert torch.equal(zero.view(torch.int16), o_s.view(torch.int16))
    diff = (half.float() - o_s.float()).abs().amax(dim=-1)  # [B, H, N]
    assert (diff[..., 256:384] == 0).all()
    assert (diff[..., :256] > 0).all() and (diff[..., 384:] > 0).all()


# ------------------------------------------------------ SLA2 mix (section 2A)
@pytest.mark.parametrize("B,H,N,d", [(1, 2, 1000, 128), (2, 1, 777, 64), (1, 3, 300, 128),
                                     (1, 1, 64, 64), (2, 2, 700, 128)])
def test_sla2_mix_small_shapes_in_full(B, H, N, d):
    rng = np.random.default_rng(11 * N + d)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits, mix_alpha
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // d), -(-N // 64)
    kept = _random_lists(rng, B, H, n_q, n_k)  # includes an empty and a full row
    idx, cnt = O.kept_to_index_list(kept)
    alpha = mix_alpha(H, d, N)
    alpha[0, :3] = (0.0, 1.0, 0.5)  # the two extremes and an exact half
    print(f"\n[mix] B={B} H={H} N={N} d={d}", flush=True)
    o = S.sla2_mix_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                            torch.from_numpy(cnt).cuda(), torch.from_numpy(alpha).cuda(), d, 64)
    torch.cuda.synchronize()
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref = O.sla2_mix_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                            O.bf16_to_f64(V[b, h]), kept[b, h], d, 64, scale,
                                            alpha[h])
            mx, mean = compare_outputs(got[b, h], ref)
            print(f"[mix] b={b} h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


def test_sla2_mix_matches_oracle_on_workload():
    """wan1.3b inputs and mask with per-channel ratios drawn in [0, 1)."""
    from block_sparse_attention_softmax_amd.workloads import mix_alpha
    wl, Q, K, V, q, k, v = workload_tensors("wan1.3b_linear")
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass)
    alpha = mix_alpha(wl.H, wl.d, 5)
    o = S.sla2_mix_attn_fwd(q, k, v, idx, cnt, torch.from_numpy(alpha).cuda(), wl.block_q,
                            wl.block_k, out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(o)
    kept = gpu_bits_to_bool(bits, wl.n_k)
    got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
    rng = np.random.default_rng(98)
    for h in sample_heads("wan1.3b_linear", wl.H, rng):
        blocks = sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, 4, replace=False)})
        ref = O.sla2_mix_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                        O.bf16_to_f64(V[0, h]), kept[0, h], wl.block_q,
                                        wl.block_k, wl.scale, alpha[h], q_blocks=blocks)
        rows = ~np.isnan(ref[:, 0])
        mx, mean = compare_outputs(got[0, h][rows], ref[rows])
        print(f"[mix] wan1.3b h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


# ------------------------------------- SALAD post-tuning branch dropping
def _drop_case(seed, H=4, N=1000, d=128):
    rng = np.random.default_rng(seed)
    from block_sparse_attention_softmax_amd.workloads import f64_to_bf16_bits
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((1, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // d), -(-N // 64)
    kept = _random_lists(rng, 1, H, n_q, n_k)
    idx, cnt = O.kept_to_index_list(kept)
    g = (to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
         torch.from_numpy(cnt).cuda())
    return Q, K, V, kept, g


@pytest.mark.parametrize("d", [128, 64])
def test_branch_dropping_matches_oracle(d):
    H, N = 4, 1000
    Q, K, V, kept, g = _drop_case(21 + d, H, N, d)
    scale, tau = S.default_scale(d), 0.05
    f = lambda x, h: O.bf16_to_f64(x[0, h])
    # added form: heads 0, 1, 3 are dropped (|alpha| <= tau), head 2 is evaluated
    a_add = np.array([0.0, 0.03, 0.2, -0.04], np.float32)
    # mix: heads 0, 1 dropped (all 1 - alpha small), 2 and 3 evaluated (3: one channel)
    a_mix = np.ones((H, d), np.float32)
    a_mix[1] = 0.97
    a_mix[2] = np.random.default_rng(d).random(d)
    a_mix[3, 5] = 0.5
    ws = torch.empty(S.linear_workspace_bytes(1, H, N, d), dtype=torch.uint8, device="cuda")
    o_add = S.sparse_linear_attn_fwd(*g, torch.from_numpy(a_add).cuda(), d, 64,
                                     drop_below=tau, workspace=ws)
    o_mix = S.sla2_mix_attn_fwd(*g, torch.from_numpy(a_mix).cuda(), d, 64, drop_below=tau,
                                workspace=ws)
    o_s = S.sparge_attn_fwd(*g, d, 64)
    torch.cuda.synchronize()
    got_add = O.bf16_to_f64(o_add.cpu().view(torch.uint16).numpy())
    got_mix = O.bf16_to_f64(o_mix.cpu().view(torch.uint16).numpy())
    print(f"\n[drop] d={d}", flush=True)
    for h in range(H):
        ref = O.sparse_linear_attention_head_dropping(f(Q, h), f(K, h), f(V, h), kept[0, h], d,
                                                      64, scale, float(a_add[h]), tau)
        mx, mean = compare_outputs(got_add[0, h], ref)
        ref = O.sla2_mix_attention_head_dropping(f(Q, h), f(K, h), f(V, h), kept[0, h], d, 64,
                                                 scale, a_mix[h], tau)
        mx2, mean2 = compare_outputs(got_mix[0, h], ref)
        print(f"[drop] h={h}: add max {mx:.2e} mean {mean:.2e}; mix max {mx2:.2e} "
              f"mean {mean2:.2e}", flush=True)
    # a dropped head of the added form is plain block-sparse attention, bit for bit
    for h in (0, 1, 3):
        assert torch.equal(o_add[0, h].view(torch.int16), o_s[0, h].view(torch.int16))
    assert torch.equal(o_mix[0, 0].view(torch.int16), o_s[0, 0].view(torch.int16))
    # the evaluated heads differ from it on rows that dropped a block
    assert not torch.equal(o_add[0, 2], o_s[0, 2]) and not torch.equal(o_mix[0, 3], o_s[0, 3])


def test_dropping_an_exactly_zero_branch_changes_no_output():
    """drop_below = 0 skips only zero branches; evaluating them instead
    (drop_below < 0) gives the same bits."""
    H, N, d = 2, 777, 128
    Q, K, V, kept, g = _drop_case(31, H, N, d)
    zero = torch.zeros(H, device="cuda")
    ones = torch.ones(H, d, device="cuda")
    outs = [S.sparse_linear_attn_fwd(*g, zero, d, 64, drop_below=t) for t in (0.0, -1.0)]
    outs += [S.sla2_mix_attn_fwd(*g, ones, d, 64, drop_below=t) for t in (0.0, -1.0)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[2].view(torch.int16), outs[3].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_drop_decision_follows_alpha_between_calls():
    """The decision is taken on the device at every call: the same workspace
    serves a call that drops a head's branch and one that evaluates it."""
    H, N, d = 2, 1000, 64
    Q, K, V, kept, g = _drop_case(41, H, N, d)
    ws = torch.empty(S.linear_workspace_bytes(1, H, N, d), dtype=torch.uint8, device="cuda")
    f = lambda x, h: O.bf16_to_f64(x[0, h])
    for a in ([0.3, 0.0], [0.0, 0.3], [0.3, 0.0]):
        alpha = np.array(a, np.float32)
        o = S.sparse_linear_attn_fwd(*g, torch.from_numpy(alpha).cuda(), d, 64,
                                     drop_below=0.0, workspace=ws)
        torch.cuda.synchronize()
        got = O.bf16_to_f64(o.cpu().view(torch.uint16).numpy())
        for h in range(H):
            ref = O.sparse_linear_attention_head_dropping(f(Q, h), f(K, h), f(V, h), kept[0, h],
                                                          d, 64, S.default_scale(d),
                                                          float(alpha[h]), 0.0)
            compare_outputs(got[0, h], ref)


@pytest.mark.parametrize("name,k_frac,p_mass", [("wan1.3b", 0.05, 0.9), ("wan1.3b", 0.05, 0.0),
                                                ("tiny", 0.1, 0.9)])
def test_mask_in_two_halves_equals_one_call(name, k_frac, p_mass):
    """sparge_mask_pool then sparge_mask_select on one stream give exactly the
    outputs of sparge_mask_predict, scores included."""
    wl, Q, K, V, q, k, v = workload_tensors(name)
    one = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, k_frac, p_mass, wl.scale,
                                return_logits=True)
    ws = S.sparge_mask_pool(q, k, wl.block_q, wl.block_k)
    two = S.sparge_mask_select(q, ws, wl.block_q, wl.block_k, k_frac, p_mass, wl.scale,
                               return_logits=True)
    torch.cuda.synchronize()
    bits1, idx1, cnt1, lg1 = one
    bits2, idx2, cnt2, lg2 = two
    assert torch.equal(bits1, bits2) and torch.equal(cnt1, cnt2) and torch.equal(lg1, lg2)
    pos = torch.arange(idx1.shape[-1], device=idx1.device)
    valid = pos < cnt1.unsqueeze(-1)
    assert torch.equal(idx1[valid], idx2[valid])


def test_binding_rejects_mismatched_buffers():
    """Index lists, outputs and workspaces of the wrong shape, dtype or device are
    refused before the library sees their pointers."""
    dev = torch.device("cuda:0")
    q, k, v = (torch.zeros((1, 2, 300, 64), dtype=torch.bfloat16, device=dev) for _ in range(3))
    bits, idx, cnt = S.sparge_mask_predict(q, k, 64, 64, 0.5, 0.5)
    with pytest.raises(ValueError):
        S.sparge_attn_fwd(q, k, v, idx[..., :-1].contiguous(), cnt, 64, 64)
    with pytest.raises(ValueError):
        S.sparge_attn_fwd(q, k, v, idx, cnt.to(torch.int64), 64, 64)
    with pytest.raises(ValueError):
        S.sparge_attn_fwd(q, k, v, idx.cpu(), cnt, 64, 64)
    with pytest.raises(ValueError):
        S.sparge_attn_fwd(q, k, v, idx, cnt, 64, 64, out=torch.empty((1, 2, 300, 64), device=dev))
    with pytest.raises(ValueError):
        S.sparge_attn_fwd(q, k, v, idx, cnt, 64, 64, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        S.sparge_mask_predict(q, k, 64, 64, 0.5, 0.5, out=(bits, idx[:, :1].contiguous(), cnt))
    with pytest.raises(ValueError):
        S.sparge_attn_fwd_packed(q, k, idx, cnt, None, 64, 64)
    # a workspace of another dtype is measured in bytes
    ws = torch.empty(S.attn_workspace_bytes(1, 2, 300, 64) // 4 + 1, dtype=torch.float32, device=dev)
    o = S.sparge_attn_fwd(q, k, v, idx, cnt, 64, 64, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("k_frac,p_mass", [(0.05, 0.9), (0.05, 0.0)])
def test_step_graph_replays_match_eager(k_frac, p_mass):
    """One forward step (pool; V repack on a second stream; select; join;
    attention) captured in a HIP graph: every replay, with eager steps and
    synchronizations between the replays, gives exactly the eager step's
    mask and output, which equal the one-call entry points' results."""
    wl, Q, K, V, q, k, v = workload_tensors("wan1.3b")
    B, H, N, d = q.shape
    dev = q.device
    bits = torch.empty((B, H, wl.n_q, -(-wl.n_k // 32)), dtype=torch.int32, device=dev)
    idx = torch.empty((B, H, wl.n_q, wl.n_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, wl.n_q), dtype=torch.int32, device=dev)
    ws = torch.empty(S.mask_workspace_bytes(B, H, N, d, wl.block_q, wl.block_k),
                     dtype=torch.uint8, device=dev)
    aws = torch.empty(S.attn_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    side, pooled = torch.cuda.Stream(), torch.cuda.Event()

    def step():
        cur = torch.cuda.current_stream()
        S.sparge_mask_pool(q, k, wl.block_q, wl.block_k, workspace=ws)
        pooled.record(cur)
        side.wait_event(pooled)
        with torch.cuda.stream(side):
            S.sparge_attn_pack(v, workspace=aws)
        S.sparge_mask_select(q, ws, wl.block_q, wl.block_k, k_frac, p_mass, wl.scale,
                             out=(bits, idx, cnt))
        cur.wait_stream(side)
        S.sparge_attn_fwd_packed(q, k, idx, cnt, aws, wl.block_q, wl.block_k, wl.scale, out=o)

    step()
    torch.cuda.synchronize()
    ref = (bits.clone(), cnt.clone(), o.clone())
    bits1, idx1, cnt1 = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, k_frac, p_mass, wl.scale)
    o1 = S.sparge_attn_fwd(q, k, v, idx1, cnt1, wl.block_q, wl.block_k, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(bits1, ref[0]) and torch.equal(cnt1, ref[1]) and torch.equal(o1, ref[2])

    graph, cs = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cs):
        step()
    for _ in range(3):
        for t in (bits, cnt, o):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits, ref[0]) and torch.equal(cnt, ref[1]) and torch.equal(o, ref[2])
        step()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref[2])
    del graph


@pytest.mark.parametrize("name", ["tiny", "wan1.3b"])
def test_one_call_entry_points_replay_from_a_graph(name):
    """The one-call mask, the forward with lse, its backward, the low-bit
    forward and its split form captured together in a HIP graph (outputs allocated in the
    graph's pool): every replay, with eager calls and synchronizations in
    between, reproduces the eager results exactly (the kernels clear their
    own counters with fill kernels and add no floating-point atomics)."""
    wl, Q, K, V, q, k, v = workload_tensors(name)
    d_o = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).to(q.device,
                                                                              torch.bfloat16)

    def calls():
        bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, wl.k_frac,
                                               wl.p_mass, wl.scale)
        o, lse = S.sparge_attn_fwd_lse(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale)
        dq, dk, dv = S.sparge_attn_bwd(q, k, v, o, d_o, lse, idx, cnt, wl.block_q, wl.block_k,
                                       wl.scale)
        ol = S.sparge_attn_fwd_lowbit(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale)
        ws, lws = S.sparge_mask_pool_lowbit(q, k, wl.block_q, wl.block_k)
        S.sparge_attn_lowbit_pack(v, lws, wl.block_q)
        _, idx2, cnt2 = S.sparge_mask_select(q, ws, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass,
                                             wl.scale)
        ol2 = S.sparge_attn_fwd_lowbit_packed(q, idx2, cnt2, lws, wl.block_q, wl.block_k,
                                              wl.scale)
        return bits, cnt, o, lse, dq, dk, dv, ol, ol2

    ref = [t.clone() for t in calls()]
    torch.cuda.synchronize()
    graph, cs = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        calls()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cs):
        outs = calls()
    names = ("bits", "cnt", "o", "lse", "dq", "dk", "dv", "o_lowbit", "o_lowbit_parts")
    for _ in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(names, outs, ref):
            assert torch.equal(a, b), n
        calls()  # eager work between the replays
        torch.cuda.synchronize()
    del graph


_CAPTURE_SCRIPT = r"""
import sys, torch
sys.path.insert(0, {root!r})
from block_sparse_attention_softmax_amd import binding as S
g = torch.Generator().manual_seed(5)
small = torch.randn(1, 2, 4000, 64, generator=g).to("cuda", torch.bfloat16)
S.sparge_mask_predict(small, small, 128, 64, 0.1, 0.9)       # width 64: the register sort
torch.cuda.synchronize()
q, k = (torch.randn(1, 1, 100000, 64, generator=g).to("cuda", torch.bfloat16) for _ in range(2))
ref = S.sparge_mask_predict(q, k, 128, 64, 0.02, 0.9)        # 782 rows of 1563: the LDS sort
torch.cuda.synchronize()
ref = [t.clone() for t in ref]
out = [torch.empty_like(t) for t in ref]
graph, cs = torch.cuda.CUDAGraph(), torch.cuda.Stream()
with torch.cuda.graph(graph, stream=cs):
    S.sparge_mask_predict(q, k, 128, 64, 0.02, 0.9, out=tuple(out))
for _ in range(3):
    for t in out:
        t.zero_()
    graph.replay()
    torch.cuda.synchronize()
    valid = torch.arange(ref[1].shape[-1], device="cuda") < ref[2].unsqueeze(-1)
    assert torch.equal(out[0], ref[0]) and torch.equal(out[2], ref[2])
    assert torch.equal(out[1][valid], ref[1][valid])
print("capture ok")
"""


def test_lds_sort_mask_captured_after_a_narrow_call():
    """In a fresh process, a mask call whose rows use the register sort comes
    first; a mask call at a width that takes the LDS sort is then captured in a
    HIP graph and replayed: the one-time LDS-limit change was already made for
    every width, so nothing is set during the capture."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _CAPTURE_SCRIPT.format(root=root)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "capture ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
