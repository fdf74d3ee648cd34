"""GPU parity of the forward's log-sum-exp and of the backward (dQ, dK, dV)
against the float64 oracle, through the C ABI.

The parity tests hand the GPU backward an O (rounded to bf16) and a
log-sum-exp (float32) that the oracle computed, and the oracle takes D =
dO.O from the same O, so they measure the backward kernels alone. The chain
tests run the GPU forward and then the backward, against the exact gradient.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_attention_softmax_amd import binding as S
from block_sparse_attention_softmax_amd.workloads import WORKLOADS, f64_to_bf16_bits, generate
from oracle import sparge_oracle as O
from parity import (assert_all_written, nan_like, DQ_CHAIN_MAX_REL, DQ_CHAIN_MEAN_REL, compare_grads, gpu_bits_to_bool,
                    to_gpu)

pytestmark = pytest.mark.gpu

# N = 1050 and N = 64 with 128-row blocks: an odd number of 64-row groups, so
# the last query block runs past the rows that 64-row padding would cover
SHAPES = [(1, 2, 1000, 128, 128), (2, 1, 777, 64, 64), (1, 3, 300, 128, 64),
          (1, 1, 64, 64, 128), (1, 2, 2048, 128, 128), (1, 1, 1500, 64, 128),
          (1, 2, 1050, 128, 128)]
NAMES = ("dq", "dk", "dv")


def _case(B, H, N, d, bq, seed):
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(4))
    n_q, n_k = -(-N // bq), -(-N // 64)
    kept = rng.random((B, H, n_q, n_k)) < rng.uniform(0.1, 0.6)
    flat = kept.reshape(-1, n_k)
    flat[0] = False                  # an empty row: O = 0, no gradient
    if flat.shape[0] > 1:
        flat[1] = True               # a dense row
    if flat.shape[0] > 2:
        flat[2] = False
        flat[2, n_k - 1] = True      # only the short last key block
    idx, cnt = O.kept_to_index_list(kept)
    return Q, K, V, dO, kept, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()


def _f(x, b, h):
    return O.bf16_to_f64(x[b, h])


def _np(t):
    return O.bf16_to_f64(t.cpu().view(torch.uint16).numpy())


def _oracle_forward(Q, K, V, kept, bq, scale, heads=None):
    """O (bf16 bits) and lse (float32) from the oracle; heads outside `heads` zero."""
    B, H, N, d = Q.shape
    o = np.zeros((B, H, N, d), np.uint16)
    lse = np.zeros((B, H, N), np.float32)
    for b, h in (np.ndindex(B, H) if heads is None else heads):
        o[b, h] = f64_to_bf16_bits(O.masked_attention_head(_f(Q, b, h), _f(K, b, h), _f(V, b, h),
                                                           kept[b, h], bq, 64, scale))
        lse[b, h] = O.masked_attention_lse_head(_f(Q, b, h), _f(K, b, h), kept[b, h], bq, 64,
                                                scale).astype(np.float32)
    return o, lse


def _report(tag, rel):
    print(f"[{tag}] " + ", ".join(f"{n} max {m:.1e} mean {a:.1e}" for n, (m, a) in
                                  zip(NAMES, rel)), flush=True)


@pytest.mark.parametrize("B,H,N,d,bq", SHAPES)
def test_forward_lse_matches_oracle(B, H, N, d, bq):
    Q, K, V, dO, kept, idx, cnt = _case(B, H, N, d, bq, 3 * N + d)
    q, k, v = to_gpu(Q), to_gpu(K), to_gpu(V)
    o, lse = S.sparge_attn_fwd_lse(q, k, v, idx, cnt, bq, 64)
    o_plain = S.sparge_attn_fwd(q, k, v, idx, cnt, bq, 64)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16))
    got = lse.cpu().numpy().astype(np.float64)
    scale = S.default_scale(d)
    print(f"\n[lse] B={B} H={H} N={N} d={d} bq={bq}", flush=True)
    for b in range(B):
        for h in range(H):
            ref = O.masked_attention_lse_head(_f(Q, b, h), _f(K, b, h), kept[b, h], bq, 64, scale)
            empty = np.isneginf(ref)
            assert np.array_equal(np.isneginf(got[b, h]), empty)
            err = np.abs(got[b, h][~empty] - ref[~empty])
            if err.size:
                # the kernel's sum runs over bf16-rounded weights: within 2^-9 relative
                assert err.max() <= 2.5e-3, err.max()
                print(f"[lse] b={b} h={h}: max {err.max():.2e}", flush=True)


@pytest.mark.parametrize("B,H,N,d,bq", SHAPES)
def test_backward_small_shapes_in_full(B, H, N, d, bq):
    Q, K, V, dO, kept, idx, cnt = _case(B, H, N, d, bq, 5 * N + d)
    scale = S.default_scale(d)
    o_bits, lse = _oracle_forward(Q, K, V, kept, bq, scale)
    print(f"\n[bwd] B={B} H={H} N={N} d={d} bq={bq}", flush=True)
    dq, dk, dv = S.sparge_attn_bwd(to_gpu(Q), to_gpu(K), to_gpu(V), to_gpu(o_bits), to_gpu(dO),
                                   torch.from_numpy(lse).cuda(), idx, cnt, bq, 64)
    torch.cuda.synchronize()
    got = [_np(t) for t in (dq, dk, dv)]
    for b in range(B):
        for h in range(H):
            ref = O.masked_attention_backward_head(_f(Q, b, h), _f(K, b, h), _f(V, b, h),
                                                   kept[b, h], bq, 64, scale, _f(dO, b, h),
                                                   o=_f(o_bits, b, h))
            _report(f"bwd b={b} h={h}", [compare_grads(g[b, h], r, n)
                                         for g, r, n in zip(got, ref, NAMES)])
    # keys no row lists get exactly zero gradients
    listed = kept.any(axis=2)                                   # [B, H, n_k]
    for b in range(B):
        for h in range(H):
            for j in np.nonzero(~listed[b, h])[0]:
                assert not got[1][b, h, 64 * j:64 * j + 64].any()
                assert not got[2][b, h, 64 * j:64 * j + 64].any()


@pytest.mark.parametrize("B,H,N,d,bq", SHAPES[:3])
def test_forward_then_backward_small_shapes(B, H, N, d, bq):
    """The GPU forward's O and lse feed the GPU backward; the exact gradient."""
    Q, K, V, dO, kept, idx, cnt = _case(B, H, N, d, bq, 7 * N + d)
    q, k, v, do = to_gpu(Q), to_gpu(K), to_gpu(V), to_gpu(dO)
    o, lse = S.sparge_attn_fwd_lse(q, k, v, idx, cnt, bq, 64)
    dq, dk, dv = S.sparge_attn_bwd(q, k, v, o, do, lse, idx, cnt, bq, 64)
    torch.cuda.synchronize()
    got = [_np(t) for t in (dq, dk, dv)]
    scale = S.default_scale(d)
    print(f"\n[chain] B={B} H={H} N={N} d={d} bq={bq}", flush=True)
    for b in range(B):
        for h in range(H):
            ref = O.masked_attention_backward_head(_f(Q, b, h), _f(K, b, h), _f(V, b, h),
                                                   kept[b, h], bq, 64, scale, _f(dO, b, h))
            _report(f"chain b={b} h={h}", [compare_grads(g[b, h], r, n)
                                           for g, r, n in zip(got, ref, NAMES)])


def test_backward_is_deterministic_and_ignores_list_order():
    B, H, N, d, bq = 1, 2, 1000, 128, 128
    Q, K, V, dO, kept, idx, cnt = _case(B, H, N, d, bq, 77)
    q, k, v, do = to_gpu(Q), to_gpu(K), to_gpu(V), to_gpu(dO)
    o, lse = S.sparge_attn_fwd_lse(q, k, v, idx, cnt, bq, 64)
    first = S.sparge_attn_bwd(q, k, v, o, do, lse, idx, cnt, bq, 64)
    again = S.sparge_attn_bwd(q, k, v, o, do, lse, idx, cnt, bq, 64)
    # the same lists in reverse order
    idx_np, cnt_np = idx.cpu().numpy().copy(), cnt.cpu().numpy()
    for r in np.ndindex(*cnt_np.shape):
        idx_np[r][:cnt_np[r]] = idx_np[r][:cnt_np[r]][::-1]
    rev = S.sparge_attn_bwd(q, k, v, o, do, lse, torch.from_numpy(idx_np).cuda(), cnt, bq, 64)
    torch.cuda.synchronize()
    for a, b2 in zip(first, again):
        assert torch.equal(a.view(torch.int16), b2.view(torch.int16))
    # dK and dV walk the transposed lists, which come out sorted either way
    assert torch.equal(first[1].view(torch.int16), rev[1].view(torch.int16))
    assert torch.equal(first[2].view(torch.int16), rev[2].view(torch.int16))
    # dQ sums the key blocks in list order: equal up to float32 rounding
    scale = S.default_scale(d)
    for h in range(H):
        ref = O.masked_attention_backward_head(_f(Q, 0, h), _f(K, 0, h), _f(V, 0, h), kept[0, h],
                                               bq, 64, scale, _f(dO, 0, h))
        compare_grads(_np(rev[0])[0, h], ref[0], "dq (reversed lists)")


def _workload(k_frac):
    wl = WORKLOADS["wan1.3b"]
    Q, K, V = generate(wl)
    rng = np.random.default_rng(17)
    dO = f64_to_bf16_bits(rng.standard_normal(Q.shape))
    q, k, v, do = to_gpu(Q), to_gpu(K), to_gpu(V), to_gpu(dO)
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, k_frac, 0.0, wl.scale)
    torch.cuda.synchronize()
    kept = gpu_bits_to_bool(bits, wl.n_k)
    return wl, rng, Q, K, V, dO, q, k, v, do, idx, cnt, kept


def _samples(wl, rng):
    heads = rng.choice(wl.H, size=2, replace=False)
    return [(h, sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, 3, replace=False)}),
             sorted({wl.n_k - 1, *rng.choice(wl.n_k, 3, replace=False)})) for h in heads]


@pytest.mark.parametrize("k_frac", [0.05, 0.10])
def test_backward_on_workload_sampled(k_frac):
    """wan1.3b at the 95% / 90% operating points (p = 0), O and lse from the
    oracle for the sampled heads: dQ of sampled query blocks and dK, dV of
    sampled key blocks."""
    wl, rng, Q, K, V, dO, q, k, v, do, idx, cnt, kept = _workload(k_frac)
    samples = _samples(wl, rng)
    o_bits, lse = _oracle_forward(Q, K, V, kept, wl.block_q, wl.scale,
                                  heads=[(0, h) for h, _, _ in samples])
    dq, dk, dv = S.sparge_attn_bwd(q, k, v, to_gpu(o_bits), do, torch.from_numpy(lse).cuda(),
                                   idx, cnt, wl.block_q, wl.block_k, wl.scale)
    torch.cuda.synchronize()
    got = [_np(t) for t in (dq, dk, dv)]
    print(f"\n[bwd workload] k={k_frac} sparsity {1 - kept.mean():.4f}", flush=True)
    for h, qb, kb in samples:
        ref = O.masked_attention_backward_sampled(_f(Q, 0, h), _f(K, 0, h), _f(V, 0, h),
                                                  kept[0, h], wl.block_q, wl.block_k, wl.scale,
                                                  _f(dO, 0, h), qb, kb, o=_f(o_bits, 0, h))
        rel = []
        for g, r, n in zip(got, ref, NAMES):
            rows = ~np.isnan(r[:, 0])
            rel.append(compare_grads(g[0, h][rows], r[rows], n))
        _report(f"bwd workload h={h}", rel)


def test_forward_then_backward_on_workload_sampled():
    """The GPU forward then the backward at the 95% point, against the exact
    gradient; dQ within its conditioning bound (see parity.py)."""
    wl, rng, Q, K, V, dO, q, k, v, do, idx, cnt, kept = _workload(0.05)
    lse0 = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, lse = S.sparge_attn_fwd_lse(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale,
                                   out=(nan_like(q), lse0))
    dq, dk, dv = S.sparge_attn_bwd(q, k, v, o, do, lse, idx, cnt, wl.block_q, wl.block_k,
                                   wl.scale, out=tuple(nan_like(q) for _ in range(3)))
    torch.cuda.synchronize()
    assert_all_written(o, lse, dq, dk, dv)   # every head, row and key
    got = [_np(t) for t in (dq, dk, dv)]
    for h, qb, kb in _samples(wl, rng):
        ref = O.masked_attention_backward_sampled(_f(Q, 0, h), _f(K, 0, h), _f(V, 0, h),
                                                  kept[0, h], wl.block_q, wl.block_k, wl.scale,
                                                  _f(dO, 0, h), qb, kb)
        rel = []
        for g, r, n in zip(got, ref, NAMES):
            rows = ~np.isnan(r[:, 0])
            lim = (DQ_CHAIN_MAX_REL, DQ_CHAIN_MEAN_REL) if n == "dq" else ()
            rel.append(compare_grads(g[0, h][rows], r[rows], n, *lim))
        _report(f"chain workload h={h}", rel)


# ------------------------------------------------------ linear branch backward
# (1, 2, 4480, 128): 35 query blocks and 70 key blocks, so the per-key-block sums of
# dH_D, dz_D run two 32-block stages over the query blocks (the second partial)
LIN_SHAPES = [(1, 3, 1000, 128), (2, 1, 777, 64), (1, 2, 300, 128), (1, 2, 2048, 128),
              (1, 2, 4480, 128), (2, 2, 700, 128)]


def _lin_alpha(mode, H, d, seed):
    rng = np.random.default_rng(seed)
    if mode == "add":
        a = rng.uniform(0.05, 0.8, H).astype(np.float32)
        a[-1] = 0.0  # a dropped branch (drop_below = 0)
    else:
        a = rng.random((H, d)).astype(np.float32)
        a[-1] = 1.0  # a dropped branch: the mix without its linear term
    return a


def _oracle_linear_forward(Q, K, V, kept, d, scale, alpha, mode, heads=None):
    B, H, N, _ = Q.shape
    o = np.zeros((B, H, N, d), np.uint16)
    lse = np.zeros((B, H, N), np.float32)
    for b, h in (np.ndindex(B, H) if heads is None else heads):
        f = [_f(x, b, h) for x in (Q, K, V)]
        if mode == "add":
            out = O.sparse_linear_attention_head(*f, kept[b, h], d, 64, scale, float(alpha[h]))
        else:
            out = O.sla2_mix_attention_head(*f, kept[b, h], d, 64, scale, alpha[h])
        o[b, h] = f64_to_bf16_bits(out)
        lse[b, h] = O.masked_attention_lse_head(f[0], f[1], kept[b, h], d, 64, scale)
    return o, lse


@pytest.mark.parametrize("mode", ["add", "mix"])
@pytest.mark.parametrize("B,H,N,d", LIN_SHAPES)
def test_linear_backward_small_shapes_in_full(B, H, N, d, mode):
    Q, K, V, dO, kept, idx, cnt = _case(B, H, N, d, d, 11 * N + d)
    scale = S.default_scale(d)
    alpha = _lin_alpha(mode, H, d, N)
    o_bits, lse = _oracle_linear_forward(Q, K, V, kept, d, scale, alpha, mode)
    fn = S.sparse_linear_attn_bwd if mode == "add" else S.sla2_mix_attn_bwd
    print(f"\n[lin bwd {mode}] B={B} H={H} N={N} d={d}", flush=True)
    grads = fn(to_gpu(Q), to_gpu(K), to_gpu(V), to_gpu(o_bits), to_gpu(dO),
               torch.from_numpy(lse).cuda(), idx, cnt, torch.from_numpy(alpha).cuda(), d, 64)
    torch.cuda.synchronize()
    got = [_np(t) for t in grads]
    for b in range(B):
        for h in range(H):
            f = [_f(x, b, h) for x in (Q, K, V)]
            if mode == "add":
                ref = O.sparse_linear_attention_backward_head(*f, kept[b, h], d, 64, scale,
                                                              float(alpha[h]), _f(dO, b, h),
                                                              o=_f(o_bits, b, h))
            else:
                ref = O.sla2_mix_attention_backward_head(*f, kept[b, h], d, 64, scale, alpha[h],
                                                         _f(dO, b, h), o=_f(o_bits, b, h))
            _report(f"lin bwd {mode} b={b} h={h}", [compare_grads(g[b, h], r, n)
                                                    for g, r, n in zip(got, ref, NAMES)])


@pytest.mark.parametrize("mode", ["add", "mix"])
def test_linear_forward_then_backward(mode):
    """The GPU linear forward's O and lse feed the GPU backward; the exact gradient."""
    B, H, N, d = 1, 3, 1000, 128
    Q, K, V, dO, kept, idx, cnt = _case(B, H, N, d, d, 1234)
    alpha = _lin_alpha(mode, H, d, 5)
    q, k, v, do = to_gpu(Q), to_gpu(K), to_gpu(V), to_gpu(dO)
    a = torch.from_numpy(alpha).cuda()
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fwd = S.sparse_linear_attn_fwd if mode == "add" else S.sla2_mix_attn_fwd
    bwd = S.sparse_linear_attn_bwd if mode == "add" else S.sla2_mix_attn_bwd
    o = fwd(q, k, v, idx, cnt, a, d, 64, lse=lse)
    o_plain = fwd(q, k, v, idx, cnt, a, d, 64)
    grads = bwd(q, k, v, o, do, lse, idx, cnt, a, d, 64)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16))
    got = [_np(t) for t in grads]
    scale = S.default_scale(d)
    print(f"\n[lin chain {mode}]", flush=True)
    for h in range(H):
        lse_ref = O.masked_attention_lse_head(_f(Q, 0, h), _f(K, 0, h), kept[0, h], d, 64, scale)
        live = ~np.isneginf(lse_ref)
        assert np.abs(lse.cpu().numpy()[0, h][live] - lse_ref[live]).max() <= 2.5e-3
        f = [_f(x, 0, h) for x in (Q, K, V)]
        if mode == "add":
            ref = O.sparse_linear_attention_backward_head(*f, kept[0, h], d, 64, scale,
                                                          float(alpha[h]), _f(dO, 0, h))
        else:
            ref = O.sla2_mix_attention_backward_head(*f, kept[0, h], d, 64, scale, alpha[h],
                                                     _f(dO, 0, h))
        _report(f"lin chain {mode} h={h}", [compare_grads(g[0, h], r, n)
                                            for g, r, n in zip(got, ref, NAMES)])


def test_linear_backward_on_workload_sampled():
    """wan1.3b at the 95% point (p = 0, k = 5%), alpha = 0.1: O and lse from the
    oracle for one head; dQ of sampled query blocks, dK, dV of sampled key blocks."""
    wl, rng, Q, K, V, dO, q, k, v, do, idx, cnt, kept = _workload(0.05)
    h = int(rng.integers(wl.H))
    alpha = np.full(wl.H, 0.1, np.float32)
    o_bits, lse = _oracle_linear_forward(Q, K, V, kept, wl.d, wl.scale, alpha, "add",
                                         heads=[(0, h)])
    grads = S.sparse_linear_attn_bwd(q, k, v, to_gpu(o_bits), do, torch.from_numpy(lse).cuda(),
                                     idx, cnt, torch.from_numpy(alpha).cuda(), wl.block_q,
                                     wl.block_k, wl.scale)
    torch.cuda.synchronize()
    got = [_np(t) for t in grads]
    qb = sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, 2, replace=False)})
    kb = sorted({wl.n_k - 1, *rng.choice(wl.n_k, 2, replace=False)})
    f = [_f(x, 0, h) for x in (Q, K, V)]
    o_s = _f(o_bits, 0, h) - 0.1 * O.linear_branch_head(*f, kept[0, h], wl.block_q, wl.block_k)
    gs = O.masked_attention_backward_sampled(*f, kept[0, h], wl.block_q, wl.block_k, wl.scale,
                                             _f(dO, 0, h), qb, kb, o=o_s)
    gl = O.linear_branch_backward_sampled(*f, kept[0, h], wl.block_q, wl.block_k,
                                          float(np.float32(0.1)) * _f(dO, 0, h), qb, kb)
    rel = []
    for g, a, b2, n in zip(got, gs, gl, NAMES):
        rows = ~np.isnan(a[:, 0])
        rel.append(compare_grads(g[0, h][rows], a[rows] + b2[rows], n))
    _report(f"lin bwd workload h={h}", rel)
