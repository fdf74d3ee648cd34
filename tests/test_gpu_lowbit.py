"""GPU parity of the low-bit sparse branch (INT8 Q/K, e4m3 P/V) against the
float64 oracle that takes the same steps, on the same ordered lists."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_attention_softmax_amd import binding as S
from block_sparse_attention_softmax_amd.workloads import WORKLOADS, f64_to_bf16_bits, generate
from oracle import sparge_oracle as O
from parity import assert_all_written, compare_outputs, gpu_bits_to_bool, nan_like, to_gpu

pytestmark = pytest.mark.gpu


def _f(x, b, h):
    return O.bf16_to_f64(x[b, h])


def _np(t):
    return O.bf16_to_f64(t.cpu().view(torch.uint16).numpy())


@pytest.mark.parametrize("B,H,N,d,bq", [(1, 2, 1000, 128, 128), (2, 1, 777, 64, 64),
                                         (1, 3, 300, 128, 64), (1, 1, 50, 64, 128),
                                         (1, 2, 2048, 128, 128)])
def test_lowbit_small_shapes_in_full(B, H, N, d, bq):
    rng = np.random.default_rng(13 * N + d)
    Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    n_q, n_k = -(-N // bq), -(-N // 64)
    kept = rng.random((B, H, n_q, n_k)) < rng.uniform(0.2, 0.7)
    flat = kept.reshape(-1, n_k)
    flat[0] = False
    if flat.shape[0] > 1:
        flat[1] = True
    idx, cnt = O.kept_to_index_list(kept)
    # every other row visits its blocks in reverse order
    for r in np.ndindex(*cnt.shape):
        if (r[-1] % 2) == 1:
            idx[r][:cnt[r]] = idx[r][:cnt[r]][::-1]
    print(f"\n[lowbit] B={B} H={H} N={N} d={d} bq={bq}", flush=True)
    o = S.sparge_attn_fwd_lowbit(to_gpu(Q), to_gpu(K), to_gpu(V), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(cnt).cuda(), bq, 64)
    torch.cuda.synchronize()
    got = _np(o)
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref = O.lowbit_attention_head(_f(Q, b, h), _f(K, b, h), _f(V, b, h), idx[b, h],
                                          cnt[b, h], bq, 64, scale)
            mx, mean = compare_outputs(got[b, h], ref)
            print(f"[lowbit] b={b} h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("k_frac,p_mass", [(0.05, 0.0), (0.05, 0.9)])
def test_lowbit_on_workload_sampled(k_frac, p_mass):
    """wan1.3b with its mask: sampled query blocks of two heads against the
    oracle, and the distance to the bf16 kernel (the quantisation's own error)."""
    wl = WORKLOADS["wan1.3b"]
    Q, K, V = generate(wl)
    q, k, v = to_gpu(Q), to_gpu(K), to_gpu(V)
    bits, idx, cnt = S.sparge_mask_predict(q, k, wl.block_q, wl.block_k, k_frac, p_mass,
                                           wl.scale)
    o = S.sparge_attn_fwd_lowbit(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale,
                                 out=nan_like(q))
    o16 = S.sparge_attn_fwd(q, k, v, idx, cnt, wl.block_q, wl.block_k, wl.scale)
    torch.cuda.synchronize()
    assert_all_written(o)
    got, got16 = _np(o), _np(o16)
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    rng = np.random.default_rng(7)
    print(f"\n[lowbit workload] k={k_frac} p={p_mass}: |lowbit - bf16| max "
          f"{np.abs(got - got16).max():.2e} mean {np.abs(got - got16).mean():.2e}", flush=True)
    for h in rng.choice(wl.H, size=4, replace=False):
        blocks = sorted({0, wl.n_q - 1, *rng.choice(wl.n_q, 4, replace=False)})
        ref = O.lowbit_attention_head(_f(Q, 0, h), _f(K, 0, h), _f(V, 0, h), idx_np[0, h],
                                      cnt_np[0, h], wl.block_q, wl.block_k, wl.scale,
                                      q_blocks=blocks)
        rows = ~np.isnan(ref[:, 0])
        mx, mean = compare_outputs(got[0, h][rows], ref[rows])
        print(f"[lowbit workload] h={h}: max {mx:.2e} mean {mean:.2e}", flush=True)


@pytest.mark.parametrize("name,B,H,N,d,bq,k_frac,p_mass", [
    ("small", 1, 2, 1000, 128, 128, 0.2, 0.9), ("small", 2, 1, 777, 64, 64, 0.3, 0.5),
    ("small", 1, 3, 300, 128, 64, 0.5, 0.0), ("small", 1, 1, 50, 64, 128, 1.0, 0.9),
    ("wan1.3b", 1, 12, 32760, 128, 128, 0.05, 0.0), ("wan1.3b", 1, 12, 32760, 128, 128, 0.05, 0.9)])
def test_lowbit_in_parts_equals_one_call(name, B, H, N, d, bq, k_frac, p_mass):
    """The pooling pass that also writes the Q and K codes, the V pack and the
    attention from the workspace give exactly the one-call mask and low-bit
    output; the pooling's means (hence the mask) are unchanged by the codes."""
    if name == "wan1.3b":
        wl = WORKLOADS["wan1.3b"]
        Q, K, V = generate(wl)
    else:
        rng = np.random.default_rng(19 * N + d)
        Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d)) * 1.3) for _ in range(3))
    q, k, v = to_gpu(Q), to_gpu(K), to_gpu(V)
    print(f"\n[lowbit parts] {name} B={B} H={H} N={N} d={d} bq={bq} k={k_frac} p={p_mass}",
          flush=True)
    ref_mask = S.sparge_mask_predict(q, k, bq, 64, k_frac, p_mass, return_logits=True)
    ref = S.sparge_attn_fwd_lowbit(q, k, v, ref_mask[1], ref_mask[2], bq, 64, out=nan_like(q))
    ws, lws = S.sparge_mask_pool_lowbit(q, k, bq, 64)
    S.sparge_attn_lowbit_pack(v, lws, bq)
    bits, idx, cnt, lg = S.sparge_mask_select(q, ws, bq, 64, k_frac, p_mass, return_logits=True)
    o = S.sparge_attn_fwd_lowbit_packed(q, idx, cnt, lws, bq, 64, out=nan_like(q))
    o2 = S.sparge_attn_fwd_lowbit_packed(q, idx, cnt, lws, bq, 64, out=nan_like(q))  # again
    torch.cuda.synchronize()
    assert_all_written(ref, o)
    assert torch.equal(bits, ref_mask[0]) and torch.equal(cnt, ref_mask[2])
    assert torch.equal(lg.view(torch.int64), ref_mask[3].view(torch.int64))
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), ref.view(torch.int16))
