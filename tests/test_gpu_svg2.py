"""GPU parity of SVG2's clustered sparse attention against the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_attention_softmax_amd import binding as S
from block_sparse_attention_softmax_amd.workloads import WORKLOADS, f64_to_bf16_bits, generate
from oracle import sparge_oracle as O
from parity import assert_all_written, compare_outputs, nan_like, to_gpu

pytestmark = pytest.mark.gpu


def _np(t):
    return O.bf16_to_f64(t.cpu().view(torch.uint16).numpy())


@pytest.mark.parametrize("B,H,N,d,bq,Cq,Ck,p", [
    (1, 2, 1000, 128, 128, 8, 16, 0.9), (2, 1, 777, 64, 64, 5, 12, 0.8),
    (1, 1, 300, 128, 64, 3, 40, 0.5), (1, 2, 2048, 64, 128, 20, 30, 0.95),
    (1, 1, 500, 128, 128, 4, 7, 1.0)])
def test_svg2_small_shapes_in_full(B, H, N, d, bq, Cq, Ck, p):
    rng = np.random.default_rng(17 * N + Ck)
    # a few semantic groups along the sequence so the clusters mean something
    centres = rng.standard_normal((6, d))
    grp = rng.integers(0, 6, N)
    mk = lambda: f64_to_bf16_bits(centres[grp][None, None] + 0.5 * rng.standard_normal((B, H, N, d)))
    Q, K = mk(), mk()
    V = f64_to_bf16_bits(rng.standard_normal((B, H, N, d)))
    print(f"\n[svg2] B={B} H={H} N={N} d={d} bq={bq} Cq={Cq} Ck={Ck} p={p}", flush=True)
    q = to_gpu(Q)
    ws = torch.empty(S.svg2_workspace_bytes(B, H, N, d, bq, Cq, Ck), dtype=torch.uint8,
                     device="cuda")
    o = S.svg2_attn_fwd(q, to_gpu(K), to_gpu(V), Cq, Ck, iters=4, p_mass=p, block_q=bq,
                        out=nan_like(q), workspace=ws)
    counts = S.svg2_attn_pair_counts(q, Cq, Ck, ws, bq).cpu().numpy()
    torch.cuda.synchronize()
    assert_all_written(o)
    got = _np(o)
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref, qa, ka, sel = O.svg2_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                                     O.bf16_to_f64(V[b, h]), Cq, Ck, 4, scale, p)
            mx, mean = compare_outputs(got[b, h], ref)
            useful = _useful_pairs(qa, ka, sel, Cq, Ck)
            assert counts[b, h, 0] == useful and counts[b, h, 1] >= useful
            print(f"[svg2] b={b} h={h}: kept pairs {sel.kept.mean():.3f} max {mx:.2e} "
                  f"mean {mean:.2e} useful/computed {useful / counts[b, h, 1]:.3f}", flush=True)


def _useful_pairs(qa, ka, sel, Cq, Ck):
    """Query-key token pairs of the oracle's selection: every query with every
    token of its cluster's kept key clusters."""
    qs, ks = np.bincount(qa, minlength=Cq), np.bincount(ka, minlength=Ck)
    return int((qs[:, None] * ks[None, :] * sel.kept).sum())


def test_svg2_on_workload_sampled():
    """wan1.3b-shaped inputs with 256 query and 512 key clusters (about one
    block's worth of tokens each), 3 rounds, p = 0.9: sampled rows of two heads."""
    wl = WORKLOADS["wan1.3b"]
    Q, K, V = generate(wl)
    q = to_gpu(Q)
    ws = torch.empty(S.svg2_workspace_bytes(wl.B, wl.H, wl.N, wl.d, 128, 256, 512),
                     dtype=torch.uint8, device="cuda")
    o = S.svg2_attn_fwd(q, to_gpu(K), to_gpu(V), 256, 512, iters=3, p_mass=0.9, out=nan_like(q),
                        workspace=ws)
    counts = S.svg2_attn_pair_counts(q, 256, 512, ws).cpu().numpy()
    torch.cuda.synchronize()
    assert_all_written(o)
    got = _np(o)
    rng = np.random.default_rng(23)
    for h in rng.choice(wl.H, size=3, replace=False):
        rows = np.sort(rng.choice(wl.N, 300, replace=False))
        ref, qa, ka, sel = O.svg2_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                                 O.bf16_to_f64(V[0, h]), 256, 512, 3, wl.scale,
                                                 0.9, q_rows=rows)
        mx, mean = compare_outputs(got[0, h][rows], ref)
        sizes = np.bincount(ka, minlength=512)
        density = (sel.kept[qa] * sizes[None]).sum() / (wl.N * wl.N)
        useful = _useful_pairs(qa, ka, sel, 256, 512)
        assert counts[0, h, 0] == useful and counts[0, h, 1] >= useful
        print(f"\n[svg2 workload] h={h}: token density {density:.3f} max {mx:.2e} "
              f"mean {mean:.2e} useful/computed {useful / counts[0, h, 1]:.3f}", flush=True)


@pytest.mark.parametrize("name,B,H,N,d,bq,Cq,Ck", [("small", 1, 2, 1000, 128, 128, 8, 16),
                                                  ("small", 2, 1, 777, 64, 64, 5, 12),
                                                  ("wan1.3b", 1, 12, 32760, 128, 128, 256, 512)])
def test_svg2_in_two_parts_equals_one_call(name, B, H, N, d, bq, Cq, Ck):
    """svg2_attn_cluster then svg2_attn_apply (twice) give exactly svg2_attn_fwd."""
    if name == "wan1.3b":
        Q, K, V = generate(WORKLOADS["wan1.3b"])
    else:
        rng = np.random.default_rng(N + Ck)
        Q, K, V = (f64_to_bf16_bits(rng.standard_normal((B, H, N, d))) for _ in range(3))
    q, k, v = to_gpu(Q), to_gpu(K), to_gpu(V)
    print(f"\n[svg2 parts] {name} B={B} H={H} N={N} d={d} bq={bq} Cq={Cq} Ck={Ck}", flush=True)
    one = S.svg2_attn_fwd(q, k, v, Cq, Ck, iters=3, p_mass=0.9, block_q=bq, out=nan_like(q))
    ws = S.svg2_attn_cluster(q, k, v, Cq, Ck, iters=3, p_mass=0.9, block_q=bq)
    a = S.svg2_attn_apply(q, Cq, Ck, ws, bq, out=nan_like(q))
    b = S.svg2_attn_apply(q, Cq, Ck, ws, bq, out=nan_like(q))
    torch.cuda.synchronize()
    assert_all_written(one)
    assert torch.equal(a.view(torch.int16), one.view(torch.int16))
    assert torch.equal(b.view(torch.int16), one.view(torch.int16))


@pytest.mark.parametrize("kind,N,d,Cq,Ck", [("ties", 600, 128, 8, 12), ("ties", 520, 64, 6, 10),
                                             ("close", 3000, 128, 16, 24)])
def test_svg2_assignment_close_calls(kind, N, d, Cq, Ck):
    """Tokens the bf16 filter of the assignment cannot decide: exact ties (rows
    drawn from five distinct vectors, so equal centroids recur and their tokens
    go to the lower cluster) and near ties (rows within 1e-3 of a few vectors,
    most of them listed for the float64 pass, many 16-token chunks per head).
    The clustering must still equal the oracle's: same useful pairs, same output."""
    B, H = 1, 2
    rng = np.random.default_rng(N + 7 * Ck)
    base = rng.standard_normal((5, d))
    def rows():
        pick = base[rng.integers(0, 5, (B, H, N))]
        if kind == "close":
            pick = pick + 1e-3 * rng.standard_normal((B, H, N, d))
        return f64_to_bf16_bits(pick)
    Q, K = rows(), rows()
    V = f64_to_bf16_bits(rng.standard_normal((B, H, N, d)))
    print(f"\n[svg2 close calls] {kind} N={N} d={d} Cq={Cq} Ck={Ck}", flush=True)
    q = to_gpu(Q)
    ws = torch.empty(S.svg2_workspace_bytes(B, H, N, d, 128, Cq, Ck), dtype=torch.uint8,
                     device="cuda")
    o = S.svg2_attn_fwd(q, to_gpu(K), to_gpu(V), Cq, Ck, iters=3, p_mass=0.9, out=nan_like(q),
                        workspace=ws)
    counts = S.svg2_attn_pair_counts(q, Cq, Ck, ws).cpu().numpy()
    torch.cuda.synchronize()
    assert_all_written(o)
    got = _np(o)
    scale = S.default_scale(d)
    for h in range(H):
        ref, qa, ka, sel = O.svg2_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                                 O.bf16_to_f64(V[0, h]), Cq, Ck, 3, scale, 0.9)
        mx, mean = compare_outputs(got[0, h], ref)
        assert counts[0, h, 0] == _useful_pairs(qa, ka, sel, Cq, Ck)
        print(f"[svg2 close calls] h={h}: clusters used q {len(np.unique(qa))} k "
              f"{len(np.unique(ka))}, max {mx:.2e} mean {mean:.2e}", flush=True)
