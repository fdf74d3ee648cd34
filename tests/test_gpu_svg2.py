"""GPU parity of SVG2's clustered sparse attention against the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_attention_softmax_amd import binding as S
from block_sparse_attention_softmax_amd.workloads import WORKLOADS, f64_to_bf16_bits, generate
from oracle import sparge_oracle as O
from parity import compare_outputs, to_gpu

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
    o = S.svg2_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), Cq, Ck, iters=4, p_mass=p, block_q=bq)
    torch.cuda.synchronize()
    got = _np(o)
    scale = S.default_scale(d)
    for b in range(B):
        for h in range(H):
            ref, qa, ka, sel = O.svg2_attention_head(O.bf16_to_f64(Q[b, h]), O.bf16_to_f64(K[b, h]),
                                                     O.bf16_to_f64(V[b, h]), Cq, Ck, 4, scale, p)
            mx, mean = compare_outputs(got[b, h], ref)
            print(f"[svg2] b={b} h={h}: kept pairs {sel.kept.mean():.3f} max {mx:.2e} "
                  f"mean {mean:.2e}", flush=True)


def test_svg2_on_workload_sampled():
    """wan1.3b-shaped inputs with 256 query and 512 key clusters (about one
    block's worth of tokens each), 3 rounds, p = 0.9: sampled rows of two heads."""
    wl = WORKLOADS["wan1.3b"]
    Q, K, V = generate(wl)
    o = S.svg2_attn_fwd(to_gpu(Q), to_gpu(K), to_gpu(V), 256, 512, iters=3, p_mass=0.9)
    torch.cuda.synchronize()
    got = _np(o)
    rng = np.random.default_rng(23)
    for h in rng.choice(wl.H, size=2, replace=False):
        rows = np.sort(rng.choice(wl.N, 300, replace=False))
        ref, qa, ka, sel = O.svg2_attention_head(O.bf16_to_f64(Q[0, h]), O.bf16_to_f64(K[0, h]),
                                                 O.bf16_to_f64(V[0, h]), 256, 512, 3, wl.scale,
                                                 0.9, q_rows=rows)
        mx, mean = compare_outputs(got[0, h][rows], ref)
        sizes = np.bincount(ka, minlength=512)
        density = (sel.kept[qa] * sizes[None]).sum() / (wl.N * wl.N)
        print(f"\n[svg2 workload] h={h}: token density {density:.3f} max {mx:.2e} "
              f"mean {mean:.2e}", flush=True)
