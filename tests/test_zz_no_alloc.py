"""The mask entry point that allocates nothing (sparge_mask_predict_noalloc),
called through the C ABI, against sparge_mask_predict: two calls in a row,
the second on a smaller input, each bit-identical to the workspace call
(mask bits, counts, index lists and float64 block scores)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_softmax_amd import binding as S
from block_sparse_attention_softmax_amd.workloads import WORKLOADS, generate
from parity import sentinel_mask_outputs, to_gpu

pytestmark = pytest.mark.gpu


def _same(a, b):
    bits, idx, cnt, lg = a
    bits2, idx2, cnt2, lg2 = b
    assert torch.equal(bits, bits2) and torch.equal(cnt, cnt2)
    valid = torch.arange(idx.shape[-1], device=idx.device) < cnt.unsqueeze(-1)
    assert torch.equal(idx[valid], idx2[valid])
    assert torch.equal(lg.view(torch.int64), lg2.view(torch.int64))


def _call_both(q, k, bq, k_frac, p_mass):
    B, H, N, d = q.shape
    n_q, n_k = -(-N // bq), -(-N // 64)
    ref = S.sparge_mask_predict(q, k, bq, 64, k_frac, p_mass, return_logits=True,
                                out=sentinel_mask_outputs(B, H, n_q, n_k, q.device))
    got = S.sparge_mask_predict_noalloc(q, k, bq, 64, k_frac, p_mass, return_logits=True,
                                        out=sentinel_mask_outputs(B, H, n_q, n_k, q.device))
    # and with the scores kept in the scratch (no block_logits)
    got2 = S.sparge_mask_predict_noalloc(q, k, bq, 64, k_frac, p_mass,
                                         out=sentinel_mask_outputs(B, H, n_q, n_k, q.device)[:3])
    torch.cuda.synchronize()
    _same(ref, got)
    _same(ref[:3] + (ref[3],), got2 + (ref[3],))
    return ref


def test_noalloc_mask_equals_workspace_mask_twice_second_smaller():
    wl = WORKLOADS["wan1.3b"]
    Q, K, _ = generate(wl)
    q, k = to_gpu(Q), to_gpu(K)
    print("\n[noalloc] wan1.3b k=0.05 p=0.9", flush=True)
    big = _call_both(q, k, wl.block_q, wl.k_frac, wl.p_mass)
    # a smaller input next: the scratch keeps the first call's contents
    rng = np.random.default_rng(3)
    qs = torch.from_numpy(rng.standard_normal((1, 3, 5000, 64)).astype(np.float32)).to(
        "cuda", torch.bfloat16)
    ks = torch.from_numpy(rng.standard_normal((1, 3, 5000, 64)).astype(np.float32)).to(
        "cuda", torch.bfloat16)
    print("[noalloc] B=1 H=3 N=5000 d=64 bq=64 k=0.1 p=0.5", flush=True)
    small = _call_both(qs, ks, 64, 0.1, 0.5)
    assert big[0].shape != small[0].shape


def test_noalloc_rejects_shapes_beyond_its_scratch():
    cap = S.lib().sparge_mask_noalloc_scratch_bytes()
    assert cap == 64 << 20
    # Wan-14B-720p: 40 heads, 591 x 1182 blocks: the scores alone are 224 MB
    q = torch.zeros((1, 40, 75600, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S.SpargeError, match="scratch"):
        S.sparge_mask_predict_noalloc(q, q, 128, 64, 0.05, 0.9)
