"""Comparison helpers shared by the GPU parity tests (not a test module).

Masks: every row must match the oracle bit for bit (bitmask, count, index
list), near-tie rows included, since both sides take the decision in float64.
Where a caller relaxes that (exact=False), rows whose oracle margin is under
1e-5 may differ, and such a GPU row is accepted if it is admissible: (i) it keeps at least K_k
blocks, (ii) its oracle probability mass is at least p - 1e-5 (or it keeps
all blocks when p >= 1), (iii) no kept block scores more than 1e-5 below a
dropped block, and (iv) it is minimal: without its lowest-scoring block it
would hold fewer than K_k blocks or less than p + 1e-5 mass.

Outputs: max |O_gpu - O_oracle| <= 2e-2 and mean <= 2e-3 over valid rows.

Coverage: outputs are pre-filled with a sentinel (bf16 NaN for tensors, a
bit pattern for masks and counts, -1 for index lists) before the call, so a
tile the kernels never write cannot pass with an earlier call's bytes that
the caching allocator handed back.

Gradients (dQ, dK, dV have no natural unit scale): relative to the oracle's
own magnitude, max |err| <= 2e-2 max |ref| and mean |err| <= 1e-2 mean |ref|.
Their arithmetic: P and dS rounded to bf16 (2^-9 relative each), float32
sums, the result rounded to bf16 (2^-9), and P recomputed from a float32
log-sum-exp taken over the forward's bf16-rounded weights (a per-row factor
within 2^-9 of 1).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import sparge_oracle as O

MAX_ABS, MEAN_ABS, TIE = 2e-2, 2e-3, 1e-5
GRAD_MAX_REL, GRAD_MEAN_REL = 2e-2, 1e-2
# dQ after the GPU forward (D = dO.O from the bf16 O): a row's dS sums to zero,
# so dQ_t = scale sum_u dS_tu K_u cancels; where the kept keys share a large
# common part its condition number sum|dS K| / |dQ| reaches 10-20 (smooth-field
# workload), and O's 2^-9 rounding moves dQ by up to ~20 * 2^-9 of |dQ|
DQ_CHAIN_MAX_REL, DQ_CHAIN_MEAN_REL = 5e-2, 2e-2


def to_gpu(bits_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits_u16)).view(torch.bfloat16).cuda()


def gpu_bits_to_bool(bits_i32: torch.Tensor, n_k: int) -> np.ndarray:
    w = bits_i32.cpu().numpy().view(np.uint32)
    j = np.arange(n_k)
    return ((w[..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)


def check_index_list(kept: np.ndarray, idx: np.ndarray, cnt: np.ndarray):
    """GPU idx/cnt must list exactly the set bits, ascending."""
    flat_k = kept.reshape(-1, kept.shape[-1])
    flat_i = idx.reshape(-1, idx.shape[-1])
    flat_c = cnt.reshape(-1)
    assert (flat_c == flat_k.sum(1)).all(), "count differs from popcount of the bitmask"
    for r in range(flat_k.shape[0]):
        want = np.nonzero(flat_k[r])[0]
        got = flat_i[r, : flat_c[r]]
        if not np.array_equal(got, want):
            raise AssertionError(f"row {r}: idx {got[:8]}... != bits {want[:8]}...")


def nan_like(t: torch.Tensor) -> torch.Tensor:
    """A tensor of t's shape, dtype and device, every element NaN."""
    return torch.full_like(t, float("nan"))


def assert_all_written(*ts: torch.Tensor):
    """Every element of these sentinel-filled outputs was overwritten with a
    finite value (checked on the device, over every head and row)."""
    for t in ts:
        bad = int((~torch.isfinite(t.float())).sum())
        assert bad == 0, f"{bad} of {t.numel()} output elements left unwritten or non-finite"


MASK_SENTINEL = 0x5A5A5A5A


def sentinel_mask_outputs(B, H, n_q, n_k, device):
    """Mask outputs (bits, idx, cnt, block scores) filled with values no call writes."""
    words = -(-n_k // 32)
    bits = torch.full((B, H, n_q, words), MASK_SENTINEL, dtype=torch.int32, device=device)
    idx = torch.full((B, H, n_q, n_k), -1, dtype=torch.int32, device=device)
    cnt = torch.full((B, H, n_q), -7, dtype=torch.int32, device=device)
    logits = torch.full((B, H, n_q, n_k), float("nan"), dtype=torch.float64, device=device)
    return bits, idx, cnt, logits


def check_bit_padding(bits: torch.Tensor, n_k: int):
    """Bits past n_k in the last word of a row name no key block, so they are clear."""
    if n_k % 32:
        last = bits[..., -1].cpu().numpy().view(np.uint32)
        assert not (last >> np.uint32(n_k % 32)).any(), "padding bits set past n_k"


def compare_masks(m: O.MaskResult, gpu_kept: np.ndarray, k_frac: float, p_mass: float,
                  exact: bool = True):
    """Returns (n_near_tie_rows, n_near_tie_rows_that_differ). Raises on failure.

    With `exact` (the default) every row must be bit-identical, near-tie rows
    included: both sides take the decision in float64 and differ only in
    summation order. Without it, near-tie rows need only be admissible."""
    n_k = gpu_kept.shape[-1]
    p = float(np.float32(p_mass))
    tie = m.margin < TIE
    same = (gpu_kept == m.kept).all(-1)
    bad = ~same & ~tie
    if bad.any():
        r = np.argwhere(bad)[0]
        raise AssertionError(f"mask differs on a row with margin {m.margin[tuple(r)]:.3e} "
                             f"at {tuple(r)}: gpu cnt {gpu_kept[tuple(r)].sum()} "
                             f"oracle cnt {m.cnt[tuple(r)]}; {bad.sum()} such rows")
    P = O.row_softmax(m.logits)
    for r in np.argwhere(tie & ~same):
        r = tuple(r)
        keep = gpu_kept[r]
        s, Pr = m.logits[r], P[r]
        assert keep.sum() >= m.K_k
        if p >= 1:
            assert keep.all()
            continue
        assert Pr[keep].sum() >= p - TIE
        if not keep.all():
            assert s[keep].min() >= s[~keep].max() - TIE
        low = np.argmin(np.where(keep, s, np.inf))
        rest = keep.copy()
        rest[low] = False
        assert rest.sum() < m.K_k or Pr[rest].sum() < p + TIE
    differ = int((tie & ~same).sum())
    if exact:
        assert differ == 0, f"{differ} near-tie rows differ from the oracle (admissible)"
    return int(tie.sum()), differ


def compare_outputs(o_gpu: np.ndarray, o_ref: np.ndarray):
    """o_gpu, o_ref: float64 arrays over the same valid rows."""
    err = np.abs(o_gpu - o_ref)
    assert np.isfinite(o_gpu).all(), "non-finite GPU output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def compare_grads(g_gpu: np.ndarray, g_ref: np.ndarray, name: str,
                  max_rel: float = GRAD_MAX_REL, mean_rel: float = GRAD_MEAN_REL):
    """Gradient arrays (float64) over the same sampled rows."""
    assert np.isfinite(g_gpu).all(), f"non-finite GPU {name}"
    err = np.abs(g_gpu - g_ref)
    scale_max, scale_mean = float(np.abs(g_ref).max()), float(np.abs(g_ref).mean())
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= max_rel * scale_max + 1e-6, f"{name}: max {mx:.3e} vs |ref| {scale_max:.3e}"
    assert mean <= mean_rel * scale_mean + 1e-7, \
        f"{name}: mean {mean:.3e} vs mean |ref| {scale_mean:.3e}"
    return mx / max(scale_max, 1e-30), mean / max(scale_mean, 1e-30)
