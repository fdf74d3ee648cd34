"""ctypes binding of libsparge.so with the C ABI's names.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. torch supplies device memory and the current HIP
stream. Importing this module does not need a GPU; calling an entry point
needs the built library (it raises if libsparge.so is missing) and
bfloat16 CUDA tensors.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparge.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3

# every symbol the public header declares
EXPORTS = ("sparge_mask_workspace_bytes", "sparge_mask_predict", "sparge_mask_pool",
           "sparge_mask_select",
           "sparge_mask_routed_workspace_bytes", "sparge_mask_predict_routed",
           "sparge_attn_workspace_bytes", "sparge_attn_fwd", "sparge_attn_pack",
           "sparge_attn_fwd_packed", "sparse_linear_workspace_bytes", "sparse_linear_attn_fwd",
           "sla2_mix_attn_fwd", "sparge_attn_fwd_lse", "sparge_attn_bwd_workspace_bytes",
           "sparge_attn_bwd", "sparse_linear_bwd_workspace_bytes", "sparse_linear_attn_bwd",
           "sla2_mix_attn_bwd", "sparge_attn_lowbit_workspace_bytes", "sparge_attn_fwd_lowbit",
           "svg2_attn_workspace_bytes", "svg2_attn_fwd", "sparge_mask_noalloc_scratch_bytes",
           "sparge_mask_predict_noalloc", "sparge_mask_pool_lowbit", "sparge_attn_lowbit_pack",
           "sparge_attn_fwd_lowbit_packed", "svg2_attn_pair_counts", "svg2_attn_cluster",
           "svg2_attn_apply", "sparge_last_error")

_lib = None


class SpargeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"sparge error {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libsparge.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_float, c_size, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
        L.sparge_mask_workspace_bytes.argtypes = [c_int] * 6
        L.sparge_mask_workspace_bytes.restype = c_size
        L.sparge_mask_predict.argtypes = [vp, vp] + [c_int] * 6 + [c_float] * 3 + [vp] * 5 + [
            c_size, vp]
        L.sparge_mask_predict.restype = c_int
        L.sparge_mask_noalloc_scratch_bytes.argtypes = []
        L.sparge_mask_noalloc_scratch_bytes.restype = c_size
        L.sparge_mask_predict_noalloc.argtypes = [vp, vp] + [c_int] * 6 + [c_float] * 3 + [
            vp] * 5
        L.sparge_mask_predict_noalloc.restype = c_int
        L.sparge_mask_pool_lowbit.argtypes = [vp, vp] + [c_int] * 6 + [vp, c_size, vp, c_size,
                                                                        vp]
        L.sparge_mask_pool_lowbit.restype = c_int
        L.sparge_attn_lowbit_pack.argtypes = [vp] + [c_int] * 5 + [vp, c_size, vp]
        L.sparge_attn_lowbit_pack.restype = c_int
        L.sparge_attn_fwd_lowbit_packed.argtypes = [vp, vp] + [c_int] * 6 + [c_float, vp, vp,
                                                                              c_size, vp]
        L.sparge_attn_fwd_lowbit_packed.restype = c_int
        L.svg2_attn_cluster.argtypes = [vp] * 3 + [c_int] * 8 + [c_float] * 2 + [vp, c_size, vp]
        L.svg2_attn_cluster.restype = c_int
        L.svg2_attn_apply.argtypes = [c_int] * 7 + [c_float, vp, vp, c_size, vp]
        L.svg2_attn_apply.restype = c_int
        L.svg2_attn_pair_counts.argtypes = [c_int] * 7 + [vp, vp, c_size, vp]
        L.svg2_attn_pair_counts.restype = c_int
        L.sparge_mask_pool.argtypes = [vp, vp] + [c_int] * 6 + [vp, c_size, vp]
        L.sparge_mask_pool.restype = c_int
        L.sparge_mask_select.argtypes = [c_int] * 6 + [c_float] * 3 + [vp] * 5 + [c_size, vp]
        L.sparge_mask_select.restype = c_int
        L.sparge_mask_routed_workspace_bytes.argtypes = [c_int] * 6
        L.sparge_mask_routed_workspace_bytes.restype = c_size
        L.sparge_mask_predict_routed.argtypes = [vp] * 4 + [c_int] * 6 + [c_float] * 3 + [
            vp] * 5 + [c_size, vp]
        L.sparge_mask_predict_routed.restype = c_int
        L.sparge_attn_workspace_bytes.argtypes = [c_int] * 4
        L.sparge_attn_workspace_bytes.restype = c_size
        L.sparge_attn_fwd.argtypes = [vp] * 5 + [c_int] * 6 + [c_float, vp, vp, c_size, vp]
        L.sparge_attn_fwd.restype = c_int
        L.sparge_attn_fwd_lse.argtypes = [vp] * 5 + [c_int] * 6 + [c_float, vp, vp, vp, c_size,
                                                                    vp]
        L.sparge_attn_fwd_lse.restype = c_int
        L.sparge_attn_bwd_workspace_bytes.argtypes = [c_int] * 6
        L.sparge_attn_bwd_workspace_bytes.restype = c_size
        L.sparge_attn_bwd.argtypes = [vp] * 8 + [c_int] * 6 + [c_float] + [vp] * 4 + [c_size, vp]
        L.sparge_attn_bwd.restype = c_int
        L.sparge_attn_lowbit_workspace_bytes.argtypes = [c_int] * 6
        L.sparge_attn_lowbit_workspace_bytes.restype = c_size
        L.sparge_attn_fwd_lowbit.argtypes = [vp] * 5 + [c_int] * 6 + [c_float, vp, vp, c_size, vp]
        L.sparge_attn_fwd_lowbit.restype = c_int
        L.svg2_attn_workspace_bytes.argtypes = [c_int] * 7
        L.svg2_attn_workspace_bytes.restype = c_size
        L.svg2_attn_fwd.argtypes = [vp] * 3 + [c_int] * 8 + [c_float, c_float, vp, vp, c_size, vp]
        L.svg2_attn_fwd.restype = c_int
        L.sparse_linear_bwd_workspace_bytes.argtypes = [c_int] * 4
        L.sparse_linear_bwd_workspace_bytes.restype = c_size
        for f in (L.sparse_linear_attn_bwd, L.sla2_mix_attn_bwd):
            f.argtypes = [vp] * 9 + [c_int] * 6 + [c_float, c_float] + [vp] * 4 + [c_size, vp]
            f.restype = c_int
        L.sparge_attn_pack.argtypes = [vp] + [c_int] * 4 + [vp, c_size, vp]
        L.sparge_attn_pack.restype = c_int
        L.sparge_attn_fwd_packed.argtypes = [vp] * 4 + [c_int] * 6 + [c_float, vp, vp, c_size, vp]
        L.sparge_attn_fwd_packed.restype = c_int
        L.sparse_linear_workspace_bytes.argtypes = [c_int] * 4
        L.sparse_linear_workspace_bytes.restype = c_size
        for f in (L.sparse_linear_attn_fwd, L.sla2_mix_attn_fwd):
            f.argtypes = [vp] * 6 + [c_int] * 6 + [c_float, c_float, vp, vp, vp, c_size, vp]
            f.restype = c_int
        L.sparge_last_error.argtypes = []
        L.sparge_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise SpargeError(rc, lib().sparge_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _qkv(*ts):
    shape = ts[0].shape
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("Q, K, V must be contiguous bfloat16 GPU tensors")
        if t.dim() != 4 or t.shape != shape:
            raise ValueError("Q, K, V must share one [B, H, N, d] shape")
    return shape


def _buf(t, name, dtype, shape, device):
    """A caller-supplied tensor the library reads or writes through a raw pointer."""
    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device
            or not t.is_contiguous() or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)} "
                         f"on {device}")
    return t


def _blocks(N, block_q, block_k):
    # invalid block sizes are left to the library, which rejects them
    return (-(-N // block_q) if block_q > 0 else 0), (-(-N // block_k) if block_k > 0 else 0)


def _lists(kv_idx, kv_cnt, q, block_q, block_k):
    B, H, N, _ = q.shape
    n_q, n_k = _blocks(N, block_q, block_k)
    _buf(kv_idx, "kv_idx", torch.int32, (B, H, n_q, n_k), q.device)
    _buf(kv_cnt, "kv_cnt", torch.int32, (B, H, n_q), q.device)


def _workspace(ws, need, device):
    """(workspace tensor, its size in bytes): a new one of `need` bytes, or the caller's."""
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    elif (not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return ws, ws.numel() * ws.element_size()


def default_scale(d: int) -> float:
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def mask_workspace_bytes(B, H, N, d, block_q, block_k) -> int:
    return lib().sparge_mask_workspace_bytes(B, H, N, d, block_q, block_k)


def _mask_outputs(q, block_q, block_k, out, return_logits):
    B, H, N, _ = q.shape
    n_q, n_k = _blocks(N, block_q, block_k)
    shapes = ((B, H, n_q, -(-n_k // 32)), (B, H, n_q, n_k), (B, H, n_q))
    if out is None:
        bits, idx, cnt = (torch.empty(sh, dtype=torch.int32, device=q.device) for sh in shapes)
    else:
        bits, idx, cnt = (_buf(t, name, torch.int32, sh, q.device)
                          for t, name, sh in zip(out, ("mask_bits", "kv_idx", "kv_cnt"), shapes))
    logits = None
    if return_logits:
        if out is not None and len(out) > 3:   # the caller's float64 score buffer
            logits = _buf(out[3], "block_logits", torch.float64, (B, H, n_q, n_k), q.device)
        else:
            logits = torch.empty((B, H, n_q, n_k), dtype=torch.float64, device=q.device)
    return bits, idx, cnt, logits


def sparge_mask_predict(q, k, block_q=128, block_k=64, k_frac=0.05, p_mass=0.9, scale=None,
                        return_logits=False, workspace=None, out=None):
    """Hybrid Top-k + Top-p block mask.

    Returns (mask_bits int32-viewed uint32 [B,H,n_q,ceil(n_k/32)], kv_idx int32
    [B,H,n_q,n_k], kv_cnt int32 [B,H,n_q][, logits float64 [B,H,n_q,n_k]]).
    `out` may name the tensors to write: (bits, idx, cnt[, logits]).
    """
    B, H, N, d = _qkv(q, k)
    bits, idx, cnt, logits = _mask_outputs(q, block_q, block_k, out, return_logits)
    workspace, ws_bytes = _workspace(workspace, mask_workspace_bytes(B, H, N, d, block_q, block_k),
                                     q.device)
    if scale is None:
        scale = default_scale(d)
    _check(lib().sparge_mask_predict(
        _ptr(q), _ptr(k), B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
        _ptr(bits), _ptr(idx), _ptr(cnt), _ptr(logits), _ptr(workspace), ws_bytes, _stream(q)))
    return (bits, idx, cnt, logits) if return_logits else (bits, idx, cnt)


def sparge_mask_predict_noalloc(q, k, block_q=128, block_k=64, k_frac=0.05, p_mass=0.9,
                                scale=None, return_logits=False, out=None):
    """sparge_mask_predict through the entry point that takes no workspace (its
    scratch is the library's per-GPU array); outputs as sparge_mask_predict.
    With `out` given (and, for return_logits, its float64 score buffer) this
    wrapper allocates nothing either."""
    B, H, N, d = _qkv(q, k)
    bits, idx, cnt, logits = _mask_outputs(q, block_q, block_k, out, return_logits)
    if scale is None:
        scale = default_scale(d)
    _check(lib().sparge_mask_predict_noalloc(
        _ptr(q), _ptr(k), B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
        _ptr(bits), _ptr(idx), _ptr(cnt), _ptr(logits), _stream(q)))
    return (bits, idx, cnt, logits) if return_logits else (bits, idx, cnt)


def sparge_mask_pool(q, k, block_q=128, block_k=64, workspace=None):
    """First half of sparge_mask_predict: pooled Q and K into the workspace,
    which it returns (pass it to sparge_mask_select)."""
    B, H, N, d = _qkv(q, k)
    workspace, ws_bytes = _workspace(workspace, mask_workspace_bytes(B, H, N, d, block_q, block_k),
                                     q.device)
    _check(lib().sparge_mask_pool(_ptr(q), _ptr(k), B, H, N, d, block_q, block_k,
                                  _ptr(workspace), ws_bytes, _stream(q)))
    return workspace


def sparge_mask_select(q, workspace, block_q=128, block_k=64, k_frac=0.05, p_mass=0.9,
                       scale=None, return_logits=False, out=None):
    """Second half of sparge_mask_predict, from the workspace sparge_mask_pool
    filled (q gives the shape, device and stream only); outputs as
    sparge_mask_predict."""
    B, H, N, d = _qkv(q)
    if workspace is None:
        raise ValueError("workspace must hold the pooled Q and K of sparge_mask_pool")
    workspace, ws_bytes = _workspace(workspace, 0, q.device)
    bits, idx, cnt, logits = _mask_outputs(q, block_q, block_k, out, return_logits)
    if scale is None:
        scale = default_scale(d)
    _check(lib().sparge_mask_select(B, H, N, d, block_q, block_k, k_frac, p_mass, scale,
                                    _ptr(bits), _ptr(idx), _ptr(cnt), _ptr(logits),
                                    _ptr(workspace), ws_bytes, _stream(q)))
    return (bits, idx, cnt, logits) if return_logits else (bits, idx, cnt)


def mask_routed_workspace_bytes(B, H, N, d, block_q, block_k) -> int:
    return lib().sparge_mask_routed_workspace_bytes(B, H, N, d, block_q, block_k)


def sparge_mask_predict_routed(q, k, w_q, w_k, block_q=128, block_k=64, k_frac=0.05,
                               p_mass=0.0, scale=None, return_logits=False, workspace=None,
                               out=None):
    """Block mask scored through the router's projections (w_q, w_k float32 GPU
    tensors [H, d, d]); outputs as sparge_mask_predict."""
    B, H, N, d = _qkv(q, k)
    for w in (w_q, w_k):
        if w.dtype != torch.float32 or w.device != q.device or tuple(w.shape) != (H, d, d):
            raise ValueError("w_q, w_k must be float32 GPU tensors [H, d, d]")
    w_q, w_k = w_q.contiguous(), w_k.contiguous()
    bits, idx, cnt, logits = _mask_outputs(q, block_q, block_k, out, return_logits)
    workspace, ws_bytes = _workspace(
        workspace, mask_routed_workspace_bytes(B, H, N, d, block_q, block_k), q.device)
    if scale is None:
        scale = default_scale(d)
    _check(lib().sparge_mask_predict_routed(
        _ptr(q), _ptr(k), _ptr(w_q), _ptr(w_k), B, H, N, d, block_q, block_k, k_frac, p_mass,
        scale, _ptr(bits), _ptr(idx), _ptr(cnt), _ptr(logits), _ptr(workspace), ws_bytes,
        _stream(q)))
    return (bits, idx, cnt, logits) if return_logits else (bits, idx, cnt)


def attn_workspace_bytes(B, H, N, d) -> int:
    return lib().sparge_attn_workspace_bytes(B, H, N, d)


def sparge_attn_fwd(q, k, v, kv_idx, kv_cnt, block_q=128, block_k=64, scale=None, out=None,
                    workspace=None):
    """Block-sparse attention over the key blocks listed in kv_idx/kv_cnt."""
    B, H, N, d = _qkv(q, k, v)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(workspace, attn_workspace_bytes(B, H, N, d), q.device)
    _check(lib().sparge_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), B, H,
                                 N, d, block_q, block_k, scale, _ptr(o), _ptr(workspace),
                                 ws_bytes, _stream(q)))
    return o


def sparge_attn_fwd_lse(q, k, v, kv_idx, kv_cnt, block_q=128, block_k=64, scale=None,
                        out=None, workspace=None):
    """sparge_attn_fwd plus each row's log-sum-exp (float32 [B, H, N]); returns (o, lse)."""
    B, H, N, d = _qkv(q, k, v)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o = _buf(out[0], "out[0]", torch.bfloat16, q.shape, q.device)
        lse = _buf(out[1], "out[1] (lse)", torch.float32, (B, H, N), q.device)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(workspace, attn_workspace_bytes(B, H, N, d), q.device)
    _check(lib().sparge_attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), B,
                                     H, N, d, block_q, block_k, scale, _ptr(o), _ptr(lse),
                                     _ptr(workspace), ws_bytes, _stream(q)))
    return o, lse


def _grads(q, out):
    if out is None:
        return tuple(torch.empty_like(q) for _ in range(3))
    return tuple(_buf(t, name, torch.bfloat16, q.shape, q.device)
                 for t, name in zip(out, ("dq", "dk", "dv")))


def attn_bwd_workspace_bytes(B, H, N, d, block_q=128, block_k=64) -> int:
    return lib().sparge_attn_bwd_workspace_bytes(B, H, N, d, block_q, block_k)


def sparge_attn_bwd(q, k, v, o, d_o, lse, kv_idx, kv_cnt, block_q=128, block_k=64, scale=None,
                    out=None, workspace=None):
    """dQ, dK, dV of the block-sparse attention for the upstream gradient d_o."""
    B, H, N, d = _qkv(q, k, v, o, d_o)
    _buf(lse, "lse", torch.float32, (B, H, N), q.device)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    dq, dk, dv = _grads(q, out)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(
        workspace, attn_bwd_workspace_bytes(B, H, N, d, block_q, block_k), q.device)
    _check(lib().sparge_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                 _ptr(kv_idx), _ptr(kv_cnt), B, H, N, d, block_q, block_k, scale,
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                 _stream(q)))
    return dq, dk, dv


def lowbit_workspace_bytes(B, H, N, d, block_q=128, block_k=64) -> int:
    return lib().sparge_attn_lowbit_workspace_bytes(B, H, N, d, block_q, block_k)


def sparge_attn_fwd_lowbit(q, k, v, kv_idx, kv_cnt, block_q=128, block_k=64, scale=None,
                           out=None, workspace=None):
    """The sparse branch with INT8 Q/K and e4m3 P/V (see sparge.h)."""
    B, H, N, d = _qkv(q, k, v)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(
        workspace, lowbit_workspace_bytes(B, H, N, d, block_q, block_k), q.device)
    _check(lib().sparge_attn_fwd_lowbit(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), B,
                                        H, N, d, block_q, block_k, scale, _ptr(o),
                                        _ptr(workspace), ws_bytes, _stream(q)))
    return o


def sparge_mask_pool_lowbit(q, k, block_q=128, block_k=64, workspace=None, lowbit_workspace=None):
    """sparge_mask_pool whose pass also writes the INT8 codes and scales of Q and K
    into the low-bit workspace; returns (workspace, lowbit_workspace)."""
    B, H, N, d = _qkv(q, k)
    workspace, ws_bytes = _workspace(workspace, mask_workspace_bytes(B, H, N, d, block_q, block_k),
                                     q.device)
    lowbit_workspace, lb_bytes = _workspace(
        lowbit_workspace, lowbit_workspace_bytes(B, H, N, d, block_q, block_k), q.device)
    _check(lib().sparge_mask_pool_lowbit(_ptr(q), _ptr(k), B, H, N, d, block_q, block_k,
                                         _ptr(workspace), ws_bytes, _ptr(lowbit_workspace),
                                         lb_bytes, _stream(q)))
    return workspace, lowbit_workspace


def sparge_attn_lowbit_pack(v, lowbit_workspace, block_q=128):
    """V's channel scales and packed e4m3 codes into the low-bit workspace."""
    B, H, N, d = _qkv(v)
    if lowbit_workspace is None:
        raise ValueError("lowbit_workspace must be the low-bit workspace of the pooling call")
    lowbit_workspace, lb_bytes = _workspace(lowbit_workspace, 0, v.device)
    _check(lib().sparge_attn_lowbit_pack(_ptr(v), B, H, N, d, block_q, _ptr(lowbit_workspace),
                                         lb_bytes, _stream(v)))
    return lowbit_workspace


def sparge_attn_fwd_lowbit_packed(q, kv_idx, kv_cnt, lowbit_workspace, block_q=128, block_k=64,
                                  scale=None, out=None):
    """The low-bit attention from the codes in the workspace (q gives the shape,
    device and stream only)."""
    B, H, N, d = _qkv(q)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    if lowbit_workspace is None:
        raise ValueError("lowbit_workspace must hold the codes of the pooling and pack calls")
    lowbit_workspace, lb_bytes = _workspace(lowbit_workspace, 0, q.device)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = default_scale(d)
    _check(lib().sparge_attn_fwd_lowbit_packed(_ptr(kv_idx), _ptr(kv_cnt), B, H, N, d, block_q,
                                               block_k, scale, _ptr(o), _ptr(lowbit_workspace),
                                               lb_bytes, _stream(q)))
    return o


def svg2_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters) -> int:
    return lib().svg2_attn_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters)


def svg2_attn_fwd(q, k, v, n_q_clusters, n_k_clusters, iters=10, p_mass=0.9, block_q=128,
                  scale=None, out=None, workspace=None):
    """SVG2: k-means permutation, size-weighted centroid Top-p, clustered attention."""
    B, H, N, d = _qkv(q, k, v)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(
        workspace, svg2_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters),
        q.device)
    _check(lib().svg2_attn_fwd(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, block_q, n_q_clusters,
                               n_k_clusters, iters, p_mass, scale, _ptr(o), _ptr(workspace),
                               ws_bytes, _stream(q)))
    return o


def svg2_attn_cluster(q, k, v, n_q_clusters, n_k_clusters, iters=10, p_mass=0.9, block_q=128,
                      scale=None, workspace=None):
    """SVG2 steps 1-3 and the gathers into the workspace, which it returns."""
    B, H, N, d = _qkv(q, k, v)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(
        workspace, svg2_workspace_bytes(B, H, N, d, block_q, n_q_clusters, n_k_clusters),
        q.device)
    _check(lib().svg2_attn_cluster(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, block_q, n_q_clusters,
                                   n_k_clusters, iters, p_mass, scale, _ptr(workspace), ws_bytes,
                                   _stream(q)))
    return workspace


def svg2_attn_apply(q, n_q_clusters, n_k_clusters, workspace, block_q=128, scale=None, out=None):
    """SVG2 step 4 from the workspace of svg2_attn_cluster (q gives the shape,
    device and stream only)."""
    B, H, N, d = _qkv(q)
    if workspace is None:
        raise ValueError("workspace must be the one svg2_attn_cluster filled")
    workspace, ws_bytes = _workspace(workspace, 0, q.device)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = default_scale(d)
    _check(lib().svg2_attn_apply(B, H, N, d, block_q, n_q_clusters, n_k_clusters, scale, _ptr(o),
                                 _ptr(workspace), ws_bytes, _stream(q)))
    return o


def svg2_attn_pair_counts(q, n_q_clusters, n_k_clusters, workspace, block_q=128):
    """After svg2_attn_fwd with this workspace: int64 [B, H, 2] of (token pairs
    that take part, pairs the kernel evaluates) per head (q gives the shape,
    device and stream only)."""
    B, H, N, d = _qkv(q)
    if workspace is None:
        raise ValueError("workspace must be the one svg2_attn_fwd used")
    workspace, ws_bytes = _workspace(workspace, 0, q.device)
    counts = torch.empty((B, H, 2), dtype=torch.int64, device=q.device)
    _check(lib().svg2_attn_pair_counts(B, H, N, d, block_q, n_q_clusters, n_k_clusters,
                                       _ptr(counts), _ptr(workspace), ws_bytes, _stream(q)))
    return counts


def linear_bwd_workspace_bytes(B, H, N, d) -> int:
    return lib().sparse_linear_bwd_workspace_bytes(B, H, N, d)


def _linear_bwd(fn, q, k, v, o, d_o, lse, kv_idx, kv_cnt, alpha, block_q, block_k, scale,
                drop_below, out, workspace):
    B, H, N, d = _qkv(q, k, v, o, d_o)
    _buf(lse, "lse", torch.float32, (B, H, N), q.device)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    dq, dk, dv = _grads(q, out)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(workspace, linear_bwd_workspace_bytes(B, H, N, d), q.device)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(kv_idx),
              _ptr(kv_cnt), _ptr(alpha), B, H, N, d, block_q, block_k, scale, drop_below,
              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(q)))
    return dq, dk, dv


def sparse_linear_attn_bwd(q, k, v, o, d_o, lse, kv_idx, kv_cnt, alpha, block_q=128, block_k=64,
                           scale=None, drop_below=0.0, out=None, workspace=None):
    """dQ, dK, dV of O = O_s + alpha[h] O_l (lse from sparse_linear_attn_fwd)."""
    H = q.shape[1]
    if alpha.dtype != torch.float32 or alpha.device != q.device or alpha.numel() != H:
        raise ValueError("alpha must be a float32 GPU tensor of H values")
    return _linear_bwd(lib().sparse_linear_attn_bwd, q, k, v, o, d_o, lse, kv_idx, kv_cnt,
                       alpha.contiguous(), block_q, block_k, scale, drop_below, out, workspace)


def sla2_mix_attn_bwd(q, k, v, o, d_o, lse, kv_idx, kv_cnt, alpha, block_q=128, block_k=64,
                      scale=None, drop_below=0.0, out=None, workspace=None):
    """dQ, dK, dV of the SLA2 mix (lse from sla2_mix_attn_fwd); alpha float32 [H, d]."""
    H, d = q.shape[1], q.shape[3]
    if alpha.dtype != torch.float32 or alpha.device != q.device or tuple(alpha.shape) != (H, d):
        raise ValueError("alpha must be a float32 GPU tensor of shape [H, d]")
    return _linear_bwd(lib().sla2_mix_attn_bwd, q, k, v, o, d_o, lse, kv_idx, kv_cnt,
                       alpha.contiguous(), block_q, block_k, scale, drop_below, out, workspace)


def sparge_attn_pack(v, workspace=None):
    """Pack V for sparge_attn_fwd_packed; returns the workspace holding it."""
    B, H, N, d = _qkv(v)
    workspace, ws_bytes = _workspace(workspace, attn_workspace_bytes(B, H, N, d), v.device)
    _check(lib().sparge_attn_pack(_ptr(v), B, H, N, d, _ptr(workspace), ws_bytes, _stream(v)))
    return workspace


def sparge_attn_fwd_packed(q, k, kv_idx, kv_cnt, workspace, block_q=128, block_k=64, scale=None,
                           out=None):
    """Block-sparse attention with V already packed into `workspace`."""
    B, H, N, d = _qkv(q, k)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if scale is None:
        scale = default_scale(d)
    if workspace is None:
        raise ValueError("workspace must hold V packed by sparge_attn_pack")
    workspace, ws_bytes = _workspace(workspace, 0, q.device)
    _check(lib().sparge_attn_fwd_packed(_ptr(q), _ptr(k), _ptr(kv_idx), _ptr(kv_cnt), B, H, N, d,
                                        block_q, block_k, scale, _ptr(o), _ptr(workspace),
                                        ws_bytes, _stream(q)))
    return o


def linear_workspace_bytes(B, H, N, d) -> int:
    return lib().sparse_linear_workspace_bytes(B, H, N, d)


def _linear(fn, q, k, v, kv_idx, kv_cnt, alpha, block_q, block_k, scale, drop_below,
            workspace, out, lse=None):
    B, H, N, d = _qkv(q, k, v)
    _lists(kv_idx, kv_cnt, q, block_q, block_k)
    o = torch.empty_like(q) if out is None else _buf(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is not None:
        _buf(lse, "lse", torch.float32, (B, H, N), q.device)
    if scale is None:
        scale = default_scale(d)
    workspace, ws_bytes = _workspace(workspace, linear_workspace_bytes(B, H, N, d), q.device)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), _ptr(alpha), B, H, N, d,
              block_q, block_k, scale, drop_below, _ptr(o), None if lse is None else _ptr(lse),
              _ptr(workspace), ws_bytes, _stream(q)))
    return o


def sparse_linear_attn_fwd(q, k, v, kv_idx, kv_cnt, alpha, block_q=128, block_k=64,
                           scale=None, drop_below=0.0, workspace=None, out=None, lse=None):
    """Sparse attention plus alpha[h] times elu+1 linear attention over dropped blocks;
    heads with |alpha[h]| <= drop_below skip the linear branch."""
    H = q.shape[1]
    if alpha.dtype != torch.float32 or alpha.device != q.device or alpha.numel() != H:
        raise ValueError("alpha must be a float32 GPU tensor of H values")
    return _linear(lib().sparse_linear_attn_fwd, q, k, v, kv_idx, kv_cnt, alpha.contiguous(),
                   block_q, block_k, scale, drop_below, workspace, out, lse)


def sla2_mix_attn_fwd(q, k, v, kv_idx, kv_cnt, alpha, block_q=128, block_k=64, scale=None,
                      drop_below=0.0, workspace=None, out=None, lse=None):
    """SLA2 mix alpha[h][c] O_s + (1 - alpha[h][c]) O_l; alpha float32 [H, d] on the GPU.
    Heads with every |1 - alpha[h][c]| <= drop_below skip the linear branch."""
    H, d = q.shape[1], q.shape[3]
    if alpha.dtype != torch.float32 or alpha.device != q.device or tuple(alpha.shape) != (H, d):
        raise ValueError("alpha must be a float32 GPU tensor of shape [H, d]")
    return _linear(lib().sla2_mix_attn_fwd, q, k, v, kv_idx, kv_cnt, alpha.contiguous(),
                   block_q, block_k, scale, drop_below, workspace, out, lse)
