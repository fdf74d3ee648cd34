"""The C ABI without a GPU: the library loads, exports every declared symbol,
sizes its workspaces, and rejects bad arguments before it touches HIP."""
import ctypes
import math
import os
import re

import pytest

from block_sparse_attention_softmax_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sparge.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libsparge.so not built")

A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: checks fail first
MIS = ctypes.c_void_p(0x10002)    # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, re.M)))


def test_header_declares_the_bound_symbols():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_mask_workspace_bytes():
    L = binding.lib()
    up = lambda x: (x + 255) // 256 * 256
    B, H, N, d = 1, 12, 32760, 128
    n_q, n_k = math.ceil(N / 128), math.ceil(N / 64)
    want = up(B * H * n_q * d * 8) + up(B * H * n_k * d * 8) + up(B * H * n_q * n_k * 8)
    assert L.sparge_mask_workspace_bytes(B, H, N, d, 128, 64) == want
    assert L.sparge_mask_workspace_bytes(1, 1, 100, 96, 128, 64) == 0       # bad d
    assert L.sparge_mask_workspace_bytes(1, 1, 64 * 4097, 64, 64, 64) == 0  # > 4096 blocks
    packed_v = 40 * math.ceil(75600 / 64) * 64 * 128 * 2
    assert L.sparge_attn_workspace_bytes(1, 40, 75600, 128) == packed_v
    assert L.sparge_attn_workspace_bytes(1, 40, 75600, 96) == 0
    n_k, n_q = math.ceil(75600 / 64), math.ceil(75600 / 128)
    lin = (packed_v
           + up(40 * n_k * 2 * (128 * 128 + 128) * 2)   # per-key-block summaries, 2 bf16 planes
           + up(40 * n_q * math.ceil(n_k / 32) * 4)     # drop bits
           + up(40 * n_q * 2 * 128 * 128 * 2)           # dropped-block sums, 2 bf16 planes
           + up(40 * n_q * 128 * 4)                     # their phi(K) sums, float32
           + up(40 * 4) + up((2 + 2 * 40) * 4))         # branch flags, head lists
    assert L.sparse_linear_workspace_bytes(1, 40, 75600, 128) == lin
    assert L.sparse_linear_workspace_bytes(1, 1, 64 * 4097, 64) == 0  # > 4096 key blocks


def _mask(**kw):
    args = dict(q=A, k=A, B=1, H=2, N=1024, d=64, bq=64, bk=64, kf=0.1, p=0.9, sc=0.125,
                bits=A, idx=A, cnt=A, logits=None, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    L = binding.lib()
    return L.sparge_mask_predict(*args.values())


def _attn(**kw):
    args = dict(q=A, k=A, v=A, idx=A, cnt=A, B=1, H=2, N=1024, d=64, bq=64, bk=64, sc=0.125,
                o=A, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_attn_fwd(*args.values())


def _pack(**kw):
    args = dict(v=A, B=1, H=2, N=1024, d=64, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_attn_pack(*args.values())


def _packed(**kw):
    args = dict(q=A, k=A, idx=A, cnt=A, B=1, H=2, N=1024, d=64, bq=64, bk=64, sc=0.125, o=A,
                ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_attn_fwd_packed(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), -1), (dict(v=MIS), -1), (dict(ws=None), -1), (dict(wsb=1000), -1),
    (dict(d=32), -2), (dict(N=0), -1)])
def test_pack_rejects_bad_arguments(kw, code):
    assert _pack(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=MIS), -1), (dict(o=None), -1), (dict(idx=None), -1),
    (dict(ws=None), -1), (dict(wsb=1000), -1), (dict(bk=16), -2), (dict(sc=0.0), -1)])
def test_packed_attn_rejects_bad_arguments(kw, code):
    assert _packed(**kw) == code


def _lin(fn="sparse_linear_attn_fwd", **kw):
    args = dict(q=A, k=A, v=A, idx=A, cnt=A, alpha=A, B=1, H=2, N=1024, d=64, bq=64, bk=64,
                sc=0.125, drop=0.0, o=A, lse=None, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return getattr(binding.lib(), fn)(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(bits=None), -1), (dict(ws=None), -1),
    (dict(q=MIS), -1), (dict(idx=ctypes.c_void_p(0x10001)), -1),
    (dict(logits=ctypes.c_void_p(0x10004)), -1),
    (dict(d=96), -2), (dict(bq=32), -2), (dict(bk=128), -2),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1),
    (dict(kf=0.0), -1), (dict(kf=1.5), -1), (dict(kf=float("nan")), -1),
    (dict(p=-0.1), -1), (dict(p=float("inf")), -1), (dict(p=float("nan")), -1),
    (dict(sc=0.0), -1), (dict(sc=float("nan")), -1),
    (dict(wsb=100), -1), (dict(N=64 * 4097), -2),
])
def test_mask_rejects_bad_arguments(kw, code):
    assert _mask(**kw) == code
    assert binding.lib().sparge_last_error().decode()


def _pool(**kw):
    args = dict(q=A, k=A, B=1, H=2, N=1024, d=64, bq=64, bk=64, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_mask_pool(*args.values())


def _select(**kw):
    args = dict(B=1, H=2, N=1024, d=64, bq=64, bk=64, kf=0.1, p=0.9, sc=0.125, bits=A, idx=A,
                cnt=A, logits=None, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_mask_select(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=MIS), -1), (dict(ws=None), -1), (dict(ws=MIS), -1),
    (dict(d=96), -2), (dict(bq=32), -2), (dict(N=0), -1), (dict(wsb=100), -1),
    (dict(N=64 * 4097), -2)])
def test_mask_pool_rejects_bad_arguments(kw, code):
    assert _pool(**kw) == code
    assert binding.lib().sparge_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(bits=None), -1), (dict(idx=MIS), -1), (dict(cnt=None), -1), (dict(ws=None), -1),
    (dict(logits=ctypes.c_void_p(0x10004)), -1), (dict(kf=0.0), -1), (dict(p=float("nan")), -1),
    (dict(sc=-1.0), -1), (dict(d=96), -2), (dict(bk=128), -2), (dict(wsb=100), -1)])
def test_mask_select_rejects_bad_arguments(kw, code):
    assert _select(**kw) == code
    assert binding.lib().sparge_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(cnt=None), -1), (dict(v=MIS), -1),
    (dict(d=80), -2), (dict(bq=256), -2), (dict(bk=32), -2), (dict(N=0), -1),
    (dict(sc=-1.0), -1), (dict(sc=float("inf")), -1),
    (dict(ws=None), -1), (dict(ws=MIS), -1), (dict(wsb=1024 * 64 * 2 * 2 - 1), -1),
    (dict(N=2**31 - 1, B=1, H=1), -1),  # block counts would overflow 32-bit arithmetic
])
def test_attn_rejects_bad_arguments(kw, code):
    assert _attn(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(alpha=None), -1), (dict(ws=None), -1), (dict(wsb=16), -1), (dict(q=None), -1),
    (dict(d=32), -2), (dict(alpha=ctypes.c_void_p(0x10001)), -1),
    (dict(bq=128), -2),  # the linear branch is built for block_q == d
])
@pytest.mark.parametrize("fn", ["sparse_linear_attn_fwd", "sla2_mix_attn_fwd"])
def test_linear_rejects_bad_arguments(fn, kw, code):
    assert _lin(fn, **kw) == code
    assert binding.lib().sparge_last_error().decode()


def test_mix_alpha_needs_16_byte_alignment():
    # the mix reads four channels of alpha at once; the added form one value
    assert _lin("sla2_mix_attn_fwd", alpha=ctypes.c_void_p(0x10004)) == -1
    assert "misaligned" in binding.lib().sparge_last_error().decode()
    assert _lin("sparse_linear_attn_fwd", alpha=ctypes.c_void_p(0x10004), q=None) == -1
    assert "null" in binding.lib().sparge_last_error().decode()


def test_error_message_is_per_call():
    assert _attn(d=80) == -2
    assert "d must be" in binding.lib().sparge_last_error().decode()
    assert _mask(kf=0.0) == -1
    assert "k_frac" in binding.lib().sparge_last_error().decode()


def test_routed_mask_workspace_bytes():
    L = binding.lib()
    up = lambda x: (x + 255) // 256 * 256
    B, H, N, d = 1, 12, 32760, 128
    n_q, n_k = math.ceil(N / 128), math.ceil(N / 64)
    plain = L.sparge_mask_workspace_bytes(B, H, N, d, 128, 64)
    want = plain + 2 * up(B * H * d * d * 8) + up(B * H * n_q * d * 8) + up(B * H * n_k * d * 8)
    assert L.sparge_mask_routed_workspace_bytes(B, H, N, d, 128, 64) == want
    assert L.sparge_mask_routed_workspace_bytes(1, 1, 100, 96, 128, 64) == 0


def _routed(**kw):
    args = dict(q=A, k=A, wq=A, wk=A, B=1, H=2, N=1024, d=64, bq=64, bk=64, kf=0.1, p=0.9,
                sc=0.125, bits=A, idx=A, cnt=A, logits=None, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_mask_predict_routed(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(wq=None), -1), (dict(wk=None), -1), (dict(wq=ctypes.c_void_p(0x10002)), -1),
    (dict(d=96), -2), (dict(kf=0.0), -1), (dict(q=None), -1),
    (dict(wsb=binding.lib().sparge_mask_workspace_bytes(1, 2, 1024, 64, 64, 64)), -1),
])
def test_routed_mask_rejects_bad_arguments(kw, code):
    assert _routed(**kw) == code
    assert binding.lib().sparge_last_error().decode()


def test_backward_workspace_bytes():
    L = binding.lib()
    up = lambda x: (x + 255) // 256 * 256
    B, H, N, d, bq = 1, 12, 32760, 128, 128
    BH, n_q, n_k = B * H, math.ceil(N / bq), math.ceil(N / 64)
    packed = up(BH * n_k * 64 * d * 2)
    want = (packed + 2 * up(BH * n_q * bq * 4) + up(BH * n_k * n_q * 4) + up(BH * n_k * 4)
            + up(BH * (n_k + 1) * 4) + up(BH * n_q * n_k * 4))
    assert L.sparge_attn_bwd_workspace_bytes(B, H, N, d, bq, 64) == want
    assert L.sparge_attn_bwd_workspace_bytes(1, 1, 100, 96, 128, 64) == 0


def _bwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, do=A, lse=A, idx=A, cnt=A, B=1, H=2, N=1024, d=64, bq=64,
                bk=64, sc=0.125, dq=A, dk=A, dv=A, ws=A, wsb=1 << 30, st=None)
    args.update(kw)
    return binding.lib().sparge_attn_bwd(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), -1), (dict(lse=None), -1), (dict(dq=None), -1), (dict(ws=None), -1),
    (dict(do=MIS), -1), (dict(dk=MIS), -1), (dict(lse=ctypes.c_void_p(0x10001)), -1),
    (dict(wsb=1024), -1), (dict(d=96), -2), (dict(bk=128), -2), (dict(sc=0.0), -1),
    (dict(q=None), -1),
])
def test_backward_rejects_bad_arguments(kw, code):
    assert _bwd(**kw) == code
    assert binding.lib().sparge_last_error().decode()


def test_forward_lse_rejects_bad_arguments():
    L = binding.lib()
    args = [A, A, A, A, A, 1, 2, 1024, 64, 64, 64, 0.125, A, None, A, 1 << 30, None]
    assert L.sparge_attn_fwd_lse(*args) == -1
    args[13] = ctypes.c_void_p(0x10002)
    assert L.sparge_attn_fwd_lse(*args) == -1
    assert "lse" in L.sparge_last_error().decode()


def test_linear_backward_workspace_and_rejections():
    L = binding.lib()
    plain = L.sparge_attn_bwd_workspace_bytes(1, 12, 32760, 128, 128, 64)
    lin = L.sparse_linear_bwd_workspace_bytes(1, 12, 32760, 128)
    assert lin > plain
    assert L.sparse_linear_bwd_workspace_bytes(1, 1, 64 * 4097, 64) == 0  # > 4096 key blocks
    args = dict(q=A, k=A, v=A, o=A, do=A, lse=A, idx=A, cnt=A, alpha=A, B=1, H=2, N=1024, d=64,
                bq=64, bk=64, sc=0.125, drop=0.0, dq=A, dk=A, dv=A, ws=A, wsb=1 << 30, st=None)
    for fn in ("sparse_linear_attn_bwd", "sla2_mix_attn_bwd"):
        for kw, code in ((dict(alpha=None), -1), (dict(bq=128), -2), (dict(wsb=1024), -1),
                         (dict(d=96), -2), (dict(do=MIS), -1)):
            a2 = dict(args)
            a2.update(kw)
            assert getattr(L, fn)(*a2.values()) == code, (fn, kw)
    a2 = dict(args)
    a2.update(alpha=ctypes.c_void_p(0x10004))  # 4-byte aligned: enough for the added form only
    assert L.sla2_mix_attn_bwd(*a2.values()) == -1


def test_lowbit_workspace_and_rejections():
    L = binding.lib()
    up = lambda x: (x + 255) // 256 * 256
    B, H, N, d = 1, 12, 32760, 128
    n_q, n_k = math.ceil(N / 128), math.ceil(N / 64)
    BH = B * H
    want = (2 * up(BH * N * d) + up(BH * n_q * 4) + up(BH * n_k * 4) + up(BH * d * 4)
            + up(BH * n_k * 64 * d))
    assert L.sparge_attn_lowbit_workspace_bytes(B, H, N, d, 128, 64) == want
    assert L.sparge_attn_lowbit_workspace_bytes(1, 1, 100, 96, 128, 64) == 0
    args = [A, A, A, A, A, 1, 2, 1024, 64, 64, 64, 0.125, A, A, 1 << 30, None]
    bad = list(args)
    bad[13] = ctypes.c_void_p(0x10010)                   # 16- but not 256-byte aligned
    assert L.sparge_attn_fwd_lowbit(*bad) == -1
    bad = list(args)
    bad[14] = 1024
    assert L.sparge_attn_fwd_lowbit(*bad) == -1
    bad = list(args)
    bad[8] = 80
    assert L.sparge_attn_fwd_lowbit(*bad) == -2


def test_svg2_workspace_and_rejections():
    L = binding.lib()
    assert L.svg2_attn_workspace_bytes(1, 12, 32760, 128, 128, 256, 512) > 0
    assert L.svg2_attn_workspace_bytes(1, 1, 100, 128, 128, 0, 8) == 0
    assert L.svg2_attn_workspace_bytes(1, 1, 100, 128, 128, 8, 101) == 0   # more clusters than tokens
    args = [A, A, A, 1, 2, 1024, 64, 64, 8, 16, 3, 0.9, 0.125, A, A, 1 << 34, None]
    for i, v, code in ((8, 0, -1), (9, 5000, -1), (10, -1, -1), (11, -0.5, -1), (12, 0.0, -1),
                       (6, 96, -2), (14, ctypes.c_void_p(0x10010), -1), (15, 1024, -1)):
        bad = list(args)
        bad[i] = v
        assert L.svg2_attn_fwd(*bad) == code, (i, v)


def _noalloc(**kw):
    args = dict(q=A, k=A, B=1, H=2, N=1024, d=64, bq=64, bk=64, kf=0.1, p=0.9, sc=0.125,
                bits=A, idx=A, cnt=A, logits=None, st=None)
    args.update(kw)
    return binding.lib().sparge_mask_predict_noalloc(*args.values())


def test_noalloc_mask_checks_arguments_before_any_hip_call():
    L = binding.lib()
    assert L.sparge_mask_noalloc_scratch_bytes() == 64 << 20
    for kw, code in [(dict(d=96), binding.ERR_UNSUPPORTED), (dict(kf=0.0), binding.ERR_INVALID_ARG),
                     (dict(p=-1.0), binding.ERR_INVALID_ARG), (dict(q=None), binding.ERR_INVALID_ARG),
                     (dict(bits=MIS), binding.ERR_INVALID_ARG),
                     (dict(logits=MIS), binding.ERR_INVALID_ARG),
                     (dict(N=64 * 4097), binding.ERR_UNSUPPORTED)]:
        assert _noalloc(**kw) == code, kw
    # beyond the 64 MiB scratch: Wan-14B-720p's scores alone are 224 MB, and its
    # means 72.6 MB, so it is refused with or without block_logits
    for logits in (None, A):
        assert _noalloc(B=1, H=40, N=75600, d=128, bq=128, logits=logits) == binding.ERR_UNSUPPORTED
        assert b"scratch" in L.sparge_last_error()
    # Wan-1.3B needs 22 MB: it passes every check (a call here would reach HIP)
    up = lambda x: (x + 255) // 256 * 256
    need = up(12 * 256 * 128 * 8) + up(12 * 512 * 128 * 8) + up(12 * 256 * 512 * 8)
    assert need < 64 << 20


def test_mask_workspace_without_scores_when_block_logits_given():
    """With block_logits the scores go to the caller's buffer: a workspace of
    the pooled means alone is enough, and one byte less is refused."""
    up = lambda x: (x + 255) // 256 * 256
    means = up(2 * 16 * 64 * 8) + up(2 * 16 * 64 * 8)
    assert _mask(wsb=means - 1, logits=A) == binding.ERR_INVALID_ARG
    assert b"workspace" in binding.lib().sparge_last_error()
    assert _mask(wsb=means + up(2 * 16 * 16 * 8) - 1) == binding.ERR_INVALID_ARG


def test_lowbit_parts_check_arguments():
    L = binding.lib()
    need = L.sparge_attn_lowbit_workspace_bytes(1, 2, 1024, 64, 64, 64)
    mws = L.sparge_mask_workspace_bytes(1, 2, 1024, 64, 64, 64)
    # pooling with codes: null / misaligned / small low-bit workspace, bad shape
    assert L.sparge_mask_pool_lowbit(A, A, 1, 2, 1024, 64, 64, 64, A, mws, None, need,
                                     None) == binding.ERR_INVALID_ARG
    assert L.sparge_mask_pool_lowbit(A, A, 1, 2, 1024, 64, 64, 64, A, mws,
                                     ctypes.c_void_p(0x10010), need, None) == binding.ERR_INVALID_ARG
    assert b"256-byte" in L.sparge_last_error()
    assert L.sparge_mask_pool_lowbit(A, A, 1, 2, 1024, 64, 64, 64, A, mws, A, need - 1,
                                     None) == binding.ERR_INVALID_ARG
    assert b"lowbit_workspace too small" in L.sparge_last_error()
    assert L.sparge_mask_pool_lowbit(A, A, 1, 2, 1024, 96, 64, 64, A, mws, A, need,
                                     None) == binding.ERR_UNSUPPORTED
    # the V pack reads v only; the attention reads lists, o and the workspace only
    assert L.sparge_attn_lowbit_pack(None, 1, 2, 1024, 64, 64, A, need, None) == binding.ERR_INVALID_ARG
    assert L.sparge_attn_lowbit_pack(MIS, 1, 2, 1024, 64, 64, A, need, None) == binding.ERR_INVALID_ARG
    assert L.sparge_attn_lowbit_pack(A, 1, 2, 1024, 64, 64, A, need - 1, None) == binding.ERR_INVALID_ARG
    f = L.sparge_attn_fwd_lowbit_packed
    assert f(A, A, 1, 2, 1024, 64, 64, 64, ctypes.c_float(0.0), A, A, need, None) == binding.ERR_INVALID_ARG
    assert f(None, A, 1, 2, 1024, 64, 64, 64, ctypes.c_float(0.125), A, A, need, None) == binding.ERR_INVALID_ARG
    assert f(A, A, 1, 2, 1024, 64, 64, 32, ctypes.c_float(0.125), A, A, need, None) == binding.ERR_UNSUPPORTED
    assert f(A, A, 1, 2, 1024, 64, 64, 64, ctypes.c_float(0.125), MIS, A, need, None) == binding.ERR_INVALID_ARG
