"""The C interface without a GPU: the library loads, exports every function include/nvfp4.h declares,
and rejects invalid arguments with the documented status before anything is launched. Pointers here
are fake aligned addresses; no call in this file reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import nvfp4_w4a4_quantized_quantize_amd as nv
from nvfp4_w4a4_quantized_quantize_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if hipbuild.stale():
        hipbuild.build()
    return nv.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(nv.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(9):
        assert nv.status_string(s) not in ("", "unknown status")
    assert nv.status_string(99) == "unknown status"
    assert nv.lib().nvfp4_gemm_workspace_bytes(32768, 12352, 5120) == 0


A16 = 0x100000  # a fake, 16-byte aligned device address (never dereferenced)


def q(L, x=A16, rows=4, K=64, ldx=64, g=1.0, codes=A16, ldc=32, scales=A16, lds=16):
    return L.nvfp4_quantize(x, rows, K, ldx, g, codes, ldc, scales, lds, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scales=None), 1),
    (dict(K=24, ldx=32), 2), (dict(rows=-1), 2), (dict(ldx=56), 2), (dict(ldc=16), 2), (dict(lds=0), 2),
    (dict(x=A16 + 8), 3), (dict(ldx=68), 3), (dict(codes=A16 + 4), 3), (dict(ldc=40), 3), (dict(lds=24), 3),
    (dict(g=0.0), 5), (dict(g=-1.0), 5), (dict(g=float("inf")), 5), (dict(g=float("nan")), 5),
])
def test_quantize_rejects(L, kw, status):
    assert q(L, **kw) == status
    assert nv.last_error() != ""


def test_quantize_empty_is_ok_without_launch(L):
    assert q(L, rows=0) == 0
    assert q(L, K=0, ldx=0) == 0


def test_global_scale_rejects(L):
    assert L.nvfp4_global_scale(None, 4, 64, 64, A16, None) == 1
    assert L.nvfp4_global_scale(A16, 4, 64, 64, None, None) == 1
    assert L.nvfp4_global_scale(A16 + 2, 4, 64, 64, A16, None) == 3
    assert L.nvfp4_global_scale(A16, 4, 64, 60, A16, None) == 2
    assert L.nvfp4_global_scale(A16, 4, 64, 64, A16 + 2, None) == 3


def seg_array(specs):
    arr = (nv._Segment * max(1, len(specs)))()
    for i, s in enumerate(specs):
        arr[i] = nv._Segment(*s)
    return arr


def g(L, M=8, N=64, K=64, segs=None, g_w=None, n_segs=None, g_a=1.0, a_codes=A16, lda_c=32, a_scales=A16,
      lda_s=16, w_codes=A16, ldw_c=32, w_scales=A16, ldw_s=16, ws=None, ws_bytes=0):
    if segs is None:
        segs = [(0, N, 0, 0, A16, N, None, None)]
    n = len(segs) if n_segs is None else n_segs
    if g_w is None:
        g_w = [1.0] * max(1, len(segs))
    gw = (ctypes.c_float * max(1, len(g_w)))(*g_w)
    return L.nvfp4_gemm(a_codes, lda_c, a_scales, lda_s, g_a, w_codes, ldw_c, w_scales, ldw_s, M, N, K,
                        seg_array(segs), gw, n, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a_codes=None), 1), (dict(w_scales=None), 1),
    (dict(K=40), 2), (dict(M=-1), 2), (dict(lda_c=16), 2), (dict(ldw_s=0), 2),
    (dict(lda_c=1 << 23), 2), (dict(ldw_s=1 << 23), 2), (dict(M=300, ldw_c=1 << 23), 2),
    (dict(M=1 << 31, N=1 << 30), 2),  # 2^23 x 2^22 output tiles: more than the tiled grid takes
    (dict(a_codes=A16 + 1), 3), (dict(lda_c=40), 3), (dict(ldw_s=24), 3),
    (dict(n_segs=0), 4), (dict(n_segs=17), 4),
    (dict(segs=[(0, 32, 0, 0, A16, 32, None, None)]), 4),
    (dict(segs=[(0, 32, 0, 0, A16, 64, None, None), (16, 48, 0, 0, A16, 64, None, None)]), 4),
    (dict(segs=[(0, 32, 0, 0, A16, 64, None, None), (40, 24, 0, 0, A16, 64, None, None)]), 4),
    (dict(segs=[(0, 0, 0, 0, A16, 64, None, None), (0, 64, 0, 0, A16, 64, None, None)]), 4),
    (dict(g_a=0.0), 5), (dict(g_w=[float("nan")]), 5), (dict(g_w=[-2.0]), 5),
    # RN32(g_a * g_w) overflowing to inf, or underflowing to a subnormal or zero
    (dict(g_a=1e30, g_w=[1e30]), 5), (dict(g_a=1e-30, g_w=[1e-30]), 5), (dict(g_a=1e-20, g_w=[1e-20]), 5),
    (dict(segs=[(0, 64, 3, 0, A16, 64, None, None)]), 6),
    (dict(segs=[(0, 64, 0, 2, A16, 64, None, None)]), 6),
    (dict(segs=[(0, 64, 1, 1, A16, 64, None, None)]), 6),
    (dict(segs=[(0, 64, 2, 0, A16, 64, None, A16)]), 6),
    (dict(segs=[(0, 64, 0, 0, None, 64, None, None)]), 1),
    (dict(segs=[(0, 64, 0, 0, A16, 32, None, None)]), 2),
    (dict(segs=[(0, 64, 0, 0, A16 + 2, 64, None, None)]), 3),
])
def test_gemm_rejects(L, kw, status):
    assert g(L, **kw) == status, nv.last_error()
    assert nv.last_error() != ""


def wide_splits(K):
    """The split-K count of the decode kernel for 32 < M <= 64, as its header states: n = ceil(K / 256)
    chunks, s0 = min(8, max(1, n // 11)), chunks per split p = ceil(n / s0) rounded up to even, splits
    ceil(n / p); from K alone."""
    n = -(-K // 256)
    if n == 0:
        return 1
    s0 = min(8, max(1, n // 11))
    p = (-(-n // s0) + 1) // 2 * 2
    return -(-n // p)


def test_gemm_workspace_bytes(L):
    """Only the split-K decode kernel (32 < M <= 64, more than one split) keeps partial sums:
    splits * N * 64 FP32."""
    W = L.nvfp4_gemm_workspace_bytes
    assert [wide_splits(K) for K in (0, 16, 5120, 5632, 8320, 17408, 17520, 1 << 20)] == [1, 1, 1, 2, 3, 6, 6, 8]
    assert W(1, 5120, 17408) == W(32, 5120, 17408) == W(65, 5120, 17408) == 0
    assert W(33, 5120, 17408) == W(64, 5120, 17408) == 6 * 5120 * 64 * 4
    assert W(64, 17408, 5120) == W(48, 100, 16) == W(48, 100, 0) == 0
    assert W(40, 300, 8320) == 3 * 300 * 64 * 4
    assert W(64, 64, 40) == W(-1, 64, 64) == 0


WIDE = dict(M=40, K=5632, lda_c=2816, lda_s=352, ldw_c=2816, ldw_s=352)  # two K splits, N = 64


@pytest.mark.parametrize("kw,status", [
    (dict(WIDE), 7), (dict(WIDE, ws=A16, ws_bytes=2 * 64 * 64 * 4 - 1), 7),
    (dict(WIDE, ws=A16 + 4, ws_bytes=2 * 64 * 64 * 4), 3),
])
def test_gemm_wide_decode_workspace_rejects(L, kw, status):
    assert L.nvfp4_gemm_workspace_bytes(40, 64, 5632) == 2 * 64 * 64 * 4
    assert g(L, **kw) == status, nv.last_error()


def test_gemm_empty_shapes_ok_without_launch(L):
    assert g(L, M=0) == 0
    assert g(L, N=0, segs=[(0, 0, 0, 0, A16, 0, None, None)], n_segs=0) == 4  # still needs one segment


# --------------------------------------------------------------- serving-path companions
def kvq(L, x=A16, rows=4, cols=64, ldx=64, s=0.5, q=A16, ldq=64):
    return L.nvfp4_kv_quantize(x, rows, cols, ldx, s, q, ldq, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(q=None), 1),
    (dict(cols=56, ldx=64, ldq=64), 2), (dict(rows=-1), 2), (dict(ldx=56), 2), (dict(ldq=32), 2),
    (dict(x=A16 + 8), 3), (dict(ldx=68), 3), (dict(q=A16 + 8), 3), (dict(ldq=72), 3),
    (dict(s=0.0), 5), (dict(s=float("nan")), 5), (dict(s=float("inf")), 5),
])
def test_kv_quantize_rejects(L, kw, status):
    assert kvq(L, **kw) == status
    assert nv.last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(y=None), 1), (dict(cols=24, ldq=32, ldy=32), 2), (dict(y=A16 + 2), 3),
    (dict(q=A16 + 8), 3), (dict(s=-2.0), 5),
])
def test_kv_dequantize_rejects(L, kw, status):
    a = dict(q=A16, rows=4, cols=64, ldq=64, s=0.5, y=A16, ldy=64)
    a.update(kw)
    assert L.nvfp4_kv_dequantize(a["q"], a["rows"], a["cols"], a["ldq"], a["s"], a["y"], a["ldy"], None) == status


def test_kv_empty_and_scale_rejects(L):
    assert kvq(L, rows=0) == 0 and kvq(L, cols=0, ldx=0, ldq=0) == 0
    assert L.nvfp4_kv_scale(A16, 4, 64, 64, None, None) == 1
    assert L.nvfp4_kv_scale(A16, 4, 64, 64, A16 + 2, None) == 3


def test_fold_rejects(L):
    assert L.nvfp4_fold_scales(None, 4, 8, 16, 0.5, None) == 1
    assert L.nvfp4_fold_scales(A16, 4, 8, 4, 0.5, None) == 2
    assert L.nvfp4_fold_scales(A16, 4, 8, 16, 0.0, None) == 5
    assert L.nvfp4_fold_scales(A16, 0, 8, 16, 0.5, None) == 0
    rows = (ctypes.c_int64 * 2)(4, 4)
    gw = (ctypes.c_float * 2)(0.5, 1.0)
    G = ctypes.c_float(0)
    assert L.nvfp4_fold_group(A16, 16, 64, rows, gw, 0, ctypes.byref(G), None) == 4
    assert L.nvfp4_fold_group(A16, 16, 60, rows, gw, 2, ctypes.byref(G), None) == 2
    bad = (ctypes.c_float * 2)(0.5, float("nan"))
    assert L.nvfp4_fold_group(A16, 16, 64, rows, bad, 2, ctypes.byref(G), None) == 5
    assert L.nvfp4_fold_group(A16, 16, 64, rows, gw, 2, None, None) == 1
    # a ratio g_w[s] / max g_w that underflows to 0 is rejected before anything is written: g_common
    # keeps its value (and no fold of an earlier segment is enqueued; the scale pointer is fake here)
    G.value = -7.0
    tiny = (ctypes.c_float * 2)(3e38, 1e-45)  # the second segment's ratio underflows
    assert L.nvfp4_fold_group(A16, 16, 64, rows, tiny, 2, ctypes.byref(G), None) == 5
    assert G.value == -7.0
    assert L.nvfp4_fold_group(None, 16, 64, rows, gw, 2, ctypes.byref(G), None) == 1
    assert L.nvfp4_fold_group(A16, 2, 64, rows, gw, 2, ctypes.byref(G), None) == 2
    assert G.value == -7.0


def rq(L, x=A16, rows=4, K=64, ldx=64, w=A16, eps=1e-6, g=1.0, codes=A16, ldc=32, scales=A16, lds=16, y=None,
       ldy=0):
    return L.nvfp4_rmsnorm_quantize(x, rows, K, ldx, w, eps, g, codes, ldc, scales, lds, y, ldy, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(codes=None), 1),
    (dict(K=24, ldx=32), 2), (dict(y=A16, ldy=32), 2),
    (dict(w=A16 + 2), 3), (dict(x=A16 + 8), 3), (dict(y=A16 + 8, ldy=64), 3),
    (dict(g=0.0), 5), (dict(eps=-1.0), 5), (dict(eps=float("nan")), 5),
])
def test_rmsnorm_quantize_rejects(L, kw, status):
    assert rq(L, **kw) == status


def gdn(L, q=A16, ldq=2048, k=A16, ldk=2048, v=A16, ldv=4096, a=A16, lda=32, b=A16, ldb=32, state=A16, B=1, T=64,
        Hv=32, Hk=16, D=128, o=A16, ldo=4096, ws=A16, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.nvfp4_gdn_workspace_bytes(B, T, Hv, Hk, D)
    return L.nvfp4_gdn_recurrence(q, ldq, k, ldk, v, ldv, a, lda, b, ldb, state, B, T, Hv, Hk, D, o, ldo, ws,
                                  ws_bytes, None)


def test_gdn_workspace_bytes(L):
    """The chunked form (32 tokens or more) keeps 21504 bytes of chunk factors per (sequence, value
    head, 64-token chunk); token-by-token calls and invalid shapes need none."""
    W = L.nvfp4_gdn_workspace_bytes
    assert W(1, 32768, 32, 16, 128) == 512 * 32 * 21504
    assert W(2, 33, 4, 2, 128) == 2 * 4 * 1 * 21504 and W(2, 65, 4, 2, 128) == 2 * 4 * 2 * 21504
    assert W(64, 1, 32, 16, 128) == 0 and W(3, 31, 4, 2, 128) == 0
    assert W(1, 64, 32, 16, 64) == 0 and W(1, 64, 30, 16, 128) == 0 and W(0, 64, 4, 2, 128) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(state=None), 1), (dict(o=None), 1),
    (dict(D=64), 2), (dict(Hv=30), 2), (dict(T=-1), 2), (dict(ldv=4000), 2), (dict(lda=16), 2),
    (dict(ldv=1 << 23), 2), (dict(ldo=1 << 23), 2),
    (dict(q=A16 + 8), 3), (dict(ldk=2052), 3), (dict(state=A16 + 4), 3), (dict(ws=A16 + 8), 3),
    (dict(ws_bytes=1024), 7), (dict(ws=None), 7),
])
def test_gdn_rejects(L, kw, status):
    assert gdn(L, **kw) == status
    assert nv.last_error() != ""


def test_gdn_empty_and_token_by_token_need_no_workspace(L):
    assert gdn(L, B=0, ws=None, ws_bytes=0) == 0
    assert gdn(L, T=0, ws=None, ws_bytes=0) == 0


def test_gemm_noalloc_rejects_before_any_launch(L):
    """The allocation-free entry point validates like nvfp4_gemm and rejects shapes needing more than
    its fixed per-GPU scratch (NVFP4_ERR_WORKSPACE) before touching the device."""
    def call(M, N, K, lda_c, lda_s):
        segs = seg_array([(0, N, 0, 0, A16, N, None, None)])
        gw = (ctypes.c_float * 1)(1.0)
        return L.nvfp4_gemm_noalloc(A16, lda_c, A16, lda_s, 1.0, A16, lda_c, A16, lda_s, M, N, K, segs, gw, 1, None)
    assert L.nvfp4_gemm_workspace_bytes(64, 100000, 17408) > nv.NOALLOC_SCRATCH_BYTES
    assert call(64, 100000, 17408, 8704, 1088) == 7
    assert "scratch" in nv.last_error()
    assert call(8, 64, 40, 32, 16) == 2
    assert call(0, 64, 64, 32, 16) == 0


def test_packed_weight_bytes(L):
    """The decode layout holds 2304 bytes per 16-row tile and 256-element chunk."""
    W = L.nvfp4_packed_weight_bytes
    assert W(16, 256) == 2304 and W(17, 256) == W(16, 272) == 2 * 2304
    assert W(17408, 5120) == 1088 * 20 * 2304 and W(5120, 17408) == 320 * 68 * 2304
    assert W(0, 256) == W(16, 0) == W(16, 24) == W(-1, 16) == 0


def pack(L, w_codes=A16, ldw_c=32, w_scales=A16, ldw_s=16, N=20, K=64, packed=A16):
    return L.nvfp4_pack_weights(w_codes, ldw_c, w_scales, ldw_s, N, K, packed, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w_codes=None), 1), (dict(w_scales=None), 1), (dict(packed=None), 1),
    (dict(K=24), 2), (dict(N=-1), 2), (dict(ldw_c=16), 2),
    (dict(packed=A16 + 4), 3), (dict(w_codes=A16 + 8), 3), (dict(ldw_s=20), 3),
])
def test_pack_weights_rejects(L, kw, status):
    assert pack(L, **kw) == status
    assert nv.last_error() != ""


def test_pack_weights_empty_is_a_no_op(L):
    assert pack(L, N=0, packed=None) == 0
    assert pack(L, K=0, packed=None) == 0


def gp(L, M=8, N=64, K=64, packed=A16, segs=None, g_a=1.0):
    if segs is None:
        segs = [(0, N, 0, 0, A16, N, None, None)]
    gw = (ctypes.c_float * len(segs))(*([1.0] * len(segs)))
    return L.nvfp4_gemm_packed(A16, 32, A16, 16, g_a, packed, M, N, K, seg_array(segs), gw, len(segs), None, 0,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=65), 2), (dict(M=4096), 2), (dict(K=24), 2), (dict(packed=None), 1), (dict(packed=A16 + 4), 3),
    (dict(segs=[(0, 32, 0, 0, A16, 32, None, None)]), 4), (dict(g_a=0.0), 5),
])
def test_gemm_packed_rejects(L, kw, status):
    assert gp(L, **kw) == status
    assert nv.last_error() != ""


def test_gemm_packed_empty_is_a_no_op(L):
    assert gp(L, M=0) == 0
    assert gp(L, N=0, segs=[]) != 0  # an empty segment table is rejected as for nvfp4_gemm
