"""Python binding of libnvfp4.so, the MI355X (gfx950) NVFP4 W4A4 quantized-linear library.

Argument marshalling only: every step of the path runs in the library's HIP kernels. PyTorch is
used for device memory and the current stream. The names mirror the C interface in
include/nvfp4.h (nvfp4_global_scale, nvfp4_quantize, nvfp4_gemm, and the serving-path companions
nvfp4_kv_scale / nvfp4_kv_quantize / nvfp4_kv_dequantize, nvfp4_fold_scales / nvfp4_fold_group,
nvfp4_rmsnorm_quantize, nvfp4_gdn_recurrence).

If the library has not been built (``python -m nvfp4_w4a4_quantized_quantize_amd.build``), or was
built from sources other than the ones in the tree, every call raises: there is no fallback
implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# NVFP4_LIB names another build of the same sources (the host-sanitizer run uses it).
LIB_PATH = os.environ.get("NVFP4_LIB") or os.path.join(_PKG, "libnvfp4.so")

OK = 0
OUT_F32, OUT_BF16 = 0, 1
EPI_NONE, EPI_SIGMOID, EPI_GDN_DECAY = 0, 1, 2
MAX_SEGMENTS = 16
_EPI = {"none": EPI_NONE, "sigmoid": EPI_SIGMOID, "gdn_decay": EPI_GDN_DECAY}

# Every function the C header declares; a test checks the library exports all of them.
EXPORTED = ("nvfp4_global_scale", "nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_workspace_bytes",
            "nvfp4_status_string", "nvfp4_last_error", "nvfp4_kv_scale", "nvfp4_kv_quantize",
            "nvfp4_kv_dequantize", "nvfp4_fold_scales", "nvfp4_fold_group", "nvfp4_rmsnorm_quantize",
            "nvfp4_gdn_recurrence", "nvfp4_gdn_workspace_bytes", "nvfp4_gemm_noalloc",
            "nvfp4_packed_weight_bytes", "nvfp4_pack_weights", "nvfp4_gemm_packed")
NOALLOC_SCRATCH_BYTES = 16 << 20


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")
        self.status = status


class _Segment(ctypes.Structure):
    _fields_ = [("n_begin", ctypes.c_int64), ("n_len", ctypes.c_int64), ("epilogue", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so (raises if it is missing: the path has no fallback)."""
    global _lib
    if _lib is None:
        from . import build as _build
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m nvfp4_w4a4_quantized_quantize_amd.build")
        if not _build.built_from_current_sources(LIB_PATH, _build.sources()):
            raise ImportError(f"{LIB_PATH} was built from other sources than the ones in the tree; rebuild it "
                              "with python -m nvfp4_w4a4_quantized_quantize_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, f32, P = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        L.nvfp4_global_scale.restype = i32
        L.nvfp4_global_scale.argtypes = [P, i64, i64, i64, P, P]
        L.nvfp4_quantize.restype = i32
        L.nvfp4_quantize.argtypes = [P, i64, i64, i64, f32, P, i64, P, i64, P]
        L.nvfp4_gemm.restype = i32
        L.nvfp4_gemm.argtypes = [P, i64, P, i64, f32, P, i64, P, i64, i64, i64, i64,
                                 ctypes.POINTER(_Segment), ctypes.POINTER(f32), i32, P, ctypes.c_size_t, P]
        L.nvfp4_gemm_noalloc.restype = i32
        L.nvfp4_gemm_noalloc.argtypes = [P, i64, P, i64, f32, P, i64, P, i64, i64, i64, i64,
                                         ctypes.POINTER(_Segment), ctypes.POINTER(f32), i32, P]
        L.nvfp4_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.nvfp4_packed_weight_bytes.restype = ctypes.c_size_t
        L.nvfp4_packed_weight_bytes.argtypes = [i64, i64]
        L.nvfp4_pack_weights.restype = i32
        L.nvfp4_pack_weights.argtypes = [P, i64, P, i64, i64, i64, P, P]
        L.nvfp4_gemm_packed.restype = i32
        L.nvfp4_gemm_packed.argtypes = [P, i64, P, i64, f32, P, i64, i64, i64,
                                        ctypes.POINTER(_Segment), ctypes.POINTER(f32), i32, P, ctypes.c_size_t, P]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_last_error.restype = ctypes.c_char_p
        L.nvfp4_last_error.argtypes = []
        L.nvfp4_kv_scale.restype = i32
        L.nvfp4_kv_scale.argtypes = [P, i64, i64, i64, P, P]
        L.nvfp4_kv_quantize.restype = i32
        L.nvfp4_kv_quantize.argtypes = [P, i64, i64, i64, f32, P, i64, P]
        L.nvfp4_kv_dequantize.restype = i32
        L.nvfp4_kv_dequantize.argtypes = [P, i64, i64, i64, f32, P, i64, P]
        L.nvfp4_fold_scales.restype = i32
        L.nvfp4_fold_scales.argtypes = [P, i64, i64, i64, f32, P]
        L.nvfp4_fold_group.restype = i32
        L.nvfp4_fold_group.argtypes = [P, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(f32), i32,
                                       ctypes.POINTER(f32), P]
        L.nvfp4_rmsnorm_quantize.restype = i32
        L.nvfp4_rmsnorm_quantize.argtypes = [P, i64, i64, i64, P, f32, f32, P, i64, P, i64, P, i64, P]
        L.nvfp4_gdn_recurrence.restype = i32
        L.nvfp4_gdn_recurrence.argtypes = [P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, i64, i32, i32, i32, P, i64,
                                           P, ctypes.c_size_t, P]
        L.nvfp4_gdn_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_gdn_workspace_bytes.argtypes = [i64, i64, i32, i32, i32]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def last_error() -> str:
    return lib().nvfp4_last_error().decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Nvfp4Error(status, where, last_error())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _round16(n: int) -> int:
    return (n + 15) // 16 * 16


def _ld(t: torch.Tensor, multiple: int) -> int:
    """Row stride in elements; a single-row tensor may carry any stride, so report a valid one."""
    if t.shape[0] > 1:
        return t.stride(0)
    return (t.shape[1] + multiple - 1) // multiple * multiple


def alloc_nvfp4(rows: int, K: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Codes [rows, K/2] and scales [rows, K/16] uint8 views with 16-byte-multiple row strides."""
    cb = torch.empty((rows, _round16(K // 2)), dtype=torch.uint8, device=device)
    sb = torch.empty((rows, _round16(K // 16)), dtype=torch.uint8, device=device)
    return cb[:, :K // 2], sb[:, :K // 16]


# --------------------------------------------------------------------------------------- a1: scale
def global_scale(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """g = RN32(max|x| / 2688) of a bf16 [rows, K] device tensor, as a float32 device tensor [1]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().nvfp4_global_scale(_ptr(x), x.shape[0], x.shape[1], _ld(x, 8), _ptr(out), _stream(stream)),
           "nvfp4_global_scale")
    return out


# ------------------------------------------------------------------------------------ a2-a4: quantize
def quantize(x: torch.Tensor, g: float, codes: Optional[torch.Tensor] = None,
             scales: Optional[torch.Tensor] = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """NVFP4-quantize a bf16 [rows, K] device tensor with FP32 global scale g.

    Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/16]) (preallocated ones may be passed).
    """
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    if codes is None or scales is None:
        codes, scales = alloc_nvfp4(rows, K, x.device)
    _check(lib().nvfp4_quantize(_ptr(x), rows, K, _ld(x, 8), float(g), _ptr(codes), _ld(codes, 16),
                                _ptr(scales), _ld(scales, 16), _stream(stream)), "nvfp4_quantize")
    return codes, scales


# ------------------------------------------------------------------------------------- a5-a7: GEMM
@dataclasses.dataclass
class Segment:
    """One output-column segment (one separately calibrated module) of a fused GEMM."""
    n: int
    g_w: float
    epilogue: str = "none"                 # "none", "sigmoid" or "gdn_decay"
    out_dtype: torch.dtype = torch.float32  # torch.float32 or torch.bfloat16
    A_log: Optional[torch.Tensor] = None    # float32 [n] device (gdn_decay)
    dt_bias: Optional[torch.Tensor] = None  # float32 [n] device (gdn_decay)
    out: Optional[torch.Tensor] = None      # preallocated [M, n] output (optional)


def _segments(a_codes: torch.Tensor, M: int, N: int, segments: Sequence[Segment]):
    assert sum(s.n for s in segments) == N, "segments must cover N"
    n_segs = len(segments)
    segs = (_Segment * max(n_segs, 1))()
    g_w = (ctypes.c_float * max(n_segs, 1))()
    outs = []
    begin = 0
    for i, s in enumerate(segments):
        dt = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[s.out_dtype]
        out = s.out if s.out is not None else torch.empty((M, s.n), dtype=s.out_dtype, device=a_codes.device)
        assert out.dtype == s.out_dtype and out.dim() == 2 and out.stride(1) == 1
        segs[i] = _Segment(begin, s.n, _EPI[s.epilogue], dt, _ptr(out), _ld(out, 1),
                           _ptr(s.A_log), _ptr(s.dt_bias))
        g_w[i] = float(s.g_w)
        outs.append(out)
        begin += s.n
    return segs, g_w, n_segs, outs


def gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, g_a: float, w_codes: torch.Tensor,
         w_scales: torch.Tensor, segments: Sequence[Segment], workspace: Optional[torch.Tensor] = None,
         stream=None) -> list[torch.Tensor]:
    """Block-scaled W4A4 GEMM Y = A W^T with one global scale per output segment.

    a_codes [M, K/2], a_scales [M, K/16]; w_codes [N, K/2], w_scales [N, K/16] (uint8, device).
    Returns one output tensor [M, n_s] per segment.
    """
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == K and a_scales.shape == (M, K // 16) and w_scales.shape == (N, K // 16)
    segs, g_w, n_segs, outs = _segments(a_codes, M, N, segments)
    need = lib().nvfp4_gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a_codes.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvfp4_gemm(_ptr(a_codes), _ld(a_codes, 16), _ptr(a_scales), _ld(a_scales, 16), float(g_a),
                            _ptr(w_codes), _ld(w_codes, 16), _ptr(w_scales), _ld(w_scales, 16), M, N, K,
                            segs, g_w, n_segs, _ptr(workspace), ws_bytes, _stream(stream)), "nvfp4_gemm")
    return outs


def pack_weights(w_codes: torch.Tensor, w_scales: torch.Tensor, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """The decode layout of NVFP4 weights (codes [N, K/2], scales [N, K/16]) for gemm_packed: a uint8
    device tensor of nvfp4_packed_weight_bytes(N, K) bytes (a preallocated one may be passed)."""
    N, K = w_codes.shape[0], w_codes.shape[1] * 2
    assert w_scales.shape == (N, K // 16)
    need = lib().nvfp4_packed_weight_bytes(N, K)
    if out is None:
        out = torch.empty(max(need, 16), dtype=torch.uint8, device=w_codes.device)
    assert out.numel() * out.element_size() >= need
    _check(lib().nvfp4_pack_weights(_ptr(w_codes), _ld(w_codes, 16), _ptr(w_scales), _ld(w_scales, 16), N, K,
                                    _ptr(out), _stream(stream)), "nvfp4_pack_weights")
    return out


def gemm_packed(a_codes: torch.Tensor, a_scales: torch.Tensor, g_a: float, w_packed: torch.Tensor, N: int,
                segments: Sequence[Segment], workspace: Optional[torch.Tensor] = None,
                stream=None) -> list[torch.Tensor]:
    """gemm() for M <= 64 activation rows with weights in the decode layout (pack_weights of the N x K
    weights, K from the activations). Returns one output tensor [M, n_s] per segment."""
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    assert a_scales.shape == (M, K // 16)
    assert w_packed.numel() * w_packed.element_size() >= lib().nvfp4_packed_weight_bytes(N, K)
    segs, g_w, n_segs, outs = _segments(a_codes, M, N, segments)
    need = lib().nvfp4_gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=a_codes.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvfp4_gemm_packed(_ptr(a_codes), _ld(a_codes, 16), _ptr(a_scales), _ld(a_scales, 16), float(g_a),
                                   _ptr(w_packed), M, N, K, segs, g_w, n_segs, _ptr(workspace), ws_bytes,
                                   _stream(stream)), "nvfp4_gemm_packed")
    return outs


def gemm_noalloc(a_codes: torch.Tensor, a_scales: torch.Tensor, g_a: float, w_codes: torch.Tensor,
                 w_scales: torch.Tensor, segments: Sequence[Segment], stream=None) -> list[torch.Tensor]:
    """gemm() through nvfp4_gemm_noalloc: the library allocates nothing (its partial sums use a fixed
    per-GPU scratch array). Outputs are allocated here unless every segment brings its own `out`."""
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == K and a_scales.shape == (M, K // 16) and w_scales.shape == (N, K // 16)
    segs, g_w, n_segs, outs = _segments(a_codes, M, N, segments)
    _check(lib().nvfp4_gemm_noalloc(_ptr(a_codes), _ld(a_codes, 16), _ptr(a_scales), _ld(a_scales, 16), float(g_a),
                                    _ptr(w_codes), _ld(w_codes, 16), _ptr(w_scales), _ld(w_scales, 16), M, N, K,
                                    segs, g_w, n_segs, _stream(stream)), "nvfp4_gemm_noalloc")
    return outs


# ------------------------------------------------------------------------ FP8 E4M3 KV-cache codec
def kv_scale(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Static KV scale s = RN32(max|x| / 448) of a bf16 [rows, cols] calibration tensor (float32 [1])."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().nvfp4_kv_scale(_ptr(x), x.shape[0], x.shape[1], _ld(x, 8), _ptr(out), _stream(stream)),
           "nvfp4_kv_scale")
    return out


def kv_quantize(x: torch.Tensor, s: float, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q = E4M3_RNE_SAT(RN32(x / s)) of a bf16 [rows, cols] tensor, as uint8 [rows, cols]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_kv_quantize(_ptr(x), x.shape[0], x.shape[1], _ld(x, 8), float(s), _ptr(out), _ld(out, 16),
                                   _stream(stream)), "nvfp4_kv_quantize")
    return out


def kv_dequantize(q: torch.Tensor, s: float, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = bf16_RNE(RN32(e4m3(q) * s)) of uint8 E4M3 codes [rows, cols], as bf16 [rows, cols]."""
    assert q.dtype == torch.uint8 and q.dim() == 2 and q.stride(1) == 1
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _check(lib().nvfp4_kv_dequantize(_ptr(q), q.shape[0], q.shape[1], _ld(q, 16), float(s), _ptr(out), _ld(out, 8),
                                     _stream(stream)), "nvfp4_kv_dequantize")
    return out


# ----------------------------------------------------------------------------- fold-in repair
def fold_scales(scales: torch.Tensor, ratio: float, stream=None) -> torch.Tensor:
    """In place: s' = E4M3_RNE_SAT(RN32(s * ratio)) over uint8 E4M3 scales [rows, nblocks]."""
    assert scales.dtype == torch.uint8 and scales.dim() == 2 and scales.stride(1) == 1
    _check(lib().nvfp4_fold_scales(_ptr(scales), scales.shape[0], scales.shape[1], _ld(scales, 1), float(ratio),
                                   _stream(stream)), "nvfp4_fold_scales")
    return scales


def fold_group(w_scales: torch.Tensor, seg_rows: Sequence[int], g_w: Sequence[float], stream=None) -> float:
    """In place fold-in repair of a fused weight's scales [N, K/16]; returns the common scale G."""
    assert w_scales.dtype == torch.uint8 and w_scales.dim() == 2 and w_scales.stride(1) == 1
    n = len(seg_rows)
    rows = (ctypes.c_int64 * max(n, 1))(*seg_rows)
    gs = (ctypes.c_float * max(n, 1))(*[float(g) for g in g_w])
    G = ctypes.c_float(0.0)
    _check(lib().nvfp4_fold_group(_ptr(w_scales), _ld(w_scales, 16), w_scales.shape[1] * 16, rows, gs, n,
                                  ctypes.byref(G), _stream(stream)), "nvfp4_fold_group")
    return G.value


# ----------------------------------------------------------------------- RMSNorm + quantize
def rmsnorm_quantize(x: torch.Tensor, w: torch.Tensor, eps: float, g: float, codes: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None, stream=None):
    """BF16 RMSNorm of x [rows, K] with weight w [K], quantized to NVFP4 with global scale g.

    Returns (codes, scales); when y (bf16 [rows, K]) is given it also receives the normalized rows.
    """
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert w.dtype == torch.bfloat16 and w.dim() == 1 and w.stride(0) == 1 and w.shape[0] == x.shape[1]
    rows, K = x.shape
    if codes is None or scales is None:
        codes, scales = alloc_nvfp4(rows, K, x.device)
    ldy = 0
    if y is not None:
        assert y.dtype == torch.bfloat16 and y.shape == x.shape and y.stride(1) == 1
        ldy = _ld(y, 8)
    _check(lib().nvfp4_rmsnorm_quantize(_ptr(x), rows, K, _ld(x, 8), _ptr(w), float(eps), float(g), _ptr(codes),
                                        _ld(codes, 16), _ptr(scales), _ld(scales, 16), _ptr(y), ldy,
                                        _stream(stream)), "nvfp4_rmsnorm_quantize")
    return codes, scales


# ----------------------------------------------------------------- Gated DeltaNet recurrence
def gdn_recurrence(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                   state: torch.Tensor, B: int, T: int, o: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T, o_t = S_t^T q_t over B sequences of T tokens.

    q, k: bf16 [B*T, Hk*128]; v: bf16 [B*T, Hv*128]; alpha, beta: float32 [B*T, Hv]; state: float32
    [B, Hv, 128, 128] holding each head's S value-major (state[b, h] = S^T), updated in place.
    Returns o float32 [B*T, Hv*128].
    """
    D = 128
    for t in (q, k, v):
        assert t.dtype == torch.bfloat16 and t.dim() == 2 and t.stride(1) == 1 and t.shape[0] == B * T
    for t in (alpha, beta):
        assert t.dtype == torch.float32 and t.dim() == 2 and t.stride(1) == 1 and t.shape[0] == B * T
    Hk, Hv = q.shape[1] // D, v.shape[1] // D
    assert state.dtype == torch.float32 and state.is_contiguous() and tuple(state.shape) == (B, Hv, D, D)
    if o is None:
        o = torch.empty((B * T, Hv * D), dtype=torch.float32, device=q.device)
    need = lib().nvfp4_gdn_workspace_bytes(B, T, Hv, Hk, D)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvfp4_gdn_recurrence(_ptr(q), _ld(q, 8), _ptr(k), _ld(k, 8), _ptr(v), _ld(v, 1), _ptr(alpha),
                                      _ld(alpha, 1), _ptr(beta), _ld(beta, 1), _ptr(state), B, T, Hv, Hk, D,
                                      _ptr(o), _ld(o, 1), _ptr(workspace), ws_bytes, _stream(stream)),
           "nvfp4_gdn_recurrence")
    return o
