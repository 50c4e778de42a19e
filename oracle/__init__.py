"""NVFP4 W4A4 reference oracle -- test infrastructure, not part of the product.

Python access (ctypes + numpy) to the plain C oracle in ``nvfp4_oracle.c``. Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package; the HIP
library never does, and this package imports nothing from it.

What is computed, and the passages each function follows, is documented in ``nvfp4_oracle.c``.
Every function here is argument marshalling only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
# NVFP4_ORACLE_LIB names another build of the same source (the host-sanitizer run uses it).
_LIB = os.environ.get("NVFP4_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, so each binary32 step rounds once, as the spec states.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.environ.get("NVFP4_ORACLE_LIB") and (not os.path.exists(_LIB) or
                                                        os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB)
        i64, f32, f64, i32 = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_int
        P = ctypes.c_void_p
        L.oracle_e2m1_value.restype = f64
        L.oracle_e2m1_value.argtypes = [i32]
        L.oracle_e4m3_value.restype = f64
        L.oracle_e4m3_value.argtypes = [i32]
        L.oracle_e4m3_from_float.restype = i32
        L.oracle_e4m3_from_float.argtypes = [f32]
        L.oracle_e2m1_from_float.restype = i32
        L.oracle_e2m1_from_float.argtypes = [f32]
        L.oracle_tensor_amax.restype = f32
        L.oracle_tensor_amax.argtypes = [P, i64, i64, i64]
        L.oracle_global_scale.restype = f32
        L.oracle_global_scale.argtypes = [f32]
        L.oracle_quantize.restype = i32
        L.oracle_quantize.argtypes = [P, i64, i64, i64, f32, P, i64, P, i64]
        L.oracle_dequantize.restype = None
        L.oracle_dequantize.argtypes = [P, i64, P, i64, i64, i64, f32, P]
        L.oracle_gemm_rows.restype = i32
        L.oracle_gemm_rows.argtypes = [P, P, i64, i64, f32, P, P, i64, i64, i64, i64, P, P, i32, P,
                                       i64, P, P]
        L.oracle_sigmoid.restype = f64
        L.oracle_sigmoid.argtypes = [f64]
        L.oracle_softplus.restype = f64
        L.oracle_softplus.argtypes = [f64]
        L.oracle_gdn_decay.restype = f64
        L.oracle_gdn_decay.argtypes = [f64, f64, f64]
        L.oracle_sigmoid_array.restype = None
        L.oracle_sigmoid_array.argtypes = [P, i64, P]
        L.oracle_gdn_decay_array.restype = None
        L.oracle_gdn_decay_array.argtypes = [P, i64, i64, P, P, P]
        L.oracle_e4m3_from_float_array.restype = None
        L.oracle_e4m3_from_float_array.argtypes = [P, i64, P]
        L.oracle_num_threads.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_e2m1_from_float_array.restype = None
        L.oracle_e2m1_from_float_array.argtypes = [P, i64, P]
        L.oracle_kv_scale.restype = f32
        L.oracle_kv_scale.argtypes = [f32]
        L.oracle_kv_quantize.restype = None
        L.oracle_kv_quantize.argtypes = [P, i64, i64, i64, f32, P, i64]
        L.oracle_kv_dequantize.restype = None
        L.oracle_kv_dequantize.argtypes = [P, i64, i64, i64, f32, P, i64]
        L.oracle_fold_common_scale.restype = f32
        L.oracle_fold_common_scale.argtypes = [P, i32]
        L.oracle_fold_ratio.restype = f32
        L.oracle_fold_ratio.argtypes = [f32, f32]
        L.oracle_fold_scales.restype = None
        L.oracle_fold_scales.argtypes = [P, i64, i64, i64, f32]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [P, i64, i64, i64, P, f32, P, i64, P]
        L.oracle_gdn_recurrence.restype = None
        L.oracle_gdn_recurrence.argtypes = [P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, i64, i64, i64, i64, P, P]
        L.oracle_gdn_recurrence_f32.restype = None
        L.oracle_gdn_recurrence_f32.argtypes = [P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, i64, i64, i64, i64,
                                                P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def set_num_threads(n: int) -> None:
    """Threads for later OpenMP row loops (the CPU-baseline timing also runs the oracle on one)."""
    lib().oracle_set_num_threads(int(n))


def num_threads() -> int:
    """Threads the oracle's OpenMP row loops use."""
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------- format helpers
def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().oracle_e4m3_value(int(byte))


def e4m3_from_float(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().oracle_e4m3_from_float_array(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_from_float(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().oracle_e2m1_from_float_array(_ptr(v), v.size, _ptr(out))
    return out


# ---------------------------------------------------------------- global scale
def tensor_amax(x_bf16: np.ndarray) -> float:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 2
    return float(lib().oracle_tensor_amax(_ptr(x), x.shape[0], x.shape[1], x.shape[1]))


def global_scale(x_bf16: np.ndarray) -> np.float32:
    """g = RN32(amax / 2688) for a bf16 tensor given as uint16 bit patterns."""
    return np.float32(lib().oracle_global_scale(np.float32(tensor_amax(x_bf16))))


# ---------------------------------------------------------------- quantizer
def quantize(x_bf16: np.ndarray, g) -> tuple[np.ndarray, np.ndarray]:
    """bf16 [R, K] (uint16 bit patterns) -> (codes uint8 [R, K/2], scales uint8 [R, K/16])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 2 and x.shape[1] % 16 == 0
    R, K = x.shape
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, K // 16), dtype=np.uint8)
    rc = lib().oracle_quantize(_ptr(x), R, K, K, np.float32(g), _ptr(codes), K // 2, _ptr(scales),
                               K // 16)
    assert rc == 0
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """Exact decode x_hat = e2m1(code) * e4m3(scale) * g, in float64 [R, K]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = c.shape[0], c.shape[1] * 2
    out = np.empty((R, K), dtype=np.float64)
    lib().oracle_dequantize(_ptr(c), c.shape[1], _ptr(s), s.shape[1], R, K, np.float32(g), _ptr(out))
    return out


# ---------------------------------------------------------------- GEMM + gates
def gemm_rows(a_codes, a_scales, g_a, w_codes, w_scales, seg_bounds, g_w, rows):
    """Exact y[i, n] and tolerance scale T[i, n] for A rows ``rows`` against all N columns.

    seg_bounds: ascending column boundaries [0, b1, ..., N]; g_w: one FP32 scale per segment.
    Returns (y float64 [len(rows), N], T float64 [len(rows), N]).
    """
    ac = np.ascontiguousarray(a_codes, dtype=np.uint8)
    asc = np.ascontiguousarray(a_scales, dtype=np.uint8)
    wc = np.ascontiguousarray(w_codes, dtype=np.uint8)
    wsc = np.ascontiguousarray(w_scales, dtype=np.uint8)
    K = ac.shape[1] * 2
    N = wc.shape[0]
    assert wc.shape[1] * 2 == K
    sb = np.ascontiguousarray(seg_bounds, dtype=np.int64)
    gw = np.ascontiguousarray(g_w, dtype=np.float32)
    assert sb[0] == 0 and sb[-1] == N and gw.size == sb.size - 1
    r = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((r.size, N), dtype=np.float64)
    T = np.empty((r.size, N), dtype=np.float64)
    rc = lib().oracle_gemm_rows(_ptr(ac), _ptr(asc), ac.shape[1], asc.shape[1], np.float32(g_a),
                                _ptr(wc), _ptr(wsc), wc.shape[1], wsc.shape[1], N, K, _ptr(sb),
                                _ptr(gw), gw.size, _ptr(r), r.size, _ptr(y), _ptr(T))
    assert rc == 0, rc
    return y, T


def sigmoid(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty_like(y)
    lib().oracle_sigmoid_array(_ptr(y), y.size, _ptr(out))
    return out


def gdn_decay(y: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """alpha = exp(-exp(A_log[j]) * softplus(y[:, j] + dt_bias[j])) for y [rows, ncols]."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    assert y.ndim == 2
    al = np.ascontiguousarray(a_log, dtype=np.float32)
    dt = np.ascontiguousarray(dt_bias, dtype=np.float32)
    assert al.size == y.shape[1] and dt.size == y.shape[1]
    out = np.empty_like(y)
    lib().oracle_gdn_decay_array(_ptr(y), y.shape[0], y.shape[1], _ptr(al), _ptr(dt), _ptr(out))
    return out


def softplus(z: float) -> float:
    return lib().oracle_softplus(float(z))


def gdn_decay_scalar(y: float, a_log: float, dt_bias: float) -> float:
    return lib().oracle_gdn_decay(float(y), float(a_log), float(dt_bias))


def sigmoid_scalar(y: float) -> float:
    return lib().oracle_sigmoid(float(y))


# ---------------------------------------------------------------- serving-path companions
def kv_scale(x_bf16: np.ndarray) -> np.float32:
    """Static FP8 KV scale of a calibration tensor: RN32(amax / 448)."""
    return np.float32(lib().oracle_kv_scale(tensor_amax(x_bf16)))


def kv_quantize(x_bf16: np.ndarray, s) -> np.ndarray:
    """bf16 bits [rows, cols] -> E4M3 bytes, q = E4M3_RNE_SAT(RN32(x / s))."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    lib().oracle_kv_quantize(_ptr(x), rows, cols, cols, float(np.float32(s)), _ptr(q), cols)
    return q


def kv_dequantize(q: np.ndarray, s) -> np.ndarray:
    """E4M3 bytes -> bf16 bits, y = bf16_RNE(RN32(e4m3(q) * s))."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows, cols = q.shape
    y = np.empty((rows, cols), np.uint16)
    lib().oracle_kv_dequantize(_ptr(q), rows, cols, cols, float(np.float32(s)), _ptr(y), cols)
    return y


def fold_common_scale(g) -> np.float32:
    g = np.ascontiguousarray(g, dtype=np.float32)
    return np.float32(lib().oracle_fold_common_scale(_ptr(g), len(g)))


def fold_ratio(g, G) -> np.float32:
    return np.float32(lib().oracle_fold_ratio(float(np.float32(g)), float(np.float32(G))))


def fold_scales(scales: np.ndarray, ratio) -> np.ndarray:
    """Returns a copy of the [rows, nblocks] scale bytes with the ratio folded in."""
    out = np.array(scales, dtype=np.uint8, copy=True, order="C")
    rows, nb = out.shape
    lib().oracle_fold_scales(_ptr(out), rows, nb, nb, float(np.float32(ratio)))
    return out


def fold_group(scales_per_module, g_per_module):
    """The fold-in repair of a fused group: (G, [folded scales per module])."""
    G = fold_common_scale(g_per_module)
    return G, [fold_scales(s, fold_ratio(g, G)) for s, g in zip(scales_per_module, g_per_module)]


def rmsnorm(x_bf16: np.ndarray, w_bf16: np.ndarray, eps) -> tuple[np.ndarray, np.ndarray]:
    """BF16 RMSNorm: (y bf16 bits [rows, K], r per row as float32)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    rows, K = x.shape
    y = np.empty((rows, K), np.uint16)
    r = np.empty(rows, np.float32)
    lib().oracle_rmsnorm(_ptr(x), rows, K, K, _ptr(w), float(np.float32(eps)), _ptr(y), K, _ptr(r))
    return y, r


def _gdn_args(q, k, v, alpha, beta, B, T):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    assert q.shape[0] == k.shape[0] == v.shape[0] == alpha.shape[0] == beta.shape[0] == B * T
    return q, k, v, alpha, beta


def gdn_recurrence(q, k, v, alpha, beta, B: int, T: int, D: int = 128, S0=None, f32: bool = False):
    """The Gated DeltaNet recurrence: q, k bf16 bits [B*T, Hk*D]; v bf16 bits [B*T, Hv*D]; alpha, beta
    float32 [B*T, Hv]; S0 [B, Hv, D, D] or None. Returns (o [B*T, Hv*D], S_T [B, Hv, D, D]) in double
    (float32 with f32=True: the float32 twin, for sizing FP32 rounding error)."""
    q, k, v, alpha, beta = _gdn_args(q, k, v, alpha, beta, B, T)
    Hk, Hv = q.shape[1] // D, v.shape[1] // D
    dt = np.float32 if f32 else np.float64
    o = np.empty((B * T, Hv * D), dt)
    S = np.empty((B, Hv, D, D), dt)
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=dt)
    fn = lib().oracle_gdn_recurrence_f32 if f32 else lib().oracle_gdn_recurrence
    fn(_ptr(q), q.shape[1], _ptr(k), k.shape[1], _ptr(v), v.shape[1], _ptr(alpha), Hv, _ptr(beta), Hv,
       None if s0 is None else _ptr(s0), B, T, Hv, Hk, D, _ptr(o), _ptr(S))
    return o, S
