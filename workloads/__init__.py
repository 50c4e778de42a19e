"""Seeded synthetic workloads for the NVFP4 W4A4 quantized linear layer.

Input generation only: this module draws the bf16 activations, bf16 weights and gate parameters of
each configuration and holds none of the method's arithmetic (no scale, no rounding to E2M1/E4M3,
no GEMM). Both the HIP path and the CPU oracle take their inputs from here.

The shapes follow the model the pages study (hidden size 5120, MLP 17408, Gated DeltaNet projection
widths q/k 2048, v/z 4096, b/a 32 heads; Japanese article, "Experiment design" and "Trap 1"). The
activation statistics imitate the heavy tails and hot channels the pages report (Japanese article,
"Mechanism 1": max/RMS about 63.5, kurtosis about 1,560, a hot channel about 100x the median), and
the per-segment weight spreads echo the fused-module global-scale ratios 1.82x (qkv vs z) and 2.75x
(b vs a) of "Trap 1". No real data, dataset or checkpoint is used.

Recipe (all seeds start from ``seed``; every tensor has its own stream):
  * "N(0, s)" means a normal with standard deviation s; Student-t has nu = 3 and is unscaled;
  * outlier channels: round(0.001 K) columns (2 for the tiny case) chosen without replacement by
    the tensor's own stream, multiplied by 50 (40 for the tiny case);
  * values are drawn in float32 and rounded to bf16 with round-to-nearest-even;
  * rows are drawn in chunks of ROW_CHUNK from numpy.random.default_rng([seed, cfg, tensor, chunk])
    so any row range can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

ROW_CHUNK = 256

# epilogue kinds and output dtypes, mirrored from the C interface
EPI_NONE, EPI_SIGMOID, EPI_GDN_DECAY = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Dist:
    kind: str               # "normal" or "student_t3"
    std: float = 1.0        # standard deviation for "normal"
    n_outliers: int = 0     # number of outlier channels (columns along K)
    outlier_mult: float = 1.0


@dataclasses.dataclass(frozen=True)
class Segment:
    name: str
    n: int                  # output columns of this module
    w_std_ratio: float      # weight std = ratio / sqrt(K)
    epilogue: int = EPI_NONE
    out_dtype: int = OUT_BF16


@dataclasses.dataclass(frozen=True)
class GemmCase:
    name: str
    cfg_id: int
    M: int
    K: int
    x_dist: Dist
    segments: tuple
    w_std_abs: float | None = None   # absolute weight std (tiny case), else ratio/sqrt(K)
    gate_params: bool = False        # draws A_log, dt_bias for gate segments

    @property
    def N(self) -> int:
        return sum(s.n for s in self.segments)

    @property
    def seg_bounds(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([s.n for s in self.segments])]).astype(np.int64)

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([seed, *ids])


def _outlier_cols(seed: int, cfg: int, tensor: int, K: int, n: int) -> np.ndarray:
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, cfg, tensor, 1_000_000).choice(K, size=n, replace=False))


def draw_matrix(seed: int, cfg: int, tensor: int, rows: int, K: int, dist: Dist,
                row_begin: int = 0, row_end: int | None = None) -> np.ndarray:
    """bf16 bits [row_end - row_begin, K] of the (rows x K) tensor ``tensor`` of config ``cfg``."""
    row_end = rows if row_end is None else row_end
    assert 0 <= row_begin <= row_end <= rows
    cols = _outlier_cols(seed, cfg, tensor, K, dist.n_outliers)
    out = np.empty((row_end - row_begin, K), dtype=np.uint16)
    c0 = row_begin // ROW_CHUNK
    c1 = (row_end + ROW_CHUNK - 1) // ROW_CHUNK
    for c in range(c0, c1):
        lo, hi = c * ROW_CHUNK, min(rows, (c + 1) * ROW_CHUNK)
        g = _rng(seed, cfg, tensor, c)
        if dist.kind == "normal":
            v = g.standard_normal((hi - lo, K), dtype=np.float32) * np.float32(dist.std)
        elif dist.kind == "student_t3":
            v = g.standard_t(3, size=(hi - lo, K)).astype(np.float32)
        else:
            raise ValueError(dist.kind)
        if cols.size:
            v[:, cols] *= np.float32(dist.outlier_mult)
        a, b = max(lo, row_begin), min(hi, row_end)
        out[a - row_begin:b - row_begin] = f32_to_bf16_bits(v[a - lo:b - lo])
    return out


def n_outliers(K: int) -> int:
    return int(round(0.001 * K))


def heavy(K: int) -> Dist:
    return Dist("student_t3", n_outliers=n_outliers(K), outlier_mult=50.0)


def normal_outliers(K: int) -> Dist:
    return Dist("normal", std=1.0, n_outliers=n_outliers(K), outlier_mult=50.0)


HIDDEN, MLP = 5120, 17408

C1 = GemmCase("tiny_16x128x256", 1, 16, 256, Dist("normal", 1.0, 2, 40.0),
              (Segment("out", 128, 0.0, EPI_NONE, OUT_F32),), w_std_abs=0.02)
C2 = GemmCase("prefill_proj_4096x5120x5120", 2, 4096, HIDDEN, heavy(HIDDEN),
              (Segment("out", HIDDEN, 1.0, EPI_NONE, OUT_BF16),))


def C3(M: int, direction: str) -> GemmCase:
    if direction == "up":
        return GemmCase(f"decode_up_M{M}", 30 + {1: 0, 16: 1, 64: 2}[M], M, HIDDEN,
                        normal_outliers(HIDDEN), (Segment("up", MLP, 1.0),))
    return GemmCase(f"decode_down_M{M}", 33 + {1: 0, 16: 1, 64: 2}[M], M, MLP,
                    normal_outliers(MLP), (Segment("down", HIDDEN, 1.0),))


C4 = GemmCase("mlp_gate_up_8192x34816x5120", 4, 8192, HIDDEN, heavy(HIDDEN),
              (Segment("gate", MLP, 1.0), Segment("up", MLP, 3.0)))

GDN_SEGMENTS = (
    Segment("q", 2048, 1.00), Segment("k", 2048, 1.25), Segment("v", 4096, 1.82),
    Segment("z", 4096, 1.00), Segment("b", 32, 2.75, EPI_SIGMOID, OUT_F32),
    Segment("a", 32, 1.00, EPI_GDN_DECAY, OUT_F32),
)
C5 = GemmCase("gdn_in_proj_32768x12352x5120", 5, 32768, HIDDEN, heavy(HIDDEN), GDN_SEGMENTS,
              gate_params=True)

ALL = {"C1": C1, "C2": C2, "C3_up_1": C3(1, "up"), "C3_up_16": C3(16, "up"),
       "C3_up_64": C3(64, "up"), "C3_down_1": C3(1, "down"), "C3_down_16": C3(16, "down"),
       "C3_down_64": C3(64, "down"), "C4": C4, "C5": C5}

X_TENSOR, GATE_TENSOR = 0, 99


def draw_x(case: GemmCase, seed: int = 0, row_begin: int = 0, row_end: int | None = None,
           M: int | None = None) -> np.ndarray:
    """Activations, bf16 bits [M, K]. ``M`` overrides the case's row count (smaller test sizes)."""
    M = case.M if M is None else M
    return draw_matrix(seed, case.cfg_id, X_TENSOR, M, case.K, case.x_dist, row_begin, row_end)


def draw_w(case: GemmCase, seg_index: int, seed: int = 0, n: int | None = None) -> np.ndarray:
    """Weights of one segment (module), bf16 bits [n, K] as in nn.Linear."""
    seg = case.segments[seg_index]
    n = seg.n if n is None else n
    std = case.w_std_abs if case.w_std_abs is not None else seg.w_std_ratio / math.sqrt(case.K)
    return draw_matrix(seed, case.cfg_id, 1 + seg_index, n, case.K, Dist("normal", std))


def draw_gate_params(case: GemmCase, seg_index: int, seed: int = 0, n: int | None = None):
    """A_log, dt_bias ~ N(0, 0.5), float32 [n] for a gate segment."""
    seg = case.segments[seg_index]
    n = seg.n if n is None else n
    g = _rng(seed, case.cfg_id, GATE_TENSOR, seg_index)
    a_log = (g.standard_normal(n, dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    dt_bias = (g.standard_normal(n, dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    return a_log, dt_bias


# ------------------------------------------------------------------ serving-path companions
@dataclasses.dataclass(frozen=True)
class KvCase:
    """K and V caches of the attention layers for one prefill: [tokens, kv_heads * head_dim] each.
    The pages give 16 softmax-attention layers out of 64 and 32 shipped KV scales (Japanese article,
    "Is FP8 enough for the KV cache?"); 8 KV heads of 128 dimensions is this recipe's choice (the
    pages do not give the attention geometry). Keys get a few hot channels, values none."""
    name: str
    cfg_id: int
    tokens: int
    kv_heads: int
    head_dim: int
    layers: int

    @property
    def cols(self) -> int:
        return self.kv_heads * self.head_dim


KV = KvCase("kv_cache_16x2x32768x1024", 40, 32768, 8, 128, 16)
KV_DISTS = (Dist("normal", 1.0, n_outliers=8, outlier_mult=10.0), Dist("normal", 1.0))


def draw_kv(case: KvCase, which: int, seed: int = 0, row_begin: int = 0, row_end: int | None = None,
            tokens: int | None = None) -> np.ndarray:
    """bf16 bits [tokens, cols] of the K (which = 0) or V (which = 1) cache of one layer."""
    tokens = case.tokens if tokens is None else tokens
    return draw_matrix(seed, case.cfg_id, which, tokens, case.cols, KV_DISTS[which], row_begin, row_end)


@dataclasses.dataclass(frozen=True)
class NormCase:
    """RMSNorm ahead of a quantized projection: X [rows, K] with the heavy-tailed activation recipe
    and a bf16 norm weight drawn uniformly from [0.5, 1.5]."""
    name: str
    cfg_id: int
    rows: int
    K: int
    x_dist: Dist


NORM = NormCase("rmsnorm_quantize_32768x5120", 50, 32768, HIDDEN, heavy(HIDDEN))


def draw_norm_x(case: NormCase, seed: int = 0, row_begin: int = 0, row_end: int | None = None,
                rows: int | None = None) -> np.ndarray:
    rows = case.rows if rows is None else rows
    return draw_matrix(seed, case.cfg_id, X_TENSOR, rows, case.K, case.x_dist, row_begin, row_end)


def draw_norm_weight(case: NormCase, seed: int = 0) -> np.ndarray:
    g = _rng(seed, case.cfg_id, GATE_TENSOR, 0)
    return f32_to_bf16_bits(g.uniform(0.5, 1.5, case.K).astype(np.float32))


@dataclasses.dataclass(frozen=True)
class GdnCase:
    """Inputs of the Gated DeltaNet recurrence after the fused in_proj GEMM: B sequences of T tokens,
    Hv value heads and Hk key heads of D dimensions (the in_proj widths: q/k 2048 = 16 x 128, v 4096
    = 32 x 128, gates 32). q and k rows are unit-norm per head (as after the model's own
    normalization, which the pages do not describe), v ~ N(0, 1); the decay alpha is 1 - 10^u with
    u drawn per head in [-5, -0.5] plus a per-token jitter of +-0.25 (decay horizons from a few
    tokens to about 10^5, covering the pages' 44K-62K), and the write strength beta ~ U(0.05, 1)."""
    name: str
    cfg_id: int
    B: int
    T: int
    Hv: int = 32
    Hk: int = 16
    D: int = 128


GDN_PREFILL = GdnCase("gdn_recurrence_1x32768", 60, 1, 32768)
GDN_DECODE = GdnCase("gdn_decode_64x1", 61, 64, 1)


def draw_gdn(case: GdnCase, seed: int = 0, T: int | None = None, B: int | None = None):
    """(q, k, v) bf16 bits and (alpha, beta) float32, rows ordered [b][t]."""
    T = case.T if T is None else T
    B = case.B if B is None else B
    g = _rng(seed, case.cfg_id, 7, B, T)
    rows = B * T

    def unit_rows(n_heads):
        x = g.standard_normal((rows, n_heads, case.D), dtype=np.float32)
        x /= np.linalg.norm(x, axis=2, keepdims=True).astype(np.float32)
        return f32_to_bf16_bits(x.reshape(rows, n_heads * case.D))

    q, k = unit_rows(case.Hk), unit_rows(case.Hk)
    v = f32_to_bf16_bits(g.standard_normal((rows, case.Hv * case.D), dtype=np.float32))
    u = g.uniform(-5.0, -0.5, case.Hv)[None, :] + g.uniform(-0.25, 0.25, (rows, case.Hv))
    alpha = (1.0 - 10.0 ** u).astype(np.float32)
    beta = g.uniform(0.05, 1.0, (rows, case.Hv)).astype(np.float32)
    return q, k, v, alpha, beta
