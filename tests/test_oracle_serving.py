"""Pins for the oracle's serving-path companions: the FP8 E4M3 KV-cache codec with static scales, the
fold-in repair of the fused-module scale mismatch, and the BF16 RMSNorm ahead of the quantizer.

Each property is fixed by something other than the oracle itself: torch's own float8_e4m3fn
conversion (an independent implementation of OCP E4M3FN rounding), exact closed forms, the E4M3
re-rounding bound 2^-4 (the pages report at most 6.2% re-rounding error for the fold-in repair),
invariants (scale invariance, RMS of a normalized row), and an exactly rounded sum (math.fsum).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

F8 = torch.float8_e4m3fn
E4M3_MIN_NORMAL = 2.0 ** -6


def bf16_bits(a) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def bf16_vals(bits) -> np.ndarray:
    return wl.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))


def torch_e4m3_bytes(t: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


# ------------------------------------------------------------------ FP8 KV codec
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kv_quantize_matches_torch_float8_in_range(seed):
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((64, 128)) * np.exp(rng.uniform(-6, 6, (64, 1))))
    s = np.float32(rng.uniform(0.001, 0.1))
    q = oracle.kv_quantize(x, s)
    t = bf16_vals(x) / s  # RN32 division, as the codec defines it
    inr = np.abs(t) <= 448
    assert inr.mean() > 0.5
    assert (q[inr] == torch_e4m3_bytes(t[inr])).all()
    # beyond the range: saturation, sign kept
    assert (q[~inr & (t > 0)] == 0x7E).all() and (q[~inr & (t < 0)] == 0xFE).all()


def test_kv_dequantize_matches_torch():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, size=(32, 256), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3C  # no NaN codes here
    s = np.float32(0.0123)
    y = oracle.kv_dequantize(q, s)
    ref = (torch.from_numpy(q).view(F8).to(torch.float32) * float(s)).to(torch.bfloat16)
    assert (y == ref.view(torch.int16).numpy().view(np.uint16)).all()


def test_kv_round_trip_of_representable_values():
    """x = e4m3(b) * s with s a power of two: exact in bf16, so q(x) = b and deq(q) = x."""
    s = np.float32(2.0 ** -3)
    b = np.array([v for v in range(256) if (v & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.array([oracle.e4m3_value(int(v) & 0x7F) * (-1 if v & 0x80 else 1) for v in b], np.float64) * float(s)
    x = bf16_bits(vals)
    assert (bf16_vals(x).astype(np.float64) == vals).all()
    q = oracle.kv_quantize(x[None, :], s)[0]
    assert (q == b).all()
    assert (oracle.kv_dequantize(q[None, :], s)[0] == x).all()


def test_kv_special_values():
    s = np.float32(0.5)
    x = np.array([[0x7F80, 0xFF80, 0x7FC0, 0x8000, 0x0000, int(bf16_bits([-1e-30])[0])]], np.uint16)
    q = oracle.kv_quantize(x, s)[0]
    assert list(q) == [0x7E, 0xFE, 0x7F, 0x80, 0x00, 0x80]
    y = oracle.kv_dequantize(np.array([[0x7F, 0x7E, 0xFE]], np.uint8), s)[0]
    assert np.isnan(bf16_vals(y[:1])).all() and list(bf16_vals(y[1:])) == [224.0, -224.0]


def test_kv_error_bound_and_scale():
    """Relative error at most 2^-4 in the normal range plus half a bf16 ulp; the calibrated scale maps
    the calibration amax onto 448."""
    rng = np.random.default_rng(9)
    x = bf16_bits(rng.standard_normal((256, 128)) * 3)
    s = oracle.kv_scale(x)
    amax = np.abs(bf16_vals(x)).max()
    assert abs(amax / float(s) - 448) <= 448 * 2.0 ** -22
    y = bf16_vals(oracle.kv_dequantize(oracle.kv_quantize(x, s), s)).astype(np.float64)
    xv = bf16_vals(x).astype(np.float64)
    normal = np.abs(xv) / float(s) >= E4M3_MIN_NORMAL
    rel = np.abs(y[normal] - xv[normal]) / np.abs(xv[normal])
    assert rel.max() <= 2.0 ** -4 + 2.0 ** -8
    assert np.abs(y[~normal] - xv[~normal]).max() <= float(s) * 2.0 ** -10 * (1 + 2.0 ** -7) + 1e-30


# ------------------------------------------------------------------ fold-in repair
FINITE_SCALES = np.arange(0x7F, dtype=np.uint8)  # every non-negative finite E4M3 byte


def decode(b) -> np.ndarray:
    return np.array([oracle.e4m3_value(int(v)) for v in np.ravel(b)], np.float64).reshape(np.shape(b))


@pytest.mark.parametrize("ratio", [1 / 1.82, 1 / 2.75, 0.999, 0.7, 0.5 + 2.0 ** -20, 0.123456, 0.031])
def test_fold_rerounding_bound(ratio):
    """P17: a folded scale is within 2^-4 (relative) of s * r in the E4M3 normal range, within half the
    subnormal spacing (2^-10) below it."""
    r = np.float32(ratio)
    folded = decode(oracle.fold_scales(FINITE_SCALES[None, :], r)[0])
    exact = decode(FINITE_SCALES) * float(r)
    normal = exact >= E4M3_MIN_NORMAL
    assert (np.abs(folded[normal] - exact[normal]) <= (2.0 ** -4 + 2.0 ** -22) * exact[normal]).all()
    assert (np.abs(folded[~normal] - exact[~normal]) <= 2.0 ** -10 * (1 + 2.0 ** -20)).all()


def test_fold_identity_and_powers_of_two():
    assert (oracle.fold_scales(FINITE_SCALES[None, :], 1.0)[0] == FINITE_SCALES).all()
    for k in (1, 2, 5):
        folded = decode(oracle.fold_scales(FINITE_SCALES[None, :], 2.0 ** -k)[0])
        exact = decode(FINITE_SCALES) * 2.0 ** -k
        representable = exact >= 2.0 ** -9  # halving stays exact down to the smallest subnormal
        # exact wherever s * 2^-k is itself an E4M3 value
        grid = set(decode(FINITE_SCALES).tolist())
        on_grid = np.array([e in grid for e in exact]) & representable
        assert on_grid.sum() >= 80
        assert (folded[on_grid] == exact[on_grid]).all()


def test_fold_monotone_sign_and_nan():
    r = np.float32(0.37)
    f = decode(oracle.fold_scales(FINITE_SCALES[None, :], r)[0])
    assert (np.diff(f) >= 0).all()
    b = np.array([[0x7F, 0xFF, 0x80 | 0x40, 0x40]], np.uint8)
    out = oracle.fold_scales(b, r)[0]
    assert out[0] == 0x7F and out[1] == 0x7F and out[2] == (0x80 | out[3])


def test_fold_group_end_to_end():
    """Two modules of one fused group: G is the larger global scale, the module holding it is left
    untouched, and every element of the other decodes within 2^-4 of its original value (normal
    blocks); the fused GEMM with G alone then tracks the exact per-segment result to that bound."""
    rng = np.random.default_rng(3)
    K = 256
    x1 = bf16_bits(rng.standard_normal((48, K)))
    x2 = bf16_bits(rng.standard_normal((40, K)) * 2.75)
    g1, g2 = oracle.global_scale(x1), oracle.global_scale(x2)
    (c1, s1), (c2, s2) = oracle.quantize(x1, g1), oracle.quantize(x2, g2)
    G, (f1, f2) = oracle.fold_group([s1, s2], [g1, g2])
    assert G == max(g1, g2) == g2
    assert (f2 == s2).all()
    orig = oracle.dequantize(c1, s1, g1)
    fold = oracle.dequantize(c1, f1, G)
    normal = (decode(s1) * float(oracle.fold_ratio(g1, G)) >= E4M3_MIN_NORMAL).repeat(16, axis=1)
    err = np.abs(fold - orig)
    assert (err[normal] <= (2.0 ** -4 + 2.0 ** -20) * np.abs(orig[normal])).all()
    # GEMM: per-segment exact vs fold-in with one scale
    a = bf16_bits(rng.standard_normal((8, K)))
    ga = oracle.global_scale(a)
    ac, as_ = oracle.quantize(a, ga)
    wc, ws = np.concatenate([c1, c2]), np.concatenate([s1, s2])
    y, T = oracle.gemm_rows(ac, as_, ga, wc, ws, [0, 48, 88], np.array([g1, g2], np.float32), np.arange(8))
    yf, _ = oracle.gemm_rows(ac, as_, ga, wc, np.concatenate([f1, f2]), [0, 88], np.array([G], np.float32),
                             np.arange(8))
    assert (np.abs(yf - y) <= (2.0 ** -4 + 2.0 ** -20) * T + 1e-12).all()
    assert (yf[:, 48:] == y[:, 48:]).all()


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_constant_rows_and_unit_weight():
    """A row of ones with eps = 0 has r = 1: y1 = x, and y = bf16(w)."""
    K = 160
    x = bf16_bits(np.ones((3, K)))
    w = bf16_bits(np.linspace(-3, 3, K))
    y, r = oracle.rmsnorm(x, w, 0.0)
    assert (r == 1.0).all()
    assert (y == w[None, :]).all()


def test_rmsnorm_scale_invariance():
    """x -> 2^k x with eps = 0 scales r by 2^-k exactly, so y does not change."""
    rng = np.random.default_rng(4)
    x = bf16_bits(rng.standard_normal((16, 512)))
    w = bf16_bits(rng.uniform(0.5, 1.5, 512))
    y, r = oracle.rmsnorm(x, w, 0.0)
    for k in (-7, 3, 20):
        xk = bf16_bits(bf16_vals(x) * np.float32(2.0 ** k))
        yk, rk = oracle.rmsnorm(xk, w, 0.0)
        assert (yk == y).all() and (rk == (r * np.float32(2.0 ** -k))).all()


def test_rmsnorm_r_from_exactly_rounded_sum_and_unit_rms():
    rng = np.random.default_rng(6)
    K, eps = 5120, np.float32(1e-6)
    x = bf16_bits(rng.standard_normal((8, K)) * np.exp(rng.uniform(-4, 4, (8, 1))))
    w = bf16_bits(np.ones(K))
    y, r = oracle.rmsnorm(x, w, eps)
    xv = bf16_vals(x).astype(np.float64)
    for i in range(8):
        ms = math.fsum(v * v for v in xv[i]) / K
        assert np.float32(1.0 / math.sqrt(ms + float(eps))) == r[i]
    # with w = 1, y = y1, and a normalized row has mean square ms / (ms + eps) up to bf16 rounding
    yv = bf16_vals(y).astype(np.float64)
    ms_rows = (xv * xv).mean(axis=1)
    assert np.allclose((yv * yv).mean(axis=1), ms_rows / (ms_rows + float(eps)), rtol=2.0 ** -7)


def test_rmsnorm_rounding_order_matches_torch_bf16_arithmetic():
    """The two bf16 roundings of the norm's output, y = bf16(w * bf16(x * r)), against PyTorch's own
    CPU arithmetic: a float32 product x * r, a cast to bf16 and a bf16 x bf16 multiply (which torch
    rounds to bf16 once). Given the oracle's r (pinned above by the exactly rounded sum), every
    output must agree bit for bit. The rows are chosen so that a single rounding of x * r * w gives a
    different answer on some elements, so the pin tells the two readings apart."""
    import torch
    rng = np.random.default_rng(31)
    K = 1024
    x = bf16_bits(rng.standard_normal((16, K)) * np.exp(rng.uniform(-3, 3, (16, 1))))
    w = bf16_bits(rng.uniform(0.3, 2.7, K))
    y, r = oracle.rmsnorm(x, w, np.float32(1e-6))
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    rt = torch.from_numpy(r)[:, None]
    ref = (wt[None, :] * (xt * rt).to(torch.bfloat16)).view(torch.int16).numpy().view(np.uint16)
    assert (y == ref).all()
    once = ((xt * rt) * wt.float()[None, :]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (once != y).sum() > 100, "the sample does not separate one rounding from two"
