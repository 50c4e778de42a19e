"""Pins for the oracle's NVFP4 quantizer and global scale (CPU only).

Recipe (Japanese article, "Mechanism 1" and FAQ "What is NVFP4?"; English abstract point (i)):
E2M1 codes, one E4M3 scale per 16 elements chosen from the block maximum, and one FP32 global scale
per module ("Trap 1"). Each test below pins the oracle to something other than itself: hand-worked
blocks, exact round trips, ties, special blocks, exact rational rounding for power-of-two global
scales, and invariants that hold for any input.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import read_golden
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e4m3(b):
    e, m = b >> 3, b & 7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


def exact_bf16(vals):
    f = np.asarray(vals, dtype=np.float32)
    bits = f32_to_bf16_bits(f)
    assert (bf16_bits_to_f32(bits).view(np.uint32) == f.view(np.uint32)).all(), "not bf16-exact"
    return bits


def unpack(codes):
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def test_worked_blocks_golden():
    for ln in read_golden("worked_blocks.txt"):
        name, g, xs, sc, cb = [p.strip() for p in ln.split("|")]
        x = exact_bf16([float(v) for v in xs.split()])[None, :]
        codes, scales = oracle.quantize(x, np.float32(float(g)))
        assert scales[0, 0] == int(sc, 16), name
        assert list(codes[0]) == [int(b, 16) for b in cb.split()], name


def test_global_scale_closed_form():
    for amax, g in [(2688.0, 1.0), (1344.0, 0.5), (5376.0, 2.0), (0.0, 0.0)]:
        x = exact_bf16([[amax / 4, -amax, amax / 2] + [0.0] * 13])
        assert oracle.global_scale(x) == np.float32(g)
    x = exact_bf16([[-3.0, 2.0] * 8])
    assert oracle.tensor_amax(x) == 3.0
    assert oracle.global_scale(x) == np.float32(3.0) / np.float32(2688.0)


def _roundtrip_blocks(j):
    """Blocks whose values are code * s * 2^j for every positive E4M3 scale s and every code."""
    g = 2.0 ** j
    order = [7, 0, 1, 2, 3, 4, 5, 6, 8, 9, 10, 11, 12, 13, 14, 15]  # first element sets amax
    rows, want_codes, want_scales = [], [], []
    for sb in range(1, 127):
        s = e4m3(sb)
        vals = [(-1 if c & 8 else 1) * E2M1[c & 7] * s * g for c in order]
        vals[8] = -0.0  # code 8 is negative zero
        rows.append(vals)
        want_codes.append(order)
        want_scales.append(sb)
    return g, exact_bf16(rows), np.array(want_codes), np.array(want_scales)


@pytest.mark.parametrize("j", list(range(-20, 11)))
def test_exact_roundtrip_power_of_two_global_scale(j):
    g, x, want_codes, want_scales = _roundtrip_blocks(j)
    codes, scales = oracle.quantize(x, np.float32(g))
    assert (scales[:, 0] == want_scales).all()
    assert (unpack(codes) == want_codes).all()


@pytest.mark.parametrize("sb", [0x01, 0x05, 0x08, 0x30, 0x38, 0x3B, 0x5D, 0x77, 0x7E])
def test_ties_and_bf16_neighbours(sb):
    g = 2.0 ** -4
    s = e4m3(sb)
    S = s * g
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    tie_code = [0, 2, 2, 4, 4, 6, 6]
    rows, expect = [], []
    for sign in (1.0, -1.0):
        for m, tc in zip(mids, tie_code):
            xm = exact_bf16([m * S])[0]
            up, down = np.uint16(xm + 1), np.uint16(xm - 1)  # next bf16 above / below (positive)
            for xb, code in [(xm, tc), (up, mids.index(m) + 1), (down, mids.index(m))]:
                row = exact_bf16([6 * S] + [0.0] * 15)
                row[1] = xb | (0x8000 if sign < 0 else 0)
                rows.append(row)
                expect.append(code | (8 if sign < 0 else 0))
    x = np.stack(rows)
    codes, scales = oracle.quantize(x, np.float32(g))
    assert (scales[:, 0] == sb).all()
    assert (unpack(codes)[:, 1] == np.array(expect)).all()
    assert (unpack(codes)[:, 0] == 7).all()


def test_zero_block():
    x = exact_bf16([[0.0] * 8 + [-0.0] * 8])
    codes, scales = oracle.quantize(x, np.float32(0.01))
    assert scales[0, 0] == 0
    assert list(unpack(codes)[0]) == [0] * 8 + [8] * 8


def test_saturating_block():
    # global scale calibrated for a tensor 8x smaller than this block: s_raw = 8 * 448 > 448
    amax = 96.0
    g = np.float32(amax) / np.float32(6 * 448 * 8)
    vals = [amax, -amax / 2, amax / 8, 1.0, -0.125, 0.0] + [2.0] * 10
    x = exact_bf16([vals])
    codes, scales = oracle.quantize(x, g)
    assert scales[0, 0] == 0x7E
    S = np.float32(448.0) * g
    mags = unpack(codes)[0] & 7
    for v, m in zip(vals, mags):
        if abs(v) / S > 5:
            assert m == 7
    assert unpack(codes)[0][1] == 15  # -48 saturates to -6


def test_underflowing_block():
    g = np.float32(2.0 ** -3)
    # amax / (6 g) <= 2^-10 rounds to scale 0 (2^-10 itself is a tie with 0 and 2^-9 -> even -> 0)
    tie = 6 * 2.0 ** -3 * 2.0 ** -10
    tie_up = float(bf16_bits_to_f32(exact_bf16([tie]) + np.uint16(1))[0])  # next bf16 above
    for amax, want in [(tie, 0), (tie / 2, 0), (tie_up, 1)]:
        x = exact_bf16([[amax, -amax / 2] + [0.0] * 14])
        codes, scales = oracle.quantize(x, g)
        assert scales[0, 0] == want
        if want == 0:
            assert list(unpack(codes)[0][:2]) == [0, 8]


def _exact_rne(v: Fraction, grid):
    if v >= grid[-1]:
        return len(grid) - 1
    lo = max(i for i, gv in enumerate(grid) if gv <= v)
    hi = lo + 1
    if v - grid[lo] < grid[hi] - v:
        return lo
    if v - grid[lo] > grid[hi] - v:
        return hi
    return lo if lo % 2 == 0 else hi


E4M3_GRID = [Fraction(e4m3(b)) for b in range(127)]
E2M1_GRID = [Fraction(v) for v in E2M1]


@pytest.mark.parametrize("j", [-12, -5, 0, 4])
def test_matches_exact_rational_rounding_for_power_of_two_g(j):
    """With g = 2^j, every FP32 step is either exact or cannot move a value across a rounding
    midpoint, so the FP32 recipe must equal exact real-number rounding (computed with fractions)."""
    rng = np.random.default_rng(100 + j)
    # heavy-tailed values spread over many binades, rounded to bf16
    x = f32_to_bf16_bits((rng.standard_t(3, size=(24, 64)) * 2.0 ** (j + 3)).astype(np.float32))
    g = Fraction(2) ** j
    codes, scales = oracle.quantize(x, np.float32(float(g)))
    xf = bf16_bits_to_f32(x).astype(np.float64)
    cu = unpack(codes)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            blk = [Fraction(float(v)) for v in xf[r, 16 * b:16 * b + 16]]
            amax = max(abs(v) for v in blk)
            sb = _exact_rne(amax / (6 * g), E4M3_GRID)
            assert scales[r, b] == sb
            s = E4M3_GRID[sb]
            for i, v in enumerate(blk):
                mag = 0 if s == 0 else _exact_rne(abs(v) / (s * g), E2M1_GRID)
                sign = 8 if np.signbit(xf[r, 16 * b + i]) else 0
                assert cu[r, 16 * b + i] == sign | mag


def _random_heavy(seed, rows, K):
    rng = np.random.default_rng(seed)
    v = rng.standard_t(3, size=(rows, K)).astype(np.float32)
    v[:, rng.choice(K, 3, replace=False)] *= 50
    v[rng.random((rows, K)) < 0.01] = 0.0
    return f32_to_bf16_bits(v)


@pytest.mark.parametrize("g_kind", ["tensor", "random"])
def test_invariants_random(g_kind):
    x = _random_heavy(7, 64, 512)
    g = oracle.global_scale(x) if g_kind == "tensor" else np.float32(0.0173)
    codes, scales = oracle.quantize(x, g)
    assert codes.shape == (64, 256) and scales.shape == (64, 32)
    cu = unpack(codes)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    xhat = oracle.dequantize(codes, scales, g)
    s = np.vectorize(e4m3)(scales.astype(int))
    S = np.repeat(s, 16, axis=1) * float(g)
    # (i) a block with a normal scale holds at least one code of magnitude 6
    mag7 = (cu & 7).reshape(64, 32, 16).max(axis=2) == 7
    assert mag7[scales >= 0x08].all()
    # (ii) off saturation, the error is at most half the local E2M1 step (plus FP32 slack)
    v = np.abs(xf) / np.where(S > 0, S, 1)
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    ok = (S == 0) | (v > 6) | (np.abs(xf - xhat) <= (half_step + 6 * 2.0 ** -23) * S)
    assert ok.all()
    # (iii) the decoded value lies on S times the E2M1 grid, with the input's sign
    grid_pos = np.abs(xhat) / np.where(S > 0, S, 1)
    assert np.isin(np.round(grid_pos, 12), E2M1).all()
    assert (np.signbit(xhat[xhat != 0]) == np.signbit(xf[xhat != 0])).all()
    # zero-scale blocks decode to zero
    assert (xhat[S == 0] == 0).all()


def test_sign_of_zero_codes_follows_input():
    g = np.float32(2.0 ** -6)
    x = exact_bf16([[3.0, -0.0, 0.0, -0.0078125, 0.0078125] + [0.0] * 11])
    codes, _ = oracle.quantize(x, g)
    assert list(unpack(codes)[0][:5]) == [7, 8, 0, 8, 0]


def test_rejects_ragged_k():
    x = np.zeros((2, 24), dtype=np.uint16)
    with pytest.raises(AssertionError):
        oracle.quantize(x, 1.0)
