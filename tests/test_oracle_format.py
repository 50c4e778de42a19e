"""Pins for the oracle's E2M1 / E4M3FN encodings (CPU only).

The oracle's format code is checked against fixtures taken from the format definitions the pages name
(E2M1 elements with E4M3 block scales: Japanese article, "Mechanism 1" and FAQ "What is NVFP4?"),
against PyTorch's independent float8_e4m3fn implementation, and against exact brute-force rounding
written here with rational arithmetic.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden

E2M1_TABLE = {int(c): float(v) for c, v in (ln.split() for ln in read_golden("e2m1_magnitudes.txt"))}


def test_e2m1_decode_matches_format_table():
    assert sorted(E2M1_TABLE) == list(range(8))
    for c, v in E2M1_TABLE.items():
        assert oracle.e2m1_value(c) == v
        neg = oracle.e2m1_value(c | 8)
        assert neg == -v and math.copysign(1.0, neg) == -1.0


def test_e4m3_decode_golden_points():
    for ln in read_golden("e4m3fn_points.txt"):
        byte_s, val_s = ln.split()[:2]
        b = int(byte_s, 16)
        got = oracle.e4m3_value(b)
        if val_s == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val_s) and math.copysign(1.0, got) == math.copysign(1.0, float(val_s))


def test_e4m3_decode_all_bytes_match_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def _e4m3_structured_inputs():
    # Every float32 in [0, 448] whose low 12 mantissa bits are one of a few edge patterns: every
    # E4M3 rounding midpoint (whose low 12 bits are zero) and both float neighbours of
    # each, across every exponent, including the subnormal-scale range.
    hi = np.arange(0, (0x43E00000 >> 12) + 1, dtype=np.uint32) << 12
    lows = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    v = bits.view(np.float32)
    return v[v <= 448.0]


def test_e4m3_encode_matches_torch_rne_structured():
    v = _e4m3_structured_inputs()
    got = oracle.e4m3_from_float(v)
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (got == ref).all(), np.flatnonzero(got != ref)[:10]


def test_e4m3_encode_matches_torch_rne_random():
    rng = np.random.default_rng(11)
    v = np.abs(rng.standard_normal(400_000).astype(np.float32) * np.float32(50.0))
    v = np.concatenate([v, rng.uniform(0, 2 ** -6, 100_000).astype(np.float32)])
    v = v[v <= 448.0]
    got = oracle.e4m3_from_float(v)
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (got == ref).all()


def test_e4m3_encode_saturates():
    v = np.array([448.0, np.nextafter(np.float32(448.0), np.float32(1e9)), 463.9, 464.0, 480.0, 1e6,
                  3.4e38, np.inf], dtype=np.float32)
    assert (oracle.e4m3_from_float(v) == 0x7E).all()


def _e4m3_grid_exact():
    vals = []
    for b in range(127):
        e, m = b >> 3, b & 7
        vals.append(Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    return vals


def _nearest_even_bruteforce(v: Fraction, grid):
    """Argmin over every candidate, ties to the even index; saturating above the top."""
    if v >= grid[-1]:
        return len(grid) - 1
    best, bestd = None, None
    for i, gval in enumerate(grid):
        d = abs(gval - v)
        if bestd is None or d < bestd or (d == bestd and i % 2 == 0):
            best, bestd = i, d
    return best


def test_e4m3_encode_bruteforce_exact_sample():
    grid = _e4m3_grid_exact()
    rng = np.random.default_rng(5)
    mids = [(grid[i] + grid[i + 1]) / 2 for i in range(126)]
    vals = [np.float32(float(m)) for m in mids]  # midpoints are exact in float32
    vals += [np.nextafter(x, np.float32(0)) for x in vals] + [np.nextafter(x, np.float32(1e9)) for x in vals]
    vals += list(np.abs(rng.standard_normal(3000).astype(np.float32)) * np.float32(30))
    vals += list(rng.uniform(0, 0.02, 1000).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    got = oracle.e4m3_from_float(vals)
    for v, gb in zip(vals, got):
        assert gb == _nearest_even_bruteforce(Fraction(float(v)), grid), float(v)
    # ties go to the even mantissa
    for i, m in enumerate(mids):
        assert oracle.e4m3_from_float([float(m)])[0] == (i if i % 2 == 0 else i + 1)


E2M1_GRID = [Fraction(E2M1_TABLE[c]) for c in range(8)]
E2M1_MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def test_e2m1_encode_midpoints_and_neighbours():
    # ties go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0
    expect_tie = [0, 2, 2, 4, 4, 6, 6]
    for mp, ec in zip(E2M1_MIDPOINTS, expect_tie):
        x = np.float32(mp)
        assert oracle.e2m1_from_float([x])[0] == ec
        lo = oracle.e2m1_from_float([np.nextafter(x, np.float32(0))])[0]
        hi = oracle.e2m1_from_float([np.nextafter(x, np.float32(10))])[0]
        assert hi == lo + 1
        assert ec in (lo, hi)


def test_e2m1_encode_bruteforce_structured_and_random():
    hi = np.arange(0, (0x41000000 >> 16) + 1, dtype=np.uint32) << 16  # [0, 8]
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0xFFFF], dtype=np.uint32)
    structured = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    rng = np.random.default_rng(3)
    rand = rng.uniform(0, 8, 200_000).astype(np.float32)
    v = np.concatenate([structured, rand, np.array([6.0, 7.0, 100.0, 3.4e38, np.inf], np.float32)])
    got = oracle.e2m1_from_float(v)
    # brute force over all 8 candidates with exact float64 distances (v - grid is exact here for
    # v >= 2^-20; below that the nearest candidate is 0 by a wide margin)
    grid = np.array([float(x) for x in E2M1_GRID])
    d = np.abs(v.astype(np.float64)[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even_pick = np.where(cand[:, ::2].any(axis=1), np.argmax(cand[:, ::2], axis=1) * 2, np.argmax(cand, axis=1))
    expect = np.where(v >= 6.0, 7, even_pick)
    assert (got == expect).all(), v[got != expect][:10]


def test_e2m1_encode_exact_fraction_sample():
    rng = np.random.default_rng(9)
    vals = rng.uniform(0, 7, 2000).astype(np.float32)
    got = oracle.e2m1_from_float(vals)
    for v, g in zip(vals, got):
        assert g == _nearest_even_bruteforce(Fraction(float(v)), E2M1_GRID)
