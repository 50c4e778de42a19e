"""Exhaustive device checks of the quantizer's fast arithmetic (E2M1 elements with an E4M3 scale per
16 elements: the Japanese article, "Mechanism 1" and FAQ "What is NVFP4?").

The NVFP4 encoder and the FP8 KV codec take every rounding decision in IEEE binary32, but compute
|x| / S with a reciprocal plus one exact-residual correction (quotient_fast), the E4M3 scale with a
clamp plus the gfx950 FP8 conversion, and the E2M1 codes with the gfx950 FP4 conversion. The
module libnvfp4_selftest.so runs the library's own helpers for these steps on the device:

* quotient_fast against the IEEE division for every finite non-negative bf16 numerator and every
  binary32 significand of the divisor, in divisor binades spread over the whole fast range
  (2^-80 .. 2^100); the IEEE division itself is pinned to numpy's binary32 division on the host;
* the FP8 and FP4 conversions over every non-negative binary32 input (and +inf): monotone, in
  range, sign-symmetric, packing into the right nibbles;
* the conversions at every grid point, every rounding midpoint and both binary32 neighbours of
  each, against the oracle's nearest-even rounding.
Monotone plus equal at all midpoints and their neighbours means equal on every input.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, host

pytestmark = pytest.mark.gpu

_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "nvfp4_w4a4_quantized_quantize_amd", "libnvfp4_selftest.so")


@pytest.fixture(scope="module")
def st():
    assert os.path.exists(_LIB), "libnvfp4_selftest.so is not built"
    L = ctypes.CDLL(_LIB)
    P, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
    L.nvfp4_selftest_quotient_scan.argtypes = [u32, P, P]
    L.nvfp4_selftest_e4m3_scan.argtypes = [P]
    L.nvfp4_selftest_e2m1_scan.argtypes = [P]
    L.nvfp4_selftest_eval.argtypes = [P, P, i64, P, P, P, P]
    for f in (L.nvfp4_selftest_quotient_scan, L.nvfp4_selftest_e4m3_scan, L.nvfp4_selftest_e2m1_scan,
              L.nvfp4_selftest_eval):
        f.restype = ctypes.c_int
    return L


def _counters(n):
    return torch.zeros(n, dtype=torch.int64, device=DEV)


def _eval(st, v, S=None):
    v = np.ascontiguousarray(v, dtype=np.float32)
    S = np.ones_like(v) if S is None else np.ascontiguousarray(S, dtype=np.float32)
    dv, dS = torch.from_numpy(v).to(DEV), torch.from_numpy(S).to(DEV)
    e4 = torch.empty(v.size, dtype=torch.uint8, device=DEV)
    e2 = torch.empty(v.size, dtype=torch.uint8, device=DEV)
    qi = torch.empty(v.size, dtype=torch.float32, device=DEV)
    qf = torch.empty(v.size, dtype=torch.float32, device=DEV)
    assert st.nvfp4_selftest_eval(dv.data_ptr(), dS.data_ptr(), v.size, e4.data_ptr(), e2.data_ptr(),
                                  qi.data_ptr(), qf.data_ptr()) == 0
    return host(e4), host(e2), host(qi), host(qf)


def _with_neighbours(points):
    p = np.asarray(points, dtype=np.float32)
    with np.errstate(over="ignore"):  # the largest float's upper neighbour is +inf, kept on purpose
        return np.unique(np.concatenate([p, np.nextafter(p, np.float32(-np.inf)), np.nextafter(p, np.float32(np.inf))]))


def e4m3_points():
    grid = np.array([oracle.e4m3_value(b) for b in range(127)], dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2  # at most 5 significant bits: exact in binary32
    extra = [448.0, 464.0, 480.0, 512.0, 2.0 ** -10, 2.0 ** -149, 2.0 ** -126, 3.0e38,
             np.finfo(np.float32).max]
    pts = _with_neighbours(np.concatenate([grid, mids, extra]).astype(np.float32))
    pts = pts[(pts >= 0) & np.isfinite(pts)]
    return np.concatenate([pts, np.array([np.inf], dtype=np.float32)])


def e2m1_points():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    extra = [7.0, 8.0, 2.0 ** -149, 2.0 ** -126, 3.0e38, np.finfo(np.float32).max]
    pts = _with_neighbours(np.concatenate([grid, mids, extra]).astype(np.float32))
    pts = pts[(pts >= 0) & np.isfinite(pts)]
    pts = np.concatenate([pts, np.array([np.inf], dtype=np.float32)])
    return np.concatenate([pts, -pts])


def test_fp8_conversion_exhaustive_monotone_and_in_range(st):
    c = _counters(3)
    assert st.nvfp4_selftest_e4m3_scan(c.data_ptr()) == 0
    checked, bad_range, bad_order = (int(v) for v in host(c))
    assert checked == 0x7F800001
    assert bad_range == 0 and bad_order == 0, (bad_range, bad_order)


def test_fp8_conversion_equals_oracle_at_every_midpoint(st):
    pts = e4m3_points()
    e4, _, _, _ = _eval(st, pts)
    ref = oracle.e4m3_from_float(pts)
    bad = np.nonzero(e4 != ref)[0]
    assert bad.size == 0, [(float(pts[i]), int(e4[i]), int(ref[i])) for i in bad[:8]]
    # the saturation edges: 448 is the top, 464 (midpoint to the next binade's 480) and above saturate
    idx = {float(p): i for i, p in enumerate(pts)}
    assert e4[idx[448.0]] == 0x7E and e4[idx[464.0]] == 0x7E and e4[idx[float(np.inf)]] == 0x7E
    assert e4[idx[float(np.nextafter(np.float32(432.0), np.float32(0)))]] == 0x7D  # below 432 rounds to 416
    assert e4[idx[2.0 ** -10]] == 0x00 and e4[idx[float(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))]] == 0x01


def test_fp4_conversion_exhaustive_monotone_signed_and_packed(st):
    c = _counters(5)
    assert st.nvfp4_selftest_e2m1_scan(c.data_ptr()) == 0
    checked, bad_sign, bad_order, bad_neg, bad_pack = (int(v) for v in host(c))
    assert checked == 0x7F800001
    assert (bad_sign, bad_order, bad_neg, bad_pack) == (0, 0, 0, 0)


def test_fp4_conversion_equals_oracle_at_every_midpoint(st):
    pts = e2m1_points()
    _, e2, _, _ = _eval(st, pts)
    ref = (np.signbit(pts).astype(np.uint8) << 3) | oracle.e2m1_from_float(np.abs(pts))
    bad = np.nonzero(e2 != ref)[0]
    assert bad.size == 0, [(float(pts[i]), int(e2[i]), int(ref[i])) for i in bad[:8]]


@pytest.fixture(scope="module")
def division_pinned(st):
    """Pins __fdiv_rn (the reference of the exhaustive scan) to numpy's IEEE binary32 division."""
    rng = np.random.default_rng(20260)
    n = 1 << 21
    a_bits = rng.integers(0, 0x7F80, n, dtype=np.uint32) << 16  # finite non-negative bf16
    s_bits = rng.integers(0x00800000, 0x7F800000, n, dtype=np.uint32)  # normal binary32 divisors
    a, S = a_bits.view(np.float32), s_bits.view(np.float32)
    _, _, qi, _ = _eval(st, a, S)
    with np.errstate(over="ignore", under="ignore"):
        ref = a / S
    assert (qi.view(np.uint32) == ref.view(np.uint32)).all(), "device __fdiv_rn differs from binary32 division"
    return True


def test_ieee_division_reference_pinned(division_pinned):
    assert division_pinned


# divisor binades (unbiased exponents) across the fast range [2^-80, 2^100]; inside a binade every
# significand is checked against every finite non-negative bf16 numerator
_BINADES = [-80, -79, -64, -30, -10, -4, -1, 0, 1, 3, 10, 30, 64, 99, 100]


@pytest.mark.parametrize("e", _BINADES)
def test_fast_quotient_equals_ieee_division(st, division_pinned, e):
    """quotient_fast equals the IEEE quotient whenever either reaches 2^-11; below that the residual
    may underflow and the last bits may differ, but every E2M1 code and E4M3 byte is the same (both
    are 0 there: the smallest nonzero decision point is 2^-10)."""
    c = _counters(4)
    first = torch.zeros(3, dtype=torch.int32, device=DEV)
    assert st.nvfp4_selftest_quotient_scan(e + 127, c.data_ptr(), first.data_ptr()) == 0
    checked, bad_big, diff_small, bad_code = (int(v) for v in host(c))
    f = host(first).view(np.uint32)
    assert checked > 0
    assert bad_big == 0 and bad_code == 0, \
        f"binade 2^{e}: {bad_big} quotients >= 2^-11 differ, {bad_code} codes differ; first a={f[0]:#010x} S={f[1]:#010x}"
    print(f"2^{e}: {checked} pairs; {diff_small} quotients below 2^-11 differ in their last bits (codes equal)")


def test_fast_quotient_at_points(st, division_pinned):
    """Random pairs inside the fast range through the point-evaluation entry, against numpy's binary32
    division: equal wherever the quotient reaches 2^-11, and below 2^-10 on both sides elsewhere."""
    rng = np.random.default_rng(7)
    n = 1 << 20
    a = (rng.integers(0, 0x7F80, n, dtype=np.uint32) << 16).view(np.float32)
    S = np.exp2(rng.uniform(-80, 100, n)).astype(np.float32)
    keep = (S >= 2.0 ** -80) & (S <= 2.0 ** 100) & (a.astype(np.float64) * 2.0 ** -100 <= S)
    a, S = a[keep], S[keep]
    _, _, _, qf = _eval(st, a, S)
    with np.errstate(over="ignore", under="ignore"):
        ref = a / S
    big = np.maximum(ref, qf) >= np.float32(2.0 ** -11)
    assert big.sum() > n // 4
    assert (qf.view(np.uint32)[big] == ref.view(np.uint32)[big]).all()
    assert (qf[~big] < np.float32(2.0 ** -10)).all()
