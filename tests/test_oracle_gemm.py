"""Pins for the oracle's block-scaled GEMM with per-segment global scales (CPU only).

The GEMM is the plain definition: y[m, n] = g_a * g_w[seg(n)] * sum_k a[m, k] w[n, k] over the
block-decoded operands. The per-segment global scale is the fused-module repair the pages describe
(Japanese article, "Trap 1"; English abstract; aimodeling.com translation, "What engineers should
actually take away"). The oracle is pinned against a hand-worked example, brute-force rational dot
products, numpy float64 matmul, special operands and the fused == unfused invariant. Operands are
decoded here independently of the oracle (golden E2M1 table, torch float8_e4m3fn).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden

E2M1 = {int(c): float(v) for c, v in (ln.split() for ln in read_golden("e2m1_magnitudes.txt"))}
E2M1_SIGNED = np.array([E2M1[c & 7] * (-1 if c & 8 else 1) for c in range(16)])
E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def decode(codes, scales):
    """Independent decode: float64 [R, K] without the global scale."""
    lo, hi = codes & 0xF, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    return E2M1_SIGNED[c] * np.repeat(E4M3[scales], 16, axis=1)


def random_operand(rng, rows, K, scale_lo=0x20, scale_hi=0x50):
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(rows, K // 16), dtype=np.uint8)
    return codes, scales


def test_worked_gemm_golden():
    d = {ln.split()[0]: ln.split()[1:] for ln in read_golden("worked_gemm.txt")}
    hexrow = lambda k: np.array([int(b, 16) for b in d[k]], dtype=np.uint8)
    a_c, a_s = hexrow("a_codes")[None], hexrow("a_scale")[None]
    w_c = np.stack([hexrow("w0_codes"), hexrow("w1_codes"), hexrow("w2_codes")])
    w_s = np.stack([hexrow("w0_scale"), hexrow("w1_scale"), hexrow("w2_scale")])
    bounds = [int(v) for v in d["seg_bounds"]]
    g_w = np.array([float(v) for v in d["g_w"]], dtype=np.float32)
    y, T = oracle.gemm_rows(a_c, a_s, np.float32(float(d["g_a"][0])), w_c, w_s, bounds, g_w, [0])
    assert list(y[0]) == [float(v) for v in d["y"]]
    scale = np.array([float(d["g_a"][0]) * g_w[0]] * 2 + [float(d["g_a"][0]) * g_w[1]])
    assert np.allclose(T[0], np.array([float(v) for v in d["abs_sum_unscaled"]]) * scale, rtol=0, atol=0)


@pytest.mark.parametrize("K", [16, 32, 256])
def test_bruteforce_rational_dot_tiny(K):
    rng = np.random.default_rng(K)
    M, N = 9, 13
    a_c, a_s = random_operand(rng, M, K, 0x01, 0x7F)
    w_c, w_s = random_operand(rng, N, K, 0x01, 0x7F)
    g_a, g_w = np.float32(0.37), np.array([1.5, 0.0625], dtype=np.float32)
    bounds = [0, 5, N]
    y, T = oracle.gemm_rows(a_c, a_s, g_a, w_c, w_s, bounds, g_w, np.arange(M))
    A, W = decode(a_c, a_s), decode(w_c, w_s)
    for m in range(M):
        for n in range(N):
            gw = g_w[0] if n < 5 else g_w[1]
            exact = sum(Fraction(A[m, k]) * Fraction(W[n, k]) for k in range(K))
            exact *= Fraction(float(g_a)) * Fraction(float(gw))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
            tabs = sum(abs(Fraction(A[m, k]) * Fraction(W[n, k])) for k in range(K))
            tabs *= Fraction(float(g_a)) * Fraction(float(gw))
            assert abs(Fraction(T[m, n]) - tabs) <= tabs * Fraction(1, 2 ** 50)


def test_bruteforce_double_triple_loop_equals_exact():
    # at these sizes a plain double triple loop is itself exact
    rng = np.random.default_rng(1)
    M, N, K = 4, 6, 32
    a_c, a_s = random_operand(rng, M, K)
    w_c, w_s = random_operand(rng, N, K)
    y, _ = oracle.gemm_rows(a_c, a_s, np.float32(1.0), w_c, w_s, [0, N], np.ones(1, np.float32), np.arange(M))
    A, W = decode(a_c, a_s), decode(w_c, w_s)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += A[m, k] * W[n, k]
            assert y[m, n] == acc


@pytest.mark.parametrize("K", [512, 5120])
def test_numpy_float64_matmul(K):
    rng = np.random.default_rng(K + 1)
    M, N = 8, 40
    a_c, a_s = random_operand(rng, M, K, 0x01, 0x7F)
    w_c, w_s = random_operand(rng, N, K, 0x01, 0x7F)
    g_a = np.float32(0.011)
    g_w = np.array([0.5, 2.0, 0.03], dtype=np.float32)
    bounds = [0, 16, 32, N]
    y, T = oracle.gemm_rows(a_c, a_s, g_a, w_c, w_s, bounds, g_w, np.arange(M))
    gcol = np.repeat(g_w.astype(np.float64), np.diff(bounds))
    ref = (decode(a_c, a_s) @ decode(w_c, w_s).T) * float(g_a) * gcol[None, :]
    assert (np.abs(y - ref) <= 2.0 ** -40 * T).all()
    tref = (np.abs(decode(a_c, a_s)) @ np.abs(decode(w_c, w_s)).T) * float(g_a) * gcol[None, :]
    assert np.allclose(T, tref, rtol=1e-12, atol=0)


def test_special_operands():
    K, N = 64, 8
    rng = np.random.default_rng(2)
    w_c, w_s = random_operand(rng, N, K)
    W = decode(w_c, w_s)
    # one-hot A: element k0 = 1.0 (code 2, scale 1.0), all others zero -> y = W[:, k0]
    for k0 in [0, 1, 17, 63]:
        a_c = np.zeros((1, K // 2), np.uint8)
        a_c[0, k0 // 2] = 2 << (4 * (k0 % 2))
        a_s = np.full((1, K // 16), 0x38, np.uint8)
        y, _ = oracle.gemm_rows(a_c, a_s, np.float32(1.0), w_c, w_s, [0, N], np.ones(1, np.float32), [0])
        assert (y[0] == W[:, k0]).all()
    # zero rows of A give exactly zero (codes 0 with any scale, or scale 0 with any code)
    a_c = np.zeros((2, K // 2), np.uint8)
    a_s = np.full((2, K // 16), 0x55, np.uint8)
    a_c[1] = 0x77
    a_s[1] = 0
    y, T = oracle.gemm_rows(a_c, a_s, np.float32(3.0), w_c, w_s, [0, N], np.ones(1, np.float32), [0, 1])
    assert (y == 0).all() and (T == 0).all()
    # selector W: row n has a single nonzero code 1.0 at column p(n) -> y[:, n] = A[:, p(n)]
    M = 5
    a_c, a_s = random_operand(rng, M, K)
    A = decode(a_c, a_s)
    perm = rng.permutation(K)[:N]
    sw_c = np.zeros((N, K // 2), np.uint8)
    for n, p in enumerate(perm):
        sw_c[n, p // 2] = 2 << (4 * (p % 2))
    sw_s = np.full((N, K // 16), 0x38, np.uint8)
    y, _ = oracle.gemm_rows(a_c, a_s, np.float32(1.0), sw_c, sw_s, [0, N], np.ones(1, np.float32), np.arange(M))
    assert (y == A[:, perm]).all()


def test_fused_equals_unfused_segments():
    rng = np.random.default_rng(4)
    K, M = 128, 6
    sizes = [16, 32, 8, 24]
    g_w = np.array([0.2, 1.7, 0.05, 3.0], dtype=np.float32)
    ws = [random_operand(rng, n, K) for n in sizes]
    a_c, a_s = random_operand(rng, M, K)
    g_a = np.float32(0.9)
    w_c = np.concatenate([w[0] for w in ws])
    w_s = np.concatenate([w[1] for w in ws])
    bounds = np.concatenate([[0], np.cumsum(sizes)])
    y, T = oracle.gemm_rows(a_c, a_s, g_a, w_c, w_s, bounds, g_w, np.arange(M))
    parts = [oracle.gemm_rows(a_c, a_s, g_a, wc, wsc, [0, n], g_w[i:i + 1], np.arange(M))
             for i, ((wc, wsc), n) in enumerate(zip(ws, sizes))]
    assert (y == np.concatenate([p[0] for p in parts], axis=1)).all()
    assert (T == np.concatenate([p[1] for p in parts], axis=1)).all()


def test_single_global_scale_reproduces_the_fused_module_trap():
    """Serving a fused GEMM with one module's global scale mis-scales the other module by the ratio
    of their global scales (the pages' "Trap 1"); the per-segment epilogue removes it."""
    rng = np.random.default_rng(6)
    K, M = 256, 4
    w1, w2 = random_operand(rng, 16, K), random_operand(rng, 16, K)
    a_c, a_s = random_operand(rng, M, K)
    g_w = np.array([0.01, 0.0275], dtype=np.float32)  # ratio 2.75
    w_c, w_s = np.concatenate([w1[0], w2[0]]), np.concatenate([w1[1], w2[1]])
    good, _ = oracle.gemm_rows(a_c, a_s, np.float32(1), w_c, w_s, [0, 16, 32], g_w, np.arange(M))
    bad, _ = oracle.gemm_rows(a_c, a_s, np.float32(1), w_c, w_s, [0, 32], g_w[:1], np.arange(M))
    rel = np.abs(bad[:, 16:] - good[:, 16:]).sum() / np.abs(good[:, 16:]).sum()
    assert abs(rel - (1 - 0.01 / 0.0275)) < 1e-6
    assert (bad[:, :16] == good[:, :16]).all()
