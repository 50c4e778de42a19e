"""Pins for the oracle's Gated DeltaNet recurrence S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T,
o_t = S_t^T q_t: the delta rule's write-then-read property, closed forms of one step and of pure decay,
an independent chunked (triangular-solve) formulation of the same recurrence, continuity of the state
across calls, and the sharing of key heads between value heads."""
import numpy as np
import pytest

import oracle
import workloads as wl


def bf16(a):
    return wl.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def val(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def small_case(rng, B, T, Hv, Hk, D, unit=True):
    def heads(n):
        x = rng.standard_normal((B * T, n, D))
        if unit:
            x /= np.linalg.norm(x, axis=2, keepdims=True)
        return bf16(x.reshape(B * T, n * D))
    q, k = heads(Hk), heads(Hk)
    v = bf16(rng.standard_normal((B * T, Hv * D)))
    alpha = rng.uniform(0.5, 1.0, (B * T, Hv)).astype(np.float32)
    beta = rng.uniform(0.05, 1.0, (B * T, Hv)).astype(np.float32)
    return q, k, v, alpha, beta


def test_write_then_read_with_one_hot_keys():
    """alpha = beta = 1 and k = e_i: the update stores v_t under key e_i, so reading with q = k
    returns v_t exactly, whatever was stored before."""
    D, T = 16, 40
    rng = np.random.default_rng(0)
    idx = rng.integers(0, D, T)
    k = np.zeros((T, D), np.float32)
    k[np.arange(T), idx] = 1
    v = bf16(rng.standard_normal((T, D)))
    ones = np.ones((T, 1), np.float32)
    o, _ = oracle.gdn_recurrence(bf16(k), bf16(k), v, ones, ones, 1, T, D=D)
    assert (o == val(v)).all()


def test_one_step_closed_form():
    """From a random S0 with q = k: o = alpha S0^T k + beta (v - S0^T k) |k|^2, and
    S1 = alpha S0 + beta k (v - S0^T k)^T."""
    D = 32
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((1, 1, D, D))
    k = bf16(rng.standard_normal((1, D)) * 0.2)
    v = bf16(rng.standard_normal((1, D)))
    a, b = np.float32(0.8), np.float32(0.3)
    o, S = oracle.gdn_recurrence(k, k, v, np.array([[a]]), np.array([[b]]), 1, 1, D=D, S0=S0)
    kv, vv, s0 = val(k)[0], val(v)[0], S0[0, 0]
    sk = s0.T @ kv
    S1 = float(a) * s0 + float(b) * np.outer(kv, vv - sk)
    assert np.allclose(S[0, 0], S1, rtol=1e-13, atol=1e-13)
    want = float(a) * sk + float(b) * (vv - sk) * (kv @ kv)
    assert np.allclose(o[0], want, rtol=1e-12, atol=1e-12)


def test_pure_decay():
    """beta = 0: the state only decays, S_t = (prod alpha) S0 and o_t = S_t^T q_t."""
    D, T = 16, 25
    rng = np.random.default_rng(2)
    q, k, v, alpha, _ = small_case(rng, 1, T, 1, 1, D)
    S0 = rng.standard_normal((1, 1, D, D))
    o, S = oracle.gdn_recurrence(q, k, v, alpha, np.zeros_like(alpha), 1, T, D=D, S0=S0)
    g = np.cumprod(alpha[:, 0].astype(np.float64))
    assert np.allclose(S[0, 0], g[-1] * S0[0, 0], rtol=1e-13)
    want = g[:, None] * (val(q) @ S0[0, 0])
    assert np.allclose(o, want, rtol=1e-12, atol=1e-14)


def chunked(q, k, v, alpha, beta, T, D, C):
    """The recurrence for one head written chunk by chunk (C tokens): within a chunk the deltas
    u_t = v_t - S_{t-1}^T k_t solve a unit lower-triangular system, with P(t, j) = prod_{j < i <= t}
    alpha_i:  u_t + sum_{j<t} P(t-1, j) beta_j (k_t . k_j) u_j = v_t - P(t-1, start) S0^T k_t;
    then o_t = P(t, start) S0^T q_t + sum_{j<=t} P(t, j) beta_j (q_t . k_j) u_j and
    S_end = P(end, start) S0 + sum_j P(end, j) beta_j k_j u_j^T."""
    S = np.zeros((D, D))
    out = np.zeros((T, D))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        K, Q, V = k[c0:c0 + n], q[c0:c0 + n], v[c0:c0 + n]
        a, b = alpha[c0:c0 + n], beta[c0:c0 + n]
        logp = np.concatenate([[0.0], np.cumsum(np.log(a))])  # logp[t+1] = log prod_{i<=t} a_i

        def P(t, j):  # prod_{j < i <= t} alpha_i, with j = -1 meaning the chunk start
            return np.exp(logp[t + 1] - logp[j + 1])
        A = K @ K.T
        R = V - np.array([P(t - 1, -1) for t in range(n)])[:, None] * (K @ S)
        L = np.zeros((n, n))
        for t in range(n):
            for j in range(t):
                L[t, j] = P(t - 1, j) * b[j] * A[t, j]
        U = np.linalg.solve(np.eye(n) + L, R)
        Bm = Q @ K.T
        for t in range(n):
            acc = P(t, -1) * (Q[t] @ S)
            for j in range(t + 1):
                acc = acc + P(t, j) * b[j] * Bm[t, j] * U[j]
            out[c0 + t] = acc
        S = P(n - 1, -1) * S + sum(P(n - 1, j) * b[j] * np.outer(K[j], U[j]) for j in range(n))
    return out, S


def test_independent_chunked_formulation():
    D, T = 16, 45
    rng = np.random.default_rng(3)
    q, k, v, alpha, beta = small_case(rng, 1, T, 1, 1, D)
    o, S = oracle.gdn_recurrence(q, k, v, alpha, beta, 1, T, D=D)
    oc, Sc = chunked(val(q), val(k), val(v), alpha[:, 0].astype(np.float64), beta[:, 0].astype(np.float64), T, D, 16)
    assert np.allclose(o, oc, rtol=1e-10, atol=1e-12)
    assert np.allclose(S[0, 0], Sc, rtol=1e-10, atol=1e-12)


def test_state_carries_across_calls_and_heads_share_keys():
    D, T1, T2, Hv, Hk = 16, 7, 9, 4, 2
    rng = np.random.default_rng(4)
    q, k, v, alpha, beta = small_case(rng, 1, T1 + T2, Hv, Hk, D)
    o, S = oracle.gdn_recurrence(q, k, v, alpha, beta, 1, T1 + T2, D=D)
    o1, S1 = oracle.gdn_recurrence(q[:T1], k[:T1], v[:T1], alpha[:T1], beta[:T1], 1, T1, D=D)
    o2, S2 = oracle.gdn_recurrence(q[T1:], k[T1:], v[T1:], alpha[T1:], beta[T1:], 1, T2, D=D, S0=S1)
    assert (np.concatenate([o1, o2]) == o).all() and (S2 == S).all()
    # value heads 0 and 1 read key head 0: with equal v, alpha, beta they give equal outputs
    v2, a2, b2 = v.copy(), alpha.copy(), beta.copy()
    v2[:, D:2 * D], a2[:, 1], b2[:, 1] = v2[:, :D], a2[:, 0], b2[:, 0]
    o3, _ = oracle.gdn_recurrence(q, k, v2, a2, b2, 1, T1 + T2, D=D)
    assert (o3[:, :D] == o3[:, D:2 * D]).all()
    assert not np.allclose(o3[:, 2 * D:3 * D], o3[:, :D])


@pytest.mark.parametrize("B,T", [(2, 64), (1, 300)])
def test_float32_twin_tracks_double(B, T):
    case = wl.GdnCase("t", 99, B, T, Hv=4, Hk=2, D=32)
    q, k, v, alpha, beta = wl.draw_gdn(case)
    o, S = oracle.gdn_recurrence(q, k, v, alpha, beta, B, T, D=32)
    o32, S32 = oracle.gdn_recurrence(q, k, v, alpha, beta, B, T, D=32, f32=True)
    assert np.abs(o32 - o).max() <= 1e-4 * np.abs(o).max()
    assert np.abs(S32 - S).max() <= 1e-4 * np.abs(S).max()
