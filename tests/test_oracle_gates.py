"""Pins for the oracle's gate epilogues (CPU only).

The gates come from the Gated DeltaNet parameterization the pages give (Japanese article,
"Mechanism 2"): the decay exponent g = -exp(A_log) * softplus(a + dt_bias), the decay alpha = exp(g),
and the write strength beta = sigmoid(b). Pinned by closed forms and identities that tie the
decay to the sigmoid through different code paths.
"""
import math

import numpy as np

import oracle


def test_closed_forms():
    assert oracle.sigmoid_scalar(0.0) == 0.5
    assert oracle.softplus(0.0) == math.log(2.0)
    assert abs(oracle.gdn_decay_scalar(0.0, 0.0, 0.0) - 0.5) < 1e-16
    # alpha -> 1 as y + dt_bias -> -inf, alpha -> 0 as it -> +inf
    assert oracle.gdn_decay_scalar(-800.0, 0.3, 0.0) == 1.0
    assert oracle.gdn_decay_scalar(800.0, 0.0, 0.0) == 0.0
    assert oracle.sigmoid_scalar(-800.0) == 0.0 and oracle.sigmoid_scalar(800.0) == 1.0


def test_decay_identities():
    z = np.linspace(-30, 30, 241)
    y = z[None, :]
    # A_log = 0: alpha = 1 / (1 + e^z) = sigmoid(-z)
    # (exp of an argument of size |z| carries a relative rounding error of about |z| * 2^-53)
    tol = 4e-16 * (1 + np.abs(z))
    alpha = oracle.gdn_decay(y, np.zeros(z.size, np.float32), np.zeros(z.size, np.float32))
    assert (np.abs(alpha[0] - oracle.sigmoid(-z)) <= tol * oracle.sigmoid(-z)).all()
    # A_log = ln 2 (as float32): alpha = sigmoid(-z) ^ exp(A_log)
    al = np.float32(math.log(2.0))
    alpha2 = oracle.gdn_decay(y, np.full(z.size, al, np.float32), np.zeros(z.size, np.float32))
    assert np.allclose(alpha2[0], oracle.sigmoid(-z) ** math.exp(float(al)), rtol=1e-14, atol=1e-300)
    # dt_bias shifts the argument
    dt = np.float32(0.75)
    alpha3 = oracle.gdn_decay(y, np.zeros(z.size, np.float32), np.full(z.size, dt, np.float32))
    ref3 = oracle.sigmoid(-(z + float(dt)))
    assert (np.abs(alpha3[0] - ref3) <= 4e-16 * (2 + np.abs(z)) * ref3).all()


def test_softplus_identity_and_stability():
    for z in [-50.0, -3.0, -1e-8, 0.0, 1e-8, 2.5, 40.0, 700.0]:
        assert abs(oracle.softplus(z) - oracle.softplus(-z) - z) <= 1e-15 * max(1.0, abs(z))
    assert oracle.softplus(1000.0) == 1000.0
    assert 0 < oracle.softplus(-700.0) < 1e-300


def test_sigmoid_symmetry():
    y = np.linspace(-40, 40, 161)
    s = oracle.sigmoid(y)
    assert np.allclose(s + oracle.sigmoid(-y), 1.0, rtol=0, atol=4.5e-16)
