"""Pins of the exact zero-order-hold option of the oracle (input coefficient
(exp(dt A) - 1) / A) against library discretisation, an ODE integrator, and
its limits. CPU only."""

import numpy as np
from scipy import integrate, signal

from oracle import input_coefficient, selective_scan, selective_state_update


def test_matches_scipy_zoh_discretisation():
    """Constant step, one state: the scan is an IIR filter whose coefficients
    are scipy's zero-order-hold discretisation of dh/dt = A h + B u."""
    A, b, dt, L = -0.7, 1.3, 0.37, 40
    Ad, Bd, _, _, _ = signal.cont2discrete((np.array([[A]]), np.array([[b]]), np.eye(1), np.zeros((1, 1))),
                                           dt, method="zoh")
    u = np.random.default_rng(0).standard_normal(L)
    y, _ = selective_scan(u.reshape(1, L, 1), np.full((1, L, 1), dt), np.array([[A]]),
                          np.full((1, L, 1), b), np.ones((1, L, 1)), zoh=True)
    ref = signal.lfilter([Bd[0, 0]], [1.0, -Ad[0, 0]], u)
    np.testing.assert_allclose(y[0, :, 0], ref, rtol=1e-12, atol=1e-13)


def test_exact_for_piecewise_constant_input():
    """Varying steps and inputs: the state at each step end equals the exact
    solution of dh/dt = A h + B_l u_l over [t_{l-1}, t_l] (held input)."""
    r = np.random.default_rng(1)
    L, N = 12, 3
    A = -np.array([0.3, 1.1, 4.0])
    dt = np.exp(r.uniform(np.log(0.01), np.log(0.5), L))
    u = r.standard_normal(L)
    Bm = r.standard_normal((L, N))
    h = np.zeros(N)
    for l in range(L):
        sol = integrate.solve_ivp(lambda t, y: A * y + Bm[l] * u[l], (0.0, dt[l]), h, rtol=1e-12, atol=1e-14)
        h = sol.y[:, -1]
    _, hf = selective_scan(u.reshape(1, L, 1), dt.reshape(1, L, 1), A.reshape(1, N), Bm.reshape(1, L, N),
                           np.ones((1, L, N)), zoh=True)
    np.testing.assert_allclose(hf[0, 0], h, rtol=1e-9, atol=1e-12)


def test_limits():
    dt = np.array([[1e-3], [0.2]])
    A = np.array([[0.0, -1e-9, -2.0]])
    k = input_coefficient(dt, A, zoh=True)
    np.testing.assert_array_equal(k[:, 0], dt[:, 0])              # A = 0: the limit dt
    np.testing.assert_allclose(k[:, 1], dt[:, 0], rtol=1e-8)      # tiny A: close to dt
    np.testing.assert_allclose(k[:, 2], np.expm1(-2.0 * dt[:, 0]) / -2.0, rtol=1e-15)
    # small steps: ZOH and the simplified form agree to first order
    r = np.random.default_rng(2)
    args = [r.standard_normal((1, 30, 2)), np.full((1, 30, 2), 1e-5), -np.abs(r.standard_normal((2, 4))),
            r.standard_normal((1, 30, 4)), r.standard_normal((1, 30, 4))]
    y0, _ = selective_scan(*args)
    y1, _ = selective_scan(*args, zoh=True)
    np.testing.assert_allclose(y1, y0, rtol=1e-4, atol=1e-9)


def test_decode_uses_the_same_coefficient():
    r = np.random.default_rng(3)
    B, d, N = 2, 3, 4
    s0, x, dl = r.standard_normal((B, d, N)), r.standard_normal((B, d)), np.abs(r.standard_normal((B, d)))
    A, Bm, Cm = -np.abs(r.standard_normal((d, N))), r.standard_normal((B, N)), r.standard_normal((B, N))
    y, s = selective_state_update(s0, x, dl, A, Bm, Cm, zoh=True)
    ys, hs = selective_scan(x[:, None], dl[:, None], A, Bm[:, None], Cm[:, None], h0=s0, zoh=True)
    np.testing.assert_allclose(y, ys[:, 0], rtol=1e-14)
    np.testing.assert_allclose(s, hs, rtol=1e-14)
