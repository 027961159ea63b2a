"""Pins of the float64 oracle to things other than itself.

Each test checks the oracle against a closed form, a brute-force expansion,
a library routine, an invariant, or a value worked out by hand. The aim is
that a plausible slip in the oracle fails at least one of them: a dropped
term, the sign of the exponent, a transposed operand, or the gate's position.
All of these run on the CPU.
"""

import os

import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, Bt=2, L=9, d=3, N=4, h0=True, gate=True, dscale=0.3):
    u = rng.standard_normal((Bt, L, d))
    delta = rng.standard_normal((Bt, L, d)) * 0.5
    bias = rng.uniform(-2.0, 0.5, d)
    A = -rng.uniform(0.2, 3.0, (d, N))
    B = rng.standard_normal((Bt, L, N))
    C = rng.standard_normal((Bt, L, N))
    D = rng.standard_normal(d)
    z = rng.standard_normal((Bt, L, d)) if gate else None
    h0v = rng.standard_normal((Bt, d, N)) * dscale if h0 else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, delta_bias=bias,
                delta_softplus=True, h0=h0v)


def np_softplus(x):
    return np.logaddexp(0.0, x)


def np_silu(z):
    return z * expit(z)


# ------------------------------------------------------------------ brute force

def brute_force(c):
    """h_t = e^{A S_t} h0 + sum_{s<=t} e^{A (S_t - S_s)} dt_s B_s u_s, S = cumsum dt.

    O(L^2) unrolled form of the recurrence: no loop-carried state at all.
    """
    dt = np_softplus(c["delta"] + c["delta_bias"])           # [Bt, L, d]
    S = np.cumsum(dt, axis=1)                                 # inclusive
    Bt, L, d = c["u"].shape
    N = c["A"].shape[1]
    A = c["A"]
    h0 = c["h0"] if c["h0"] is not None else np.zeros((Bt, d, N))
    hs = np.zeros((Bt, L, d, N))
    for t in range(L):
        acc = np.exp(A[None] * S[:, t, :, None]) * h0
        for s in range(t + 1):
            w = np.exp(A[None] * (S[:, t, :, None] - S[:, s, :, None]))
            acc = acc + w * (dt[:, s, :, None] * c["B"][:, s, None, :] * c["u"][:, s, :, None])
        hs[:, t] = acc
    y = np.einsum("bldn,bln->bld", hs, c["C"]) + c["D"] * c["u"]
    if c["z"] is not None:
        y = y * np_silu(c["z"])
    return y, hs[:, -1]


def test_bruteforce_unrolled_sum():
    rng = np.random.default_rng(1)
    for gate in (True, False):
        c = rand_case(rng, gate=gate)
        y, h = oracle.selective_scan(**c)
        yb, hb = brute_force(c)
        np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(h, hb, rtol=1e-12, atol=1e-13)


def test_single_step_closed_form():
    """L = 1: y = (sum_n C (e^{dt A} h0 + dt B u) + D u) silu(z)."""
    rng = np.random.default_rng(2)
    c = rand_case(rng, Bt=3, L=1, d=5, N=7)
    y, h = oracle.selective_scan(**c)
    dt = np_softplus(c["delta"][:, 0] + c["delta_bias"])      # [Bt, d]
    hc = np.exp(dt[..., None] * c["A"]) * c["h0"] + dt[..., None] * c["B"][:, 0, None, :] * c["u"][:, 0, :, None]
    yc = (np.einsum("bdn,bn->bd", hc, c["C"][:, 0]) + c["D"] * c["u"][:, 0]) * np_silu(c["z"][:, 0])
    np.testing.assert_allclose(h, hc, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[:, 0], yc, rtol=1e-13, atol=1e-14)


def test_zero_step_keeps_state():
    """delta == 0 (softplus off): the state never moves, y_t = C_t h0 + D u_t."""
    rng = np.random.default_rng(3)
    c = rand_case(rng, gate=False)
    c["delta"] = np.zeros_like(c["delta"])
    c["delta_bias"] = None
    c["delta_softplus"] = False
    y, h = oracle.selective_scan(**c)
    assert np.array_equal(h, c["h0"])
    yc = np.einsum("bdn,bln->bld", c["h0"], c["C"]) + c["D"] * c["u"]
    np.testing.assert_allclose(y, yc, rtol=1e-14, atol=1e-15)


def test_small_step_derivative_sign():
    """(h1 - h0)/dt -> A h0 + B u as dt -> 0. Catches exp(-dt A) and dropped dt."""
    rng = np.random.default_rng(4)
    c = rand_case(rng, L=1, gate=False)
    eps = 1e-7
    c["delta"] = np.full_like(c["delta"], eps)
    c["delta_bias"] = None
    c["delta_softplus"] = False
    _, h1 = oracle.selective_scan(**c)
    deriv = (h1 - c["h0"]) / eps
    expect = c["A"][None] * c["h0"] + c["B"][:, 0, None, :] * c["u"][:, 0, :, None]
    np.testing.assert_allclose(deriv, expect, rtol=2e-5, atol=2e-6)
    # A < 0 is stable: with no input the state decays.
    c["u"] = np.zeros_like(c["u"])
    c["delta"] = np.full_like(c["delta"], 0.5)
    _, h1 = oracle.selective_scan(**c)
    assert np.all(np.abs(h1) < np.abs(c["h0"]))


# ------------------------------------------------------------------ associative operator

def combine(e, l):
    """(A_i, b_i) (+) (A_j, b_j) = (A_j A_i, A_j b_i + b_j), i earlier than j.

    The operator of "Mamba的隐藏代价" (kongchang.com), section on sequential
    gradients; diagonal A makes A_j A_i elementwise.
    """
    Ai, bi = e
    Aj, bj = l
    return Aj * Ai, Aj * bi + bj


def tree_fold(items):
    if len(items) == 1:
        return items[0]
    m = len(items) // 2
    return combine(tree_fold(items[:m]), tree_fold(items[m:]))


def random_fold(items, rng):
    items = list(items)
    while len(items) > 1:
        k = rng.integers(0, len(items) - 1)
        items[k:k + 2] = [combine(items[k], items[k + 1])]
    return items[0]


def test_associative_combine_equals_sequential():
    rng = np.random.default_rng(5)
    c = rand_case(rng, Bt=2, L=13, d=3, N=5)
    _, h = oracle.selective_scan(**c)
    dt = np_softplus(c["delta"] + c["delta_bias"])
    pairs = [(np.exp(dt[:, t, :, None] * c["A"][None]),
              dt[:, t, :, None] * c["B"][:, t, None, :] * c["u"][:, t, :, None])
             for t in range(c["u"].shape[1])]
    for fold in (tree_fold(pairs), random_fold(pairs, rng), random_fold(pairs, rng)):
        P, b = fold
        np.testing.assert_allclose(P * c["h0"] + b, h, rtol=1e-12, atol=1e-14)
        # The product of the transitions is exp(A * total step).
        np.testing.assert_allclose(P, np.exp(c["A"][None] * dt.sum(axis=1)[..., None]), rtol=1e-12)


# ------------------------------------------------------------------ library routines

def test_time_invariant_case_is_a_convolution():
    """Constant dt, B, C: y = (K * u)[:L] + D u, K_k = sum_n C_n e^{k dt A_n} dt B_n."""
    rng = np.random.default_rng(6)
    L, d, N = 40, 3, 6
    dt = rng.uniform(0.05, 0.4, d)
    A = -rng.uniform(0.1, 2.0, (d, N))
    Bc = rng.standard_normal(N)
    Cc = rng.standard_normal(N)
    u = rng.standard_normal((1, L, d))
    D = rng.standard_normal(d)
    y, _ = oracle.selective_scan(u, np.broadcast_to(dt, (1, L, d)), A,
                                 np.broadcast_to(Bc, (1, L, N)), np.broadcast_to(Cc, (1, L, N)), D=D)
    k = np.arange(L)
    for ch in range(d):
        K = (Cc[None, :] * np.exp(k[:, None] * dt[ch] * A[ch][None, :]) * dt[ch] * Bc[None, :]).sum(axis=1)
        yc = np.convolve(K, u[0, :, ch])[:L] + D[ch] * u[0, :, ch]
        np.testing.assert_allclose(y[0, :, ch], yc, rtol=1e-11, atol=1e-12)


def test_one_state_constant_step_is_an_iir_filter():
    """N = 1, constant dt and B: h = lfilter([dt B], [1, -e^{dt A}], u)."""
    rng = np.random.default_rng(7)
    L = 200
    dt, A, Bc, Cc = 0.07, -1.3, 0.8, -1.7
    u = rng.standard_normal(L)
    y, h = oracle.selective_scan(u[None, :, None], np.full((1, L, 1), dt), np.array([[A]]),
                                 np.full((1, L, 1), Bc), np.full((1, L, 1), Cc))
    hf = lfilter([dt * Bc], [1.0, -np.exp(dt * A)], u)
    np.testing.assert_allclose(y[0, :, 0], Cc * hf, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(h[0, 0, 0], hf[-1], rtol=1e-12)


def test_softplus_and_silu_closed_forms():
    x = np.concatenate([np.linspace(-60, 60, 2001), [-745.0, -40.0, 0.0, 40.0, 700.0]])
    np.testing.assert_allclose(oracle.softplus(x), np.logaddexp(0.0, x), rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)
    assert np.isnan(oracle.silu(np.array([np.nan]))[0])


# ------------------------------------------------------------------ decode

def test_decode_repeated_token_geometric_closed_form():
    """k re-applications of one token: s_k = e^{k dt A} s0 + dt B x expm1(k dt A)/expm1(dt A)."""
    rng = np.random.default_rng(8)
    Bt, d, N, k = 3, 4, 5, 60
    s0 = rng.standard_normal((Bt, d, N)) * 0.1
    x = rng.standard_normal((Bt, d))
    dr = rng.standard_normal((Bt, d))
    bias = rng.uniform(-3, 0, d)
    A = -rng.uniform(0.1, 2, (d, N))
    Bm = rng.standard_normal((Bt, N))
    Cm = rng.standard_normal((Bt, N))
    D = rng.standard_normal(d)
    z = rng.standard_normal((Bt, d))
    s = s0
    for _ in range(k):
        y, s = oracle.selective_state_update(s, x, dr, A, Bm, Cm, D=D, z=z, delta_bias=bias, delta_softplus=True)
    dt = np_softplus(dr + bias)[..., None]
    q = dt * A[None]
    sk = np.exp(k * q) * s0 + dt * Bm[:, None, :] * x[..., None] * np.expm1(k * q) / np.expm1(q)
    np.testing.assert_allclose(s, sk, rtol=1e-12, atol=1e-14)
    yk = ((sk * Cm[:, None, :]).sum(-1) + D * x) * np_silu(z)
    np.testing.assert_allclose(y, yk, rtol=1e-11, atol=1e-13)


def test_scan_then_decode_equals_longer_scan():
    rng = np.random.default_rng(9)
    c = rand_case(rng, L=12)
    y, h = oracle.selective_scan(**c)
    c1 = dict(c)
    for key in ("u", "delta", "B", "C", "z"):
        c1[key] = c[key][:, :-1]
    _, h_prev = oracle.selective_scan(**c1)
    yd, sd = oracle.selective_state_update(h_prev, c["u"][:, -1], c["delta"][:, -1], c["A"],
                                           c["B"][:, -1], c["C"][:, -1], D=c["D"], z=c["z"][:, -1],
                                           delta_bias=c["delta_bias"], delta_softplus=True)
    np.testing.assert_allclose(sd, h, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(yd, y[:, -1], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ invariants

def test_split_invariance():
    rng = np.random.default_rng(10)
    c = rand_case(rng, L=17)
    y, h = oracle.selective_scan(**c)
    for L1 in (1, 8, 16):
        a = dict(c)
        b = dict(c)
        for key in ("u", "delta", "B", "C", "z"):
            a[key] = c[key][:, :L1]
            b[key] = c[key][:, L1:]
        ya, ha = oracle.selective_scan(**a)
        b["h0"] = ha
        yb, hb = oracle.selective_scan(**b)
        np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(hb, h, rtol=1e-13, atol=1e-15)


def test_linearity_in_u_from_zero_state():
    rng = np.random.default_rng(11)
    c = rand_case(rng, h0=False)
    u1 = c["u"]
    u2 = rng.standard_normal(u1.shape)
    c1, c2, c3 = dict(c), dict(c), dict(c)
    c1["u"], c2["u"], c3["u"] = u1, u2, 2.5 * u1 - 0.75 * u2
    y1, _ = oracle.selective_scan(**c1)
    y2, _ = oracle.selective_scan(**c2)
    y3, _ = oracle.selective_scan(**c3)
    np.testing.assert_allclose(y3, 2.5 * y1 - 0.75 * y2, rtol=1e-11, atol=1e-13)


def test_causality():
    rng = np.random.default_rng(12)
    c = rand_case(rng, L=15)
    y, _ = oracle.selective_scan(**c)
    t = 6
    c2 = dict(c)
    for key in ("u", "delta", "B", "C", "z"):
        v = c[key].copy()
        v[:, t + 1:] = rng.standard_normal(v[:, t + 1:].shape)
        c2[key] = v
    y2, _ = oracle.selective_scan(**c2)
    assert np.array_equal(y[:, :t + 1], y2[:, :t + 1])
    assert not np.allclose(y[:, t + 1:], y2[:, t + 1:])


def test_magnitude_companion_bounds():
    rng = np.random.default_rng(13)
    c = rand_case(rng, L=20)
    y, h, ym, hm = oracle.selective_scan(**c, want_magnitude=True)
    assert np.all(np.abs(y) <= ym * (1 + 1e-14))
    assert np.all(np.abs(h) <= hm * (1 + 1e-14))
    # With every term non-negative the bound is attained.
    cp = dict(c)
    for key in ("u", "B", "C", "z"):
        cp[key] = np.abs(c[key])
    cp["D"] = np.abs(c["D"])
    cp["h0"] = np.abs(c["h0"])
    y, h, ym, hm = oracle.selective_scan(**cp, want_magnitude=True)
    np.testing.assert_allclose(y, ym, rtol=1e-14)
    np.testing.assert_allclose(h, hm, rtol=1e-14)
    yd, sd, ydm, sdm = oracle.selective_state_update(c["h0"], c["u"][:, 0], c["delta"][:, 0], c["A"],
                                                     c["B"][:, 0], c["C"][:, 0], D=c["D"], z=c["z"][:, 0],
                                                     delta_bias=c["delta_bias"], delta_softplus=True,
                                                     want_magnitude=True)
    assert np.all(np.abs(yd) <= ydm * (1 + 1e-14)) and np.all(np.abs(sd) <= sdm * (1 + 1e-14))


def test_empty_sequence():
    rng = np.random.default_rng(14)
    c = rand_case(rng, L=0)
    y, h = oracle.selective_scan(**c)
    assert y.shape == (2, 0, 3)
    assert np.array_equal(h, c["h0"])


def test_scaled_error_metric():
    ref = np.array([1.0, -2.0, 0.0, np.nan])
    mag = np.array([2.0, 4.0, 0.0, 1.0])
    assert oracle.scaled_error(ref, ref, mag) == 0.0
    got = np.array([1.5, -2.0, 0.0, np.nan])
    assert oracle.scaled_error(got, ref, mag) == pytest.approx(0.25)
    got = np.array([1.0, -2.0, 1e-30, np.nan])
    assert oracle.scaled_error(got, ref, mag) == np.inf
    got = np.array([1.0, -2.0, 0.0, 0.0])
    assert oracle.scaled_error(got, ref, mag) == np.inf


# ------------------------------------------------------------------ hand-worked golden values

def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            vals[k] = np.array([float(x) for x in v])
    return vals


def test_golden_scalar_scan():
    g = read_golden("scalar_scan_worked.txt")
    L = len(g["u"])
    y, h = oracle.selective_scan(g["u"].reshape(1, L, 1), g["delta"].reshape(1, L, 1),
                                 g["A"].reshape(1, 1), g["B"].reshape(1, L, 1), g["C"].reshape(1, L, 1),
                                 D=g["D"])
    np.testing.assert_allclose(y[0, :, 0], g["y"], rtol=1e-14)
    np.testing.assert_allclose(h[0, 0, 0], g["h"][-1], rtol=1e-14)
    # Every intermediate state: scan prefixes.
    for t in range(L):
        _, ht = oracle.selective_scan(g["u"][:t + 1].reshape(1, -1, 1), g["delta"][:t + 1].reshape(1, -1, 1),
                                      g["A"].reshape(1, 1), g["B"][:t + 1].reshape(1, -1, 1),
                                      g["C"][:t + 1].reshape(1, -1, 1), D=g["D"])
        assert ht[0, 0, 0] == pytest.approx(g["h"][t], rel=1e-14)


def test_golden_gated_decode():
    g = read_golden("gated_decode_worked.txt")
    N = len(g["A"])
    y, s = oracle.selective_state_update(g["state"].reshape(1, 1, N), g["x"].reshape(1, 1), g["delta"].reshape(1, 1),
                                         g["A"].reshape(1, N), g["B"].reshape(1, N), g["C"].reshape(1, N),
                                         D=g["D"], z=g["z"].reshape(1, 1))
    np.testing.assert_allclose(s[0, 0], g["state_new"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[0, 0], g["y"][0], rtol=1e-14)
