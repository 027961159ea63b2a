"""Float64 NumPy oracle of the selective scan and the decode state update.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package's smoke check
and by the benchmark's CPU-baseline leg, never by the product path. It shares
no code with the HIP kernels or their binding. Source tags ([TtoM], [Notes],
[HiddenCost], [Paradigm], [Breakthrough]) are expanded in ``oracle/__init__.py``.

What it computes (per batch b, channel d, state n; time index l):

    delta[b,l,d] = softplus(delta_raw[b,l,d] + bias[d])   (or without softplus)
    Abar         = exp(delta * A[d,n])
    h            = Abar * h + delta * B[b,l,n] * u[b,l,d]
    y[b,l,d]     = (sum_n C[b,l,n] * h[n] + D[d] * u[b,l,d]) * silu(z[b,l,d])

Readings of the pages taken here (the pages disagree or are silent):

- The exponent is exp(delta * A) with A <= 0 passed in directly. One listing
  on [TtoM] negates the exponent while also negating A, which makes every
  step grow; the discretisation snippet in [TtoM] section 3.1 has no minus.
- B-bar x is delta * B * x (the simplified form both listings in [TtoM] use)
  by default; the exact zero-order-hold integral that [Breakthrough] section
  2.3 names, (exp(delta A) - 1) / A * B * x, is an option (``zoh=True``).
- The optional bias is added before softplus ([TtoM] section 5: the step-size
  projection has a bias and its output goes through softplus).
- The gate multiplies after the D skip: out = (C h + D u) * silu(z)
  ([TtoM] section 5, the block's gate branch; [Notes] "block structure").
- Absent D, bias, z or h0 mean 0, 0, no gate, and a zero initial state
  ([TtoM] section 5 starts the state at zero).

No step here is blocked, fused or reordered: one time step after another.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "softplus",
    "silu",
    "discretize_delta",
    "selective_scan",
    "selective_state_update",
    "input_coefficient",
    "scaled_error",
]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def softplus(x):
    """softplus(x) = log(1 + e^x), in the overflow-free form max(x,0) + log1p(e^-|x|).

    [TtoM] section 3 (selectivity snippet) and section 5 (the step size goes
    through softplus so that it is positive).
    """
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z), evaluated without overflow.

    [TtoM] section 5, MambaBlock: the gate branch z goes through SiLU and
    multiplies the scan output. [Notes] "block structure": the second branch
    gates the main branch after an activation.
    """
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    neg = ~pos
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[neg])
    out[neg] = z[neg] * ez / (1.0 + ez)
    nan = np.isnan(z)
    out[nan] = np.nan
    return out


def discretize_delta(delta_raw, delta_bias=None, delta_softplus=False):
    """Step size per (b, l, d): softplus(delta_raw + bias[d]) or delta_raw + bias[d].

    [TtoM] section 3 (delta depends on the input and passes through softplus)
    and section 5 (the step-size projection carries a bias; softplus follows).
    """
    dt = _f64(delta_raw)
    if delta_bias is not None:
        dt = dt + _f64(delta_bias)
    if delta_softplus:
        dt = softplus(dt)
    return dt


def input_coefficient(dt, A, zoh=False):
    """Coefficient k of the input term, B-bar x = k * B * x, per (.., d, n).

    Simplified form (default): k = dt, the form of both listings in [TtoM]
    (sections 3.1 and 5). Exact zero-order hold ([Breakthrough] section 二.3
    names ZOH; for a diagonal A the integral of exp(A s) over one step is
    closed-form): k = (exp(dt A) - 1) / A, and k = dt where A = 0 (the limit).
    dt: [..., d, 1] or broadcastable; A: [d, N].
    """
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    if not zoh:
        return np.broadcast_to(dt, np.broadcast_shapes(dt.shape, A.shape))
    x = dt * A
    safe_A = np.where(A == 0.0, 1.0, A)
    return np.where(A == 0.0, dt, np.expm1(x) / safe_A)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus=False, h0=None, want_magnitude=False, zoh=False):
    """Sequential selective scan in float64.

    Shapes follow the selective_scan docstring of [TtoM] section 3.1:
    u, delta, z: [Bt, L, d]; A: [d, N]; B, C: [Bt, L, N]; D, delta_bias: [d];
    h0: [Bt, d, N].

    The time loop follows the reference recurrence of [TtoM] section 5
    (SelectiveScan.forward): per step, the transition exp(delta*A), the input
    term delta*B*u, the state update, and the readout sum_n h*C; then the D
    skip. Discrete form: [TtoM] section 2, [Notes] "Selective State Space"
    (y_t = C_t h_t + D x_t), and [HiddenCost] "math foundations".

    Returns (y, h_final) or, with want_magnitude, (y, h_final, y_mag, h_mag):
    the magnitude companions run the same recurrence on absolute values,
    h_mag <- Abar*h_mag + |delta*B*u| from |h0|, and
    y_mag = (sum_n |C| h_mag + |D u|) * |silu(z)|, so |y| <= y_mag and
    |h| <= h_mag elementwise (triangle inequality). They scale the parity error.
    """
    u = _f64(u)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    Bt, L, d = u.shape
    N = A.shape[1]
    dt = discretize_delta(delta, delta_bias, delta_softplus)
    if h0 is None:
        h = np.zeros((Bt, d, N))
    else:
        h = _f64(h0).copy()
    y = np.zeros((Bt, L, d))
    if want_magnitude:
        h_mag = np.abs(h)
        y_mag = np.zeros((Bt, L, d))
    for l in range(L):
        dt_l = dt[:, l, :]                                   # [Bt, d]
        a = np.exp(dt_l[:, :, None] * A[None, :, :])         # Abar  [Bt, d, N]
        k = input_coefficient(dt_l[:, :, None], A[None, :, :], zoh)
        bx = k * B[:, l, None, :] * u[:, l, :, None]                 # Bbar x
        h = a * h + bx
        y[:, l, :] = (h * C[:, l, None, :]).sum(axis=-1)
        if want_magnitude:
            h_mag = a * h_mag + np.abs(bx)
            y_mag[:, l, :] = (h_mag * np.abs(C[:, l, None, :])).sum(axis=-1)
    if D is not None:
        du = _f64(D)[None, None, :] * u
        y = y + du
        if want_magnitude:
            y_mag = y_mag + np.abs(du)
    if z is not None:
        g = silu(z)
        y = y * g
        if want_magnitude:
            y_mag = y_mag * np.abs(g)
    if want_magnitude:
        return y, h, y_mag, h_mag
    return y, h


def selective_state_update(state, x, delta, A, B, C, D=None, z=None,
                           delta_bias=None, delta_softplus=False,
                           want_magnitude=False, zoh=False):
    """One decode step: new state and output for a single token, in float64.

    [TtoM] section 6.3 (each generation step does a fixed amount of work on
    a fixed-size state and never revisits history; it maps the old state and
    the token to a new state and an output) and [Notes] "linear scaling"
    (the recurrent ssm_state kept between tokens). The step itself is the
    scan's step for one token:

    state, new_state: [Bt, d, N]; x, delta, z: [Bt, d]; B, C: [Bt, N];
    A: [d, N]; D, delta_bias: [d].

    Returns (y, new_state) or, with want_magnitude, (y, new_state, y_mag, s_mag).
    """
    s = _f64(state)
    x = _f64(x)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    dt = discretize_delta(delta, delta_bias, delta_softplus)   # [Bt, d]
    a = np.exp(dt[:, :, None] * A[None, :, :])
    bx = input_coefficient(dt[:, :, None], A[None, :, :], zoh) * B[:, None, :] * x[:, :, None]
    s_new = a * s + bx
    y = (s_new * C[:, None, :]).sum(axis=-1)
    if want_magnitude:
        s_mag = a * np.abs(s) + np.abs(bx)
        y_mag = (s_mag * np.abs(C[:, None, :])).sum(axis=-1)
    if D is not None:
        du = _f64(D)[None, :] * x
        y = y + du
        if want_magnitude:
            y_mag = y_mag + np.abs(du)
    if z is not None:
        g = silu(z)
        y = y * g
        if want_magnitude:
            y_mag = y_mag * np.abs(g)
    if want_magnitude:
        return y, s_new, y_mag, s_mag
    return y, s_new


def scaled_error(got, ref, mag):
    """max_i |got_i - ref_i| / mag_i: the parity metric.

    mag is the oracle's magnitude companion (|ref| <= mag). Where mag is 0 the
    reference is exactly 0 and only an exact match counts as error 0. NaN in
    the same places on both sides counts as a match; NaN on one side only is
    an infinite error.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    if got.size == 0:
        return 0.0
    nan_g = np.isnan(got)
    nan_r = np.isnan(ref)
    if np.any(nan_g != nan_r):
        return float("inf")
    ok = ~nan_r
    g, r = got[ok], ref[ok]
    with np.errstate(invalid="ignore"):
        diff = np.where(g == r, 0.0, np.abs(g - r))
    m = mag[ok]
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(m > 0, diff / np.where(m > 0, m, 1.0), np.where(diff == 0, 0.0, np.inf))
    return float(e.max()) if e.size else 0.0
