"""Float64 NumPy oracle of the selective scan's backward pass (gradients of a
loss through the forward of ``ssm_oracle.selective_scan``).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); no code shared with the
HIP path.

The forward, per batch b, channel d, state n, step l ([TtoM] sections 2, 3.1
and 5):

    x_l   = delta_raw_l + bias;  dt_l = softplus(x_l) (or x_l)
    a_l   = exp(dt_l A);         h_l = a_l h_{l-1} + dt_l B_l u_l   (h_{-1} = h0)
    p_l   = sum_n C_l h_l + D u_l;   y_l = p_l silu(z_l)   (or p_l)

Given dy = dL/dy (and optionally dh_final = dL/dh_{L-1} from a loss on the
final state), reverse-mode differentiation of exactly these steps gives, with
lam_l = dL/dh_l (total) and dp_l = dy_l silu(z_l):

    lam_l    = dp_l C_l + a_{l+1} lam_{l+1}        (lam_{L-1} = dp C + dh_final)
    dC_l[n]  = sum_d dp_l h_l                     dB_l[n] = sum_d lam_l dt_l u_l
    du_l     = dp_l D + sum_n lam_l dt_l B_l
    ddt_l    = sum_n lam_l (A a_l h_{l-1} + B_l u_l)
    dA[d,n]  = sum_{b,l} lam_l dt_l a_l h_{l-1}
    dh0      = a_0 lam_0
    dz_l     = dy_l p_l silu'(z_l),  silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
    ddelta_l = ddt_l sigmoid(x_l) (softplus' = sigmoid)   (or ddt_l)
    dD[d]    = sum_{b,l} dp_l u_l;   dbias[d] = sum_{b,l} ddelta_l

The reverse recurrence over lam is the adjoint of the forward recurrence: the
same sequential dependence, run backwards in time ([HiddenCost], section on
the optimisation problems of sequential gradients: every token's gradient
flows back through all the states after it).

Exact zero-order hold (``zoh=True``; [Breakthrough] section 二.3, the forward
of ``input_coefficient``): the input term is k_l B_l u_l with
k = (exp(dt A) - 1) / A (k = dt at A = 0). Its derivatives replace dt where
it multiplies B u, and add the dependence of k on dt and A:

    dk/ddt = a,   dk/dA = dt^2 phi'(dt A),  phi(x) = expm1(x) / x,
    phi'(x) = (x e^x - e^x + 1) / x^2  (= 1/2 + x/3 + x^2/8 + ... near 0)

so that dB_l = sum_d lam_l k_l u_l, du_l = dp_l D + sum_n lam_l k_l B_l,
ddt_l = sum_n lam_l a_l (A h_{l-1} + B_l u_l) and
dA = sum_{b,l} lam_l (dt_l a_l h_{l-1} + dt_l^2 phi'(dt_l A) B_l u_l).

Magnitude companions (``want_magnitude``): the same formulas evaluated on
absolute values (|dy|, |C|, |B|, |u|, |A|, |D|, the forward's magnitude
companion h_mag for |h|), so every gradient entry is bounded by its companion
(triangle inequality). They scale the parity error of the GPU gradients.
"""

from __future__ import annotations

import numpy as np

from .ssm_oracle import input_coefficient, silu, softplus

__all__ = ["selective_scan_bwd"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def _dphi(x):
    """phi'(x) for phi(x) = expm1(x) / x (phi(0) = 1): the closed form away
    from 0, its Taylor series (to x^4) where the closed form cancels."""
    x = np.asarray(x, dtype=np.float64)
    small = np.abs(x) < 1e-3
    xs = np.where(small, 1.0, x)
    closed = (xs * np.exp(xs) - np.expm1(xs)) / (xs * xs)
    series = 0.5 + x / 3.0 + x * x / 8.0 + x ** 3 / 30.0 + x ** 4 / 144.0
    return np.where(small, series, closed)


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                       delta_softplus=False, h0=None, dh_final=None, want_magnitude=False, zoh=False):
    """Gradients of the selective scan. Shapes as ``selective_scan``; dy [Bt, L, d],
    dh_final [Bt, d, N] (optional).

    Returns a dict with du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0
    (dD / dz / ddelta_bias are None when D / z / delta_bias are None). With
    want_magnitude, a second dict of magnitude companions with the same keys.
    """
    u, A, B, C, dy = _f64(u), _f64(A), _f64(B), _f64(C), _f64(dy)
    Bt, L, d = u.shape
    N = A.shape[1]
    x = _f64(delta)
    if delta_bias is not None:
        x = x + _f64(delta_bias)
    dt = softplus(x) if delta_softplus else x
    dsp = _sigmoid(x) if delta_softplus else np.ones_like(x)

    # Forward, keeping every state: hs[:, l+1] = h_l, hs[:, 0] = h0.
    hs = np.empty((Bt, L + 1, d, N))
    hs[:, 0] = 0.0 if h0 is None else _f64(h0)
    hm = np.empty((Bt, L + 1, d, N))           # magnitude companion of h
    hm[:, 0] = np.abs(hs[:, 0])
    abar = np.exp(dt[..., None] * A[None, None])                   # [Bt, L, d, N]
    kco = input_coefficient(dt[..., None], A[None, None], zoh=zoh)  # [Bt, L, d, N]
    for l in range(L):
        bx = kco[:, l] * B[:, l, None, :] * u[:, l, :, None]
        hs[:, l + 1] = abar[:, l] * hs[:, l] + bx
        hm[:, l + 1] = abar[:, l] * hm[:, l] + np.abs(bx)
    p = (hs[:, 1:] * C[:, :, None, :]).sum(-1)
    pm = (hm[:, 1:] * np.abs(C[:, :, None, :])).sum(-1)
    if D is not None:
        D = _f64(D)
        p = p + D * u
        pm = pm + np.abs(D * u)

    if z is not None:
        z = _f64(z)
        s = _sigmoid(z)
        g = silu(z)
        dsilu = s * (1.0 + z * (1.0 - s))
        dp, dpm = dy * g, np.abs(dy * g)
        # silu' = s + s z (1 - s): its companion bounds the two terms
        # separately (they cancel near z = -1.28).
        dz, dzm = dy * p * dsilu, np.abs(dy) * pm * (s * (1.0 + np.abs(z) * (1.0 - s)))
    else:
        dp, dpm = dy.copy(), np.abs(dy)
        dz = dzm = None

    du = np.zeros((Bt, L, d))
    dum = np.zeros((Bt, L, d))
    dD = dDm = None
    if D is not None:
        du += dp * D
        dum += np.abs(dp * D)
        dD = (dp * u).sum((0, 1))
        dDm = np.abs(dp * u).sum((0, 1))

    ddt = np.zeros((Bt, L, d))
    ddtm = np.zeros((Bt, L, d))
    dA = np.zeros((d, N))
    dAm = np.zeros((d, N))
    dB = np.zeros((Bt, L, N))
    dBm = np.zeros((Bt, L, N))
    dC = np.zeros((Bt, L, N))
    dCm = np.zeros((Bt, L, N))
    lam_next = np.zeros((Bt, d, N)) if dh_final is None else _f64(dh_final).copy()
    lam_next_m = np.abs(lam_next)
    for l in reversed(range(L)):
        Cl = C[:, l, None, :]
        Bl = B[:, l, None, :]
        lam = dp[:, l, :, None] * Cl + lam_next                      # dL/dh_l
        lam_m = dpm[:, l, :, None] * np.abs(Cl) + lam_next_m
        dC[:, l] = (dp[:, l, :, None] * hs[:, l + 1]).sum(1)
        dCm[:, l] = (dpm[:, l, :, None] * hm[:, l + 1]).sum(1)
        k = kco[:, l]                                                # [Bt, d, N]
        ku = k * u[:, l, :, None]
        dB[:, l] = (lam * ku).sum(1)
        dBm[:, l] = (lam_m * np.abs(ku)).sum(1)
        du[:, l] += (lam * k * Bl).sum(-1)
        dum[:, l] += (lam_m * np.abs(k * Bl)).sum(-1)
        ah = abar[:, l] * hs[:, l]                                   # a_l h_{l-1}
        ahm = abar[:, l] * hm[:, l]
        bu = Bl * u[:, l, :, None]
        dkdt = abar[:, l] if zoh else 1.0                            # dk/ddt
        ddt[:, l] = (lam * (A * ah + dkdt * bu)).sum(-1)
        ddtm[:, l] = (lam_m * (np.abs(A) * ahm + np.abs(dkdt * bu))).sum(-1)
        dtl = dt[:, l, :, None]
        dA += (lam * dtl * ah).sum(0)
        dAm += (lam_m * np.abs(dtl) * ahm).sum(0)
        if zoh:
            dkdA = dtl * dtl * _dphi(dtl * A)                        # dk/dA
            dA += (lam * dkdA * bu).sum(0)
            dAm += (lam_m * np.abs(dkdA * bu)).sum(0)
        lam_next = abar[:, l] * lam
        lam_next_m = abar[:, l] * lam_m
    ddelta = ddt * dsp
    ddeltam = ddtm * np.abs(dsp)
    dbias = dbiasm = None
    if delta_bias is not None:
        dbias = ddelta.sum((0, 1))
        dbiasm = ddeltam.sum((0, 1))
    grads = dict(du=du, ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, dz=dz, ddelta_bias=dbias,
                 dh0=lam_next)
    if not want_magnitude:
        return grads
    mags = dict(du=dum, ddelta=ddeltam, dA=dAm, dB=dBm, dC=dCm, dD=dDm, dz=dzm, ddelta_bias=dbiasm,
                dh0=lam_next_m)
    return grads, mags
