"""Pins of the SSD oracle (Mamba-2's structured state-space duality) against
things other than itself. CPU only.

- Duality: the recurrence (``ssd_recurrent``, through the selective scan) and
  the matrix form (``ssd_quadratic``, scores masked by the semiseparable M)
  are two independent computations of one map; they must agree to rounding,
  with and without an initial state, softplus, bias, D and the gate.
- Semiseparability: every submatrix of the strictly lower part of
  M o (C B^T) has rank at most N (the property the pages state).
- Closed forms: N = 1 with B = C = 1 and a = 0 is a running sum of dt x; a
  single step is dt B.x-weighted readout.
- Mutants: plausible mistakes in the matrix form (decay including the
  current step, the wrong sign, B and C swapped, a per-channel instead of
  per-head step) break the duality test's agreement.
"""

import numpy as np
import pytest

from oracle.ssd_oracle import ssd_quadratic, ssd_recurrent
from oracle.ssm_oracle import discretize_delta, silu


def inputs(Bt=2, L=23, H=3, P=4, N=5, seed=0):
    r = np.random.default_rng(seed)
    return dict(x=r.standard_normal((Bt, L, H, P)), dt=r.standard_normal((Bt, L, H)) * 0.7 - 1.0,
                a=-np.exp(r.standard_normal(H)), B=r.standard_normal((Bt, L, N)), C=r.standard_normal((Bt, L, N)),
                D=r.standard_normal(H), z=r.standard_normal((Bt, L, H, P)), dt_bias=r.standard_normal(H) * 0.3,
                h0=r.standard_normal((Bt, H, P, N)))


@pytest.mark.parametrize("opts", [
    dict(), dict(h0=None), dict(D=None, z=None), dict(dt_bias=None), dict(softplus=False),
])
def test_recurrence_equals_matrix_form(opts):
    inp = inputs(seed=1)
    sp = opts.pop("softplus", True)
    for k, v in opts.items():
        inp[k] = v
    if not sp:
        inp["dt"] = np.abs(inp["dt"]) * 0.1
    y_rec, _ = ssd_recurrent(dt_softplus=sp, **inp)
    y_mat = ssd_quadratic(dt_softplus=sp, **inp)
    np.testing.assert_allclose(y_mat, y_rec, rtol=1e-11, atol=1e-11 * np.abs(y_rec).max())


def test_final_state_matches_matrix_form_of_state():
    """h_final = sum_s exp(a (cum_T - cum_s)) dt_s B_s x_s + exp(a cum_T) h0,
    written as a matrix product over the sequence."""
    inp = inputs(Bt=1, L=17, H=2, P=3, N=4, seed=2)
    _, hf = ssd_recurrent(dt_softplus=True, **inp)
    dt = discretize_delta(inp["dt"], inp["dt_bias"], True)
    for h in range(2):
        cum = np.cumsum(dt[0, :, h])
        w = np.exp(inp["a"][h] * (cum[-1] - cum)) * dt[0, :, h]          # [L]
        expect = (inp["x"][0, :, h, :] * w[:, None]).T @ inp["B"][0] + np.exp(inp["a"][h] * cum[-1]) * inp["h0"][0, h]
        np.testing.assert_allclose(hf[0, h], expect, rtol=1e-12, atol=1e-13)


def test_semiseparable_rank():
    Bt, L, H, P, N = 1, 40, 1, 1, 3
    inp = inputs(Bt, L, H, P, N, seed=3)
    dt = discretize_delta(inp["dt"], None, True)
    cum = np.cumsum(dt[0, :, 0])
    tri = np.tril(np.ones((L, L), dtype=bool))
    M = np.where(tri, np.exp(inp["a"][0] * np.where(tri, cum[:, None] - cum[None, :], 0.0)), 0.0)
    S = M * (inp["C"][0] @ inp["B"][0].T)
    for t0 in (5, 17, 30):
        assert np.linalg.matrix_rank(S[t0:, :t0], tol=1e-9 * np.abs(S).max()) <= N
    # ... while the whole lower triangle is of full rank
    assert np.linalg.matrix_rank(S) > N


def test_running_sum_closed_form():
    """N = 1, B = C = 1, a = 0: no decay, so y_t = sum_{s<=t} dt_s x_s."""
    r = np.random.default_rng(4)
    Bt, L, H, P = 2, 30, 2, 3
    x, dt = r.standard_normal((Bt, L, H, P)), np.abs(r.standard_normal((Bt, L, H)))
    ones = np.ones((Bt, L, 1))
    y, _ = ssd_recurrent(x, dt, np.zeros(H), ones, ones)
    np.testing.assert_allclose(y, np.cumsum(dt[..., None] * x, axis=1), rtol=1e-13)


def test_single_step():
    Bt, H, P, N = 2, 2, 3, 4
    inp = inputs(Bt, 1, H, P, N, seed=5)
    y, hf = ssd_recurrent(inp["x"], inp["dt"], inp["a"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                          dt_bias=inp["dt_bias"], dt_softplus=True, h0=inp["h0"])
    dt = discretize_delta(inp["dt"], inp["dt_bias"], True)[:, 0]                  # [Bt, H]
    decay = np.exp(dt * inp["a"])                                                  # [Bt, H]
    h1 = decay[:, :, None, None] * inp["h0"] + (dt[:, :, None] * inp["x"][:, 0])[..., None] * inp["B"][:, 0, None, None, :]
    np.testing.assert_allclose(hf, h1, rtol=1e-13)
    yy = (h1 * inp["C"][:, 0, None, None, :]).sum(-1) + inp["D"][None, :, None] * inp["x"][:, 0]
    np.testing.assert_allclose(y[:, 0], yy * silu(inp["z"][:, 0]), rtol=1e-12)


def _mutant_quadratic(inp, mistake):
    x, B, C, a = inp["x"], inp["B"], inp["C"], inp["a"]
    Bt, L, H, P = x.shape
    dt = discretize_delta(inp["dt"], None, True)
    if mistake == "per_channel_dt":
        dt = np.repeat(dt, P, axis=2)[:, :, :H]       # head h reads channel h's step
    tri = np.tril(np.ones((L, L), dtype=bool))
    y = np.zeros_like(x)
    for b in range(Bt):
        sc = (B[b] @ C[b].T) if mistake == "swap_bc" else (C[b] @ B[b].T)
        for h in range(H):
            cum = np.cumsum(dt[b, :, h])
            seg = cum[:, None] - cum[None, :]
            if mistake == "include_current":
                seg = seg + dt[b, None, :, h]
            sgn = -1.0 if mistake == "sign" else 1.0
            M = np.where(tri, np.exp(sgn * a[h] * np.where(tri, seg, 0.0)), 0.0)
            y[b, :, h] = (M * sc) @ (dt[b, :, h, None] * x[b, :, h])
    return y


@pytest.mark.parametrize("mistake", ["include_current", "sign", "swap_bc", "per_channel_dt"])
def test_duality_check_catches_mutants(mistake):
    inp = inputs(Bt=1, L=15, H=3, P=2, N=3, seed=6)
    y_rec, _ = ssd_recurrent(inp["x"], inp["dt"], inp["a"], inp["B"], inp["C"], dt_softplus=True)
    y_mut = _mutant_quadratic(inp, mistake)
    assert np.abs(y_mut - y_rec).max() > 1e-3 * np.abs(y_rec).max()
