"""Pins of the backward oracle against things other than itself:

- central finite differences of the forward oracle (a different computation:
  only forward evaluations of a scalar loss), for every input;
- reverse-mode automatic differentiation (torch.autograd, float64, CPU) of a
  plain torch statement of the forward recurrence written here;
- the magnitude companions bound every gradient;
- closed forms at L = 1 and for zero steps.

CPU only.
"""

import numpy as np
import pytest
import torch

from oracle import selective_scan
from oracle.scan_bwd_oracle import selective_scan_bwd


def inputs(B, L, d, N, seed=0, softplus=True):
    r = np.random.default_rng(seed)
    return dict(
        u=r.standard_normal((B, L, d)), delta=r.standard_normal((B, L, d)) * (1.0 if softplus else 0.1) +
        (0.0 if softplus else 0.5),
        A=-np.exp(r.standard_normal((d, N)) * 0.5), B=r.standard_normal((B, L, N)),
        C=r.standard_normal((B, L, N)), D=r.standard_normal(d), z=r.standard_normal((B, L, d)),
        delta_bias=r.standard_normal(d) * 0.3, h0=r.standard_normal((B, d, N)))


def loss(inp, dy, dhf, softplus):
    y, hf = selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                           delta_bias=inp["delta_bias"], delta_softplus=softplus, h0=inp["h0"])
    return float((y * dy).sum() + (hf * dhf).sum())


GRAD_OF = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz", delta_bias="ddelta_bias",
               h0="dh0")


@pytest.mark.parametrize("softplus", [True, False])
def test_finite_differences(softplus):
    B, L, d, N = 2, 5, 2, 3
    inp = inputs(B, L, d, N, seed=1, softplus=softplus)
    r = np.random.default_rng(2)
    dy, dhf = r.standard_normal((B, L, d)), r.standard_normal((B, d, N))
    g = selective_scan_bwd(dy=dy, dh_final=dhf, delta_softplus=softplus, **inp)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        base = inp[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus = dict(inp)
            minus = dict(inp)
            plus[name] = base.copy()
            minus[name] = base.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (loss(plus, dy, dhf, softplus) - loss(minus, dy, dhf, softplus)) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=2e-6, atol=2e-7 * (1 + np.abs(fd).max()),
                                   err_msg=f"d{name}")


def torch_forward(t, softplus):
    """The forward recurrence in plain torch ops (float64), step by step."""
    x = t["delta"] + t["delta_bias"]
    dt = torch.nn.functional.softplus(x) if softplus else x
    h = t["h0"]
    ys = []
    for l in range(t["u"].shape[1]):
        a = torch.exp(dt[:, l, :, None] * t["A"])
        h = a * h + dt[:, l, :, None] * t["B"][:, l, None, :] * t["u"][:, l, :, None]
        ys.append((h * t["C"][:, l, None, :]).sum(-1))
    y = torch.stack(ys, 1) + t["D"] * t["u"]
    y = y * torch.nn.functional.silu(t["z"])
    return y, h


def test_matches_torch_autograd():
    B, L, d, N = 2, 23, 3, 4
    inp = inputs(B, L, d, N, seed=3)
    r = np.random.default_rng(4)
    dy, dhf = r.standard_normal((B, L, d)), r.standard_normal((B, d, N))
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    y, hf = torch_forward(t, True)
    (y * torch.tensor(dy)).sum().add((hf * torch.tensor(dhf)).sum()).backward()
    g = selective_scan_bwd(dy=dy, dh_final=dhf, delta_softplus=True, **inp)
    for name, gname in GRAD_OF.items():
        np.testing.assert_allclose(g[gname], t[name].grad.numpy(), rtol=1e-11, atol=1e-12, err_msg=gname)


def test_magnitude_companions_bound_gradients():
    B, L, d, N = 2, 40, 3, 5
    inp = inputs(B, L, d, N, seed=5)
    r = np.random.default_rng(6)
    g, m = selective_scan_bwd(dy=r.standard_normal((B, L, d)), dh_final=r.standard_normal((B, d, N)),
                              delta_softplus=True, want_magnitude=True, **inp)
    for k in g:
        assert np.all(np.abs(g[k]) <= m[k] * (1 + 1e-12) + 1e-300), k


def test_single_step_closed_form():
    """L = 1, no gate, no bias, no softplus: all gradients in closed form."""
    r = np.random.default_rng(7)
    B, d, N = 2, 3, 4
    u, dl, A = r.standard_normal((B, 1, d)), np.abs(r.standard_normal((B, 1, d))), -np.abs(r.standard_normal((d, N)))
    Bm, Cm, D, h0 = r.standard_normal((B, 1, N)), r.standard_normal((B, 1, N)), r.standard_normal(d), r.standard_normal((B, d, N))
    dy = r.standard_normal((B, 1, d))
    g = selective_scan_bwd(u, dl, A, Bm, Cm, dy, D=D, h0=h0)
    dt = dl[:, 0, :, None]
    a = np.exp(dt * A)
    lam = dy[:, 0, :, None] * Cm[:, 0, None, :]
    h1 = a * h0 + dt * Bm[:, 0, None, :] * u[:, 0, :, None]
    np.testing.assert_allclose(g["dh0"], a * lam, rtol=1e-14)
    np.testing.assert_allclose(g["dC"][:, 0], (dy[:, 0, :, None] * h1).sum(1), rtol=1e-13)
    np.testing.assert_allclose(g["du"][:, 0], dy[:, 0] * D + (lam * dt * Bm[:, 0, None, :]).sum(-1), rtol=1e-13)
    np.testing.assert_allclose(g["ddelta"][:, 0], (lam * (A * a * h0 + Bm[:, 0, None, :] * u[:, 0, :, None])).sum(-1),
                               rtol=1e-12)
    np.testing.assert_allclose(g["dA"], (lam * dt * a * h0).sum(0), rtol=1e-12)


def test_zero_steps_pass_state_gradient_through():
    """dt = 0 everywhere (no softplus, no bias): the state is frozen, so dh0 is
    dh_final plus the readouts' sum of dy C, and dB is zero."""
    r = np.random.default_rng(8)
    B, L, d, N = 1, 6, 2, 3
    u, A = r.standard_normal((B, L, d)), -np.abs(r.standard_normal((d, N)))
    Bm, Cm, dy, dhf = r.standard_normal((B, L, N)), r.standard_normal((B, L, N)), r.standard_normal((B, L, d)), \
        r.standard_normal((B, d, N))
    g = selective_scan_bwd(u, np.zeros((B, L, d)), A, Bm, Cm, dy, h0=r.standard_normal((B, d, N)), dh_final=dhf)
    expect = dhf + (dy[:, :, :, None] * Cm[:, :, None, :]).sum(1)
    np.testing.assert_allclose(g["dh0"], expect, rtol=1e-14)
    assert np.all(g["dB"] == 0)
