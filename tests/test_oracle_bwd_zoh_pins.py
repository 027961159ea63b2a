"""Pins of the backward oracle's exact zero-order-hold form (input coefficient
k = (exp(dt A) - 1) / A) against things other than itself: central finite
differences of the forward oracle with zoh=True (including A = 0 entries),
torch.autograd of a plain torch statement of that forward, the derivative of
expm1(x) / x by finite differences, and planted mistakes. CPU only.
"""

import inspect

import numpy as np
import pytest
import torch

import oracle.scan_bwd_oracle as bwd_mod
from oracle import selective_scan
from oracle.scan_bwd_oracle import _dphi, selective_scan_bwd
from tests.test_oracle_bwd_pins import GRAD_OF, inputs


def loss(inp, dy, dhf):
    y, hf = selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                           delta_bias=inp["delta_bias"], delta_softplus=True, h0=inp["h0"], zoh=True)
    return float((y * dy).sum() + (hf * dhf).sum())


def test_finite_differences_zoh():
    B, L, d, N = 2, 5, 2, 3
    inp = inputs(B, L, d, N, seed=21)
    inp["A"][0, 1] = 0.0          # the A = 0 limit, k = dt
    r = np.random.default_rng(22)
    dy, dhf = r.standard_normal((B, L, d)), r.standard_normal((B, d, N))
    g = selective_scan_bwd(dy=dy, dh_final=dhf, delta_softplus=True, zoh=True, **inp)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        base = inp[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = dict(inp), dict(inp)
            plus[name], minus[name] = base.copy(), base.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (loss(plus, dy, dhf) - loss(minus, dy, dhf)) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=2e-6, atol=2e-7 * (1 + np.abs(fd).max()),
                                   err_msg=f"d{name}")


def torch_forward_zoh(t):
    """The forward recurrence with the exact zero-order hold, plain torch ops (float64)."""
    dt = torch.nn.functional.softplus(t["delta"] + t["delta_bias"])
    h = t["h0"]
    ys = []
    for l in range(t["u"].shape[1]):
        x = dt[:, l, :, None] * t["A"]
        k = torch.expm1(x) / t["A"]
        h = torch.exp(x) * h + k * t["B"][:, l, None, :] * t["u"][:, l, :, None]
        ys.append((h * t["C"][:, l, None, :]).sum(-1))
    y = torch.stack(ys, 1) + t["D"] * t["u"]
    return y * torch.nn.functional.silu(t["z"]), h


def autograd_agrees(bwd, seed=23):
    B, L, d, N = 2, 17, 3, 4
    inp = inputs(B, L, d, N, seed=seed)
    r = np.random.default_rng(seed + 1)
    dy, dhf = r.standard_normal((B, L, d)), r.standard_normal((B, d, N))
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    y, hf = torch_forward_zoh(t)
    (y * torch.tensor(dy)).sum().add((hf * torch.tensor(dhf)).sum()).backward()
    g = bwd(dy=dy, dh_final=dhf, delta_softplus=True, zoh=True, **inp)
    return {n: np.allclose(g[gn], t[n].grad.numpy(), rtol=1e-10, atol=1e-11) for n, gn in GRAD_OF.items()}


def test_matches_torch_autograd_zoh():
    ok = autograd_agrees(selective_scan_bwd)
    assert all(ok.values()), ok


def test_dphi_is_the_derivative_of_expm1_over_x():
    def phi(x):
        return np.where(x == 0.0, 1.0, np.expm1(x) / np.where(x == 0.0, 1.0, x))
    x = np.array([-40.0, -7.5, -1.0, -0.3, -2e-2, -1.2e-3, 1.5e-3, 0.4, 2.0])
    h = 1e-5 * np.maximum(1.0, np.abs(x))
    fd = (phi(x + h) - phi(x - h)) / (2 * h)
    np.testing.assert_allclose(_dphi(x), fd, rtol=1e-7, atol=1e-12)
    # the closed form and the series agree where the oracle switches between them
    for s in (-1.0, 1.0):
        lo, hi = _dphi(np.array([s * (1e-3 - 1e-12)])), _dphi(np.array([s * (1e-3 + 1e-12)]))
        np.testing.assert_allclose(lo, hi, rtol=1e-11)   # the closed form rounds to ~1e-12 there
    assert _dphi(np.array([0.0]))[0] == 0.5


MUTANTS = {
    # d k / d dt taken as 1 (the simplified form's derivative)
    "zoh_ddt_as_default": ("dkdt = abar[:, l] if zoh else 1.0", "dkdt = 1.0"),
    # the dependence of k on A dropped from dA
    "zoh_no_dk_dA": ("dA += (lam * dkdA * bu).sum(0)", "dA += 0.0 * (lam * dkdA * bu).sum(0)"),
    # k in dB replaced by dt
    "zoh_dB_with_dt": ("ku = k * u[:, l, :, None]", "ku = dt[:, l, :, None] * u[:, l, :, None]"),
}


def mutant(kind):
    src = inspect.getsource(bwd_mod)
    a, b = MUTANTS[kind]
    assert a in src, kind
    ns = {}
    exec(compile(src.replace(a, b).replace("from .ssm_oracle import", "from oracle.ssm_oracle import"),
                 "<mutant>", "exec"), ns)
    return ns["selective_scan_bwd"]


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_zoh_mutant_is_rejected(kind):
    assert not all(autograd_agrees(mutant(kind)).values())
