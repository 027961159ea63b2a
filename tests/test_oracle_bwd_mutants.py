"""Plant plausible mistakes in a copy of the backward oracle (by editing its
source text) and check the autograd pin rejects each. CPU only."""

import inspect

import numpy as np
import pytest
import torch

import oracle.scan_bwd_oracle as bwd_mod
from tests.test_oracle_bwd_pins import GRAD_OF, inputs, torch_forward

MUTANTS = {
    # propagate lam with the wrong step's transition
    "lam_wrong_transition": ("lam_next = abar[:, l] * lam\n", "lam_next = abar[:, max(l - 1, 0)] * lam\n"),
    # forget the loss on the final state
    "ignore_dh_final": ("else _f64(dh_final).copy()", "else 0.0 * _f64(dh_final)"),
    # drop the input term from d(loss)/d(dt)
    "ddt_without_input_term": ("(lam * (A * ah + dkdt * bu)).sum(-1)", "(lam * (A * ah)).sum(-1)"),
    # silu' taken as sigmoid only
    "silu_derivative_wrong": ("dsilu = s * (1.0 + z * (1.0 - s))", "dsilu = s"),
    # state gradient read out with the previous state
    "dC_with_previous_state": ("dC[:, l] = (dp[:, l, :, None] * hs[:, l + 1]).sum(1)",
                               "dC[:, l] = (dp[:, l, :, None] * hs[:, l]).sum(1)"),
}


def mutant(kind):
    src = inspect.getsource(bwd_mod)
    a, b = MUTANTS[kind]
    assert a in src, kind
    ns = {}
    exec(compile(src.replace(a, b).replace("from .ssm_oracle import", "from oracle.ssm_oracle import"),
                 "<mutant>", "exec"), ns)
    return ns["selective_scan_bwd"]


def pins_pass(bwd):
    B, L, d, N = 2, 9, 3, 4
    inp = inputs(B, L, d, N, seed=11)
    r = np.random.default_rng(12)
    dy, dhf = r.standard_normal((B, L, d)), r.standard_normal((B, d, N))
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    y, hf = torch_forward(t, True)
    (y * torch.tensor(dy)).sum().add((hf * torch.tensor(dhf)).sum()).backward()
    g = bwd(dy=dy, dh_final=dhf, delta_softplus=True, **inp)
    return all(np.allclose(g[gn], t[n].grad.numpy(), rtol=1e-10, atol=1e-11) for n, gn in GRAD_OF.items())


def test_unmutated_copy_passes():
    assert pins_pass(bwd_mod.selective_scan_bwd)


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_mutant_is_rejected(kind):
    assert not pins_pass(mutant(kind))
