"""Plant plausible mistakes in a copy of the oracle's scan step and check the pins reject them.

A mutant is the oracle's time loop with one slip: the exponent's sign, the
step dropped from B-bar, the gate applied before the D skip, B and C swapped,
the readout taken before the update, or D multiplying the state. Each must
disagree with the brute-force expansion, or with the hand-worked golden scan,
or with the small-step derivative. Everything runs on the CPU; nothing here
touches the product path.
"""

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import brute_force, rand_case, read_golden


def mutant_scan(kind):
    def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None):
        u, A, B, C = (np.asarray(v, dtype=np.float64) for v in (u, A, B, C))
        Bt, L, d = u.shape
        N = A.shape[1]
        dt = oracle.discretize_delta(delta, delta_bias, delta_softplus)
        h = np.zeros((Bt, d, N)) if h0 is None else np.array(h0, dtype=np.float64)
        y = np.zeros((Bt, L, d))
        for l in range(L):
            dl = dt[:, l, :, None]
            sign = -1.0 if kind == "exp_sign" else 1.0
            a = np.exp(sign * dl * A[None])
            Bl, Cl = (C, B) if kind == "swap_BC" else (B, C)
            step = 1.0 if kind == "drop_dt_in_B" else dl
            bx = step * Bl[:, l, None, :] * u[:, l, :, None]
            if kind == "readout_before_update":
                y[:, l] = (h * Cl[:, l, None, :]).sum(-1)
                h = a * h + bx
            else:
                h = a * h + bx
                y[:, l] = (h * Cl[:, l, None, :]).sum(-1)
        if kind == "gate_before_skip" and z is not None:
            y = y * oracle.silu(z)
        if D is not None:
            y = y + np.asarray(D)[None, None, :] * u
        if kind != "gate_before_skip" and z is not None:
            y = y * oracle.silu(z)
        return y, h
    return scan


def pins_pass(scan):
    """True when the scan passes every pin used here."""
    rng = np.random.default_rng(21)
    c = rand_case(rng)
    y, h = scan(**c)
    yb, hb = brute_force(c)
    if not (np.allclose(y, yb, rtol=1e-10, atol=1e-12) and np.allclose(h, hb, rtol=1e-10, atol=1e-12)):
        return False
    g = read_golden("scalar_scan_worked.txt")
    L = len(g["u"])
    y, h = scan(g["u"].reshape(1, L, 1), g["delta"].reshape(1, L, 1), g["A"].reshape(1, 1),
                g["B"].reshape(1, L, 1), g["C"].reshape(1, L, 1), D=g["D"])
    if not np.allclose(y[0, :, 0], g["y"], rtol=1e-12):
        return False
    c = rand_case(rng, L=1, gate=False)
    c["delta"] = np.full_like(c["delta"], 1e-7)
    c["delta_bias"] = None
    c["delta_softplus"] = False
    _, h1 = scan(**c)
    expect = c["A"][None] * c["h0"] + c["B"][:, 0, None, :] * c["u"][:, 0, :, None]
    return bool(np.allclose((h1 - c["h0"]) / 1e-7, expect, rtol=2e-5, atol=2e-6))


def test_unmutated_copy_passes():
    assert pins_pass(mutant_scan("none"))
    assert pins_pass(oracle.selective_scan)


@pytest.mark.parametrize("kind", ["exp_sign", "drop_dt_in_B", "gate_before_skip", "swap_BC",
                                  "readout_before_update"])
def test_mutant_is_rejected(kind):
    assert not pins_pass(mutant_scan(kind))
