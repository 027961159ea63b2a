"""Pins of the conv1d oracle against things other than itself: a library
convolution and filter, the impulse response, a hand-worked fixture, the
SiLU closed form, continuation through the carried state, and causality.

CPU only.
"""

import os

import numpy as np
import pytest
from scipy import signal

import oracle
from oracle import causal_conv1d, causal_conv1d_update

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


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


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7])
def test_matches_numpy_convolve(K):
    B, L, d = 2, 37, 5
    x, w, b = rnd(B, L, d, seed=1), rnd(d, K, seed=2), rnd(d, seed=3)
    y, _ = causal_conv1d(x, w, b, silu_activation=False)
    for bi in range(B):
        for di in range(d):
            ref = np.convolve(x[bi, :, di], w[di, ::-1])[:L] + b[di]
            np.testing.assert_allclose(y[bi, :, di], ref, rtol=1e-13, atol=1e-13)


def test_matches_fir_filter_with_initial_conditions():
    """lfilter with FIR taps reversed, continuing from a carried state."""
    K, L, d = 4, 50, 3
    x, w, st = rnd(1, L, d, seed=4), rnd(d, K, seed=5), rnd(1, d, K - 1, seed=6)
    y, _ = causal_conv1d(x, w, None, silu_activation=False, state=st)
    for di in range(d):
        full = np.concatenate([st[0, di], x[0, :, di]])
        ref = signal.lfilter(w[di, ::-1], [1.0], full)[K - 1:]
        np.testing.assert_allclose(y[0, :, di], ref, rtol=1e-13, atol=1e-13)


def test_impulse_response_is_the_reversed_filter():
    K, L = 4, 10
    w = np.array([[0.25, -1.0, 2.0, 3.5]])
    x = np.zeros((1, L, 1))
    x[0, 2, 0] = 1.0
    y, _ = causal_conv1d(x, w, None, silu_activation=False)
    expect = np.zeros(L)
    expect[2:2 + K] = w[0, ::-1]      # the newest-input tap answers first
    np.testing.assert_array_equal(y[0, :, 0], expect)


def test_golden_worked_example():
    g = read_golden("conv_worked.txt")
    K = len(g["weight"])
    L = len(g["x"])
    y, st = causal_conv1d(g["x"].reshape(1, L, 1), g["weight"].reshape(1, K), g["bias"],
                          silu_activation=False, state=g["state"].reshape(1, 1, K - 1))
    np.testing.assert_allclose(y[0, :, 0], g["y"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(st[0, 0], g["state_out"], rtol=0, atol=0)


def test_silu_applied_after_bias():
    x, w, b = rnd(2, 9, 4, seed=7), rnd(4, 3, seed=8), rnd(4, seed=9)
    lin, _ = causal_conv1d(x, w, b, silu_activation=False)
    y, _ = causal_conv1d(x, w, b, silu_activation=True)
    np.testing.assert_allclose(y, lin / (1.0 + np.exp(-lin)), rtol=1e-14, atol=1e-15)


def test_state_continuation_equals_one_pass():
    K, L1, L2, d = 4, 23, 2, 6
    x, w, b, s0 = rnd(2, L1 + L2, d, seed=10), rnd(d, K, seed=11), rnd(d, seed=12), rnd(2, d, K - 1, seed=13)
    y, s = causal_conv1d(x, w, b, state=s0)
    ya, sa = causal_conv1d(x[:, :L1], w, b, state=s0)
    yb, sb = causal_conv1d(x[:, L1:], w, b, state=sa)
    np.testing.assert_allclose(np.concatenate([ya, yb], 1), y, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(sb, s)
    # the carried state holds the last K-1 inputs, oldest first
    np.testing.assert_array_equal(s, np.transpose(x[:, -(K - 1):], (0, 2, 1)))


def test_short_sequence_state_comes_partly_from_the_old_state():
    K, d = 5, 3
    x, w, s0 = rnd(1, 2, d, seed=14), rnd(d, K, seed=15), rnd(1, d, K - 1, seed=16)
    _, s = causal_conv1d(x, w, None, state=s0)
    expect = np.concatenate([s0[0, :, 2:], x[0].T], axis=1)[None]
    np.testing.assert_array_equal(s, expect)


def test_update_steps_equal_the_sequence():
    K, L, d = 4, 12, 5
    x, w, b = rnd(3, L, d, seed=17), rnd(d, K, seed=18), rnd(d, seed=19)
    y, s_end = causal_conv1d(x, w, b)
    s = np.zeros((3, d, K - 1))
    for t in range(L):
        yt, s = causal_conv1d_update(s, x[:, t], w, b)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(s, s_end)


def test_causality_and_width_one():
    x, w = rnd(1, 20, 2, seed=20), rnd(2, 4, seed=21)
    y1, _ = causal_conv1d(x, w)
    x2 = x.copy()
    x2[0, 11:] += 5.0
    y2, _ = causal_conv1d(x2, w)
    np.testing.assert_array_equal(y1[0, :11], y2[0, :11])
    assert not np.allclose(y1[0, 11:], y2[0, 11:])
    # K = 1: a per-channel scale and shift, no state
    w1, b1 = rnd(2, 1, seed=22), rnd(2, seed=23)
    y, s = causal_conv1d(x, w1, b1, silu_activation=False)
    np.testing.assert_allclose(y, x * w1[:, 0] + b1, rtol=1e-15)
    assert s.shape == (1, 2, 0)


def test_empty_sequence_keeps_state():
    s0 = rnd(2, 3, 3, seed=24)
    y, s = causal_conv1d(np.zeros((2, 0, 3)), rnd(3, 4, seed=25), state=s0)
    assert y.shape == (2, 0, 3)
    np.testing.assert_array_equal(s, s0)


def test_oracle_module_exports():
    assert oracle.causal_conv1d is causal_conv1d
