"""Plant plausible mistakes in a copy of the conv1d oracle and check that the
pins of tests/test_oracle_conv_pins.py reject each one. CPU only."""

import numpy as np
import pytest
from scipy import signal

from oracle import causal_conv1d


def mutant(kind):
    def conv(x, weight, bias=None, silu_activation=True, state=None):
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(weight, dtype=np.float64)
        if kind == "taps_reversed":
            w = w[:, ::-1]
        Bt, L, d = x.shape
        K = w.shape[1]
        prefix = np.zeros((Bt, K - 1, d)) if state is None else np.transpose(np.asarray(state, float), (0, 2, 1))
        if kind == "state_reversed" and state is not None:
            prefix = prefix[:, ::-1]
        xe = np.concatenate([prefix, x], axis=1)
        shift = 1 if kind == "off_by_one" else 0
        out = np.zeros((Bt, L, d))
        for k in range(K):
            seg = xe[:, k + shift:k + shift + L, :]
            if seg.shape[1] < L:
                seg = np.concatenate([seg, np.zeros((Bt, L - seg.shape[1], d))], axis=1)
            out += w[:, k] * seg
        if kind == "silu_before_bias":
            out = out / (1 + np.exp(-out)) if silu_activation else out
            if bias is not None:
                out = out + bias
            return out, None
        if bias is not None:
            out = out + bias
        y = out / (1 + np.exp(-out)) if silu_activation else out
        return y, np.transpose(xe[:, L:L + K - 1], (0, 2, 1))
    return conv


def pins_pass(conv):
    rng = np.random.default_rng(0)
    # library convolution
    x, w, b = rng.standard_normal((1, 20, 3)), rng.standard_normal((3, 4)), rng.standard_normal(3)
    y, _ = conv(x, w, b, silu_activation=False)
    for di in range(3):
        if not np.allclose(y[0, :, di], np.convolve(x[0, :, di], w[di, ::-1])[:20] + b[di]):
            return False
    # FIR filter continuing from a state
    st = rng.standard_normal((1, 3, 3))
    y, _ = conv(x, w, None, silu_activation=False, state=st)
    for di in range(3):
        ref = signal.lfilter(w[di, ::-1], [1.0], np.concatenate([st[0, di], x[0, :, di]]))[3:]
        if not np.allclose(y[0, :, di], ref):
            return False
    # SiLU after the bias
    lin, _ = conv(x, w, b, silu_activation=False)
    y, _ = conv(x, w, b, silu_activation=True)
    return bool(np.allclose(y, lin / (1 + np.exp(-lin))))


def test_unmutated_copy_passes():
    assert pins_pass(mutant("none"))
    assert pins_pass(causal_conv1d)


@pytest.mark.parametrize("kind", ["taps_reversed", "off_by_one", "state_reversed", "silu_before_bias"])
def test_mutant_is_rejected(kind):
    assert not pins_pass(mutant(kind))
