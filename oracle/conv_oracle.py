"""Float64 NumPy oracle of the causal depthwise conv1d + SiLU that precedes
the selective scan, and of its single-token decode update.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Shares no code with the
HIP kernels or their binding.

What it computes, per batch b, channel d and step l, for a filter of width K
([TtoM] section 5: the block's depthwise Conv1d over the sequence, padded by
K-1 and truncated to the first L outputs, then SiLU; [Notes] "Mamba block 的
结构": a short local convolution before the selective SSM):

    out[b,l,d] = bias[d] + sum_{k=0}^{K-1} weight[d,k] * x[b, l-(K-1)+k, d]
    y[b,l,d]   = silu(out[b,l,d])        (or out itself without the activation)

Inputs before step 0 come from an optional carried state (else zero): the
fixed-size conv_state kept between tokens ([Notes], "Mamba block 的结构"):

    state[b,d,j] = x[b, j-(K-1), d],  j = 0..K-2   (oldest first)

and the state after the sequence holds its last K-1 inputs the same way.

Readings taken (the pages are silent): the filter is applied as a
cross-correlation, the form of the Conv1d module the listing uses, so weight
[d, K-1] multiplies the newest input; the convolution has a bias (the module's
default); the carried state is float32 [B, d, K-1], oldest input first.
"""

from __future__ import annotations

import numpy as np

from .ssm_oracle import silu

__all__ = ["causal_conv1d", "causal_conv1d_update"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def causal_conv1d(x, weight, bias=None, silu_activation=True, state=None):
    """Causal depthwise conv1d (+ SiLU) over [B, L, d]; returns (y, state_out).

    x [B, L, d]; weight [d, K]; bias [d] or None; state [B, d, K-1] or None.
    y [B, L, d]; state_out [B, d, K-1] (the last K-1 inputs, oldest first).
    """
    x = _f64(x)
    w = _f64(weight)
    Bt, L, d = x.shape
    K = w.shape[1]
    if state is None:
        prefix = np.zeros((Bt, K - 1, d))
    else:
        prefix = np.transpose(_f64(state), (0, 2, 1))          # [B, K-1, d]
    xe = np.concatenate([prefix, x], axis=1)                    # xe[:, i] = x[:, i-(K-1)]
    out = np.zeros((Bt, L, d)) if bias is None else np.broadcast_to(_f64(bias), (Bt, L, d)).copy()
    for k in range(K):
        # term k: weight[:, k] * x[l-(K-1)+k] = xe[l+k]
        out += w[:, k] * xe[:, k:k + L, :]
    y = silu(out) if silu_activation else out
    state_out = np.transpose(xe[:, L:L + K - 1, :], (0, 2, 1)).copy()   # last K-1 of xe
    return y, state_out


def causal_conv1d_update(state, x, weight, bias=None, silu_activation=True):
    """One decode step: x [B, d] is the new input; returns (y [B, d], new state [B, d, K-1])."""
    x = _f64(x)
    y, state_out = causal_conv1d(x[:, None, :], weight, bias, silu_activation, state)
    return y[:, 0, :], state_out
