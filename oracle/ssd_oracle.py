"""Float64 NumPy oracle of the structured state-space duality (SSD) layer of
Mamba-2: TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); it shares no
code with the HIP path.

[HiddenCost] (section on the value and limits of the argument) states that
Mamba-2 recasts the selective SSM as a structured state-space duality: its
input-output map is y = M o (Q K^T) V with M lower triangular and
semiseparable, Q given by C and K by B, every submatrix of the lower part of
rank at most N, which lets the layer run either as a recurrence or as
attention-like matrix products (on matrix cores). [TtoM] section 9.1 adds
that Mamba-2's state matrix is diagonal.

Reading taken (the pages leave the details open): for M to be one matrix
applied to Q K^T for all states at once, the decay between two steps cannot
depend on the state index n. So A is one scalar per head, and the layer is
the selective scan of ``ssm_oracle`` with, per head h of P channels:

    A[d, n] = a[h],   delta[b, l, d] = dt[b, l, h],   D[d] = D[h],
    bias[d] = dt_bias[h]                  for every channel d = h*P + p,

B and C shared by all heads (one group). Shapes: x, z [Bt, L, H, P];
dt [Bt, L, H]; a, D, dt_bias [H]; B, C [Bt, L, N]; h0, h_final [Bt, H, P, N].

Two forms are given, computed independently of each other:

- ``ssd_recurrent``: the recurrence (the plain definition), through
  ``selective_scan`` with the per-head parameters broadcast to channels;
- ``ssd_quadratic``: the matrix form, per (batch, head)
      y = (M o (C B^T)) (dt x) + (C h0 scaled by the decay from the start)
          + D x,                                  then the gate,
  with M[t, s] = exp(a * (sum of dt over steps s+1 .. t)) for t >= s, else 0.
  Quadratic in L; for small cases.
"""

from __future__ import annotations

import numpy as np

from .ssm_oracle import discretize_delta, selective_scan, silu

__all__ = ["ssd_expand", "ssd_recurrent", "ssd_quadratic"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def ssd_expand(x, dt, a, D=None, dt_bias=None, z=None, h0=None):
    """Per-head parameters broadcast to the channels d = h*P + p of the
    selective scan: returns (u, delta, A_full, D_full, bias_full, z, h0) in
    ``selective_scan``'s shapes, for a given state size N taken from h0 or
    left for the caller (A_full is [d, 1] and broadcasts over n)."""
    x = _f64(x)
    Bt, L, H, P = x.shape
    u = x.reshape(Bt, L, H * P)
    delta = np.repeat(_f64(dt), P, axis=2)                     # [Bt, L, H*P]
    A_col = np.repeat(_f64(a), P)[:, None]                     # [H*P, 1]
    D_full = None if D is None else np.repeat(_f64(D), P)
    bias_full = None if dt_bias is None else np.repeat(_f64(dt_bias), P)
    z_full = None if z is None else _f64(z).reshape(Bt, L, H * P)
    h0_full = None if h0 is None else _f64(h0).reshape(Bt, H * P, -1)
    return u, delta, A_col, D_full, bias_full, z_full, h0_full


def ssd_recurrent(x, dt, a, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, h0=None,
                  want_magnitude=False):
    """The SSD layer as its recurrence: ``selective_scan`` with A[d, n] = a[h]
    for all n. Returns y [Bt, L, H, P] and h_final [Bt, H, P, N] (and their
    magnitude companions with want_magnitude)."""
    x = _f64(x)
    Bt, L, H, P = x.shape
    N = np.asarray(B).shape[-1]
    u, delta, A_col, D_full, bias_full, z_full, h0_full = ssd_expand(x, dt, a, D, dt_bias, z, h0)
    A_full = np.repeat(A_col, N, axis=1)                       # [H*P, N]
    out = selective_scan(u, delta, A_full, _f64(B), _f64(C), D=D_full, z=z_full, delta_bias=bias_full,
                         delta_softplus=dt_softplus, h0=h0_full, want_magnitude=want_magnitude)
    shape_y, shape_h = (Bt, L, H, P), (Bt, H, P, N)
    if want_magnitude:
        y, hf, ym, hm = out
        return y.reshape(shape_y), hf.reshape(shape_h), ym.reshape(shape_y), hm.reshape(shape_h)
    y, hf = out
    return y.reshape(shape_y), hf.reshape(shape_h)


def ssd_quadratic(x, dt, a, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, h0=None):
    """The SSD layer in its matrix ("attention-like") form, per (batch, head):
    scores C_t . B_s, masked and decayed by the semiseparable M, applied to
    dt x; plus the initial state's contribution C_t . h0 decayed from the
    start, the D skip, and the gate. Returns y [Bt, L, H, P]."""
    x, B, C = _f64(x), _f64(B), _f64(C)
    Bt, L, H, P = x.shape
    dt_full = discretize_delta(_f64(dt), None if dt_bias is None else _f64(dt_bias)[None, None, :], dt_softplus)
    a = _f64(a)
    y = np.zeros((Bt, L, H, P))
    tri = np.tril(np.ones((L, L), dtype=bool))
    for b in range(Bt):
        scores = C[b] @ B[b].T                                  # [L, L]: C_t . B_s
        for h in range(H):
            cum = np.cumsum(dt_full[b, :, h])                   # sum of dt over steps 0..t
            seg = cum[:, None] - cum[None, :]                   # sum over s+1..t
            M = np.where(tri, np.exp(a[h] * np.where(tri, seg, 0.0)), 0.0)
            v = dt_full[b, :, h, None] * x[b, :, h, :]          # [L, P]
            y[b, :, h, :] = (M * scores) @ v
            if h0 is not None:
                # the state entering step 0, decayed through steps 0..t
                y[b, :, h, :] += np.exp(a[h] * cum)[:, None] * (C[b] @ _f64(h0)[b, h].T)
    if D is not None:
        y += _f64(D)[None, None, :, None] * x
    if z is not None:
        y *= silu(_f64(z))
    return y
