"""Seeded synthetic inputs for the scan and the decode state update.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the scan's arithmetic. The tests and the benchmark use it to
feed both the HIP path and the CPU oracle with identical values.

Recipe (the same for every workload; the sizes differ):

- u, delta_raw, B, C, z ~ N(0, 1), drawn as float32.
- A[d, n] = -(n + 1) (the S4D-real initialisation, A = -exp(log(1..N))).
- D = 1.
- delta_bias per channel: a target step dt_d = exp(U(ln lo, ln hi)) is drawn
  per channel. The bias is then softplus^-1(dt_d) = dt + log(-expm1(-dt)), in
  float64, cast to float32. With softplus on and delta_raw ~ N(0,1), each
  channel's median step is log-uniform in [lo, hi].
- Decode state: 0.1 * N(0, 1), float32.
- Convolution before the scan (width K): x ~ N(0, 1) in the storage dtype;
  weight [d, K] and bias [d] ~ U(-1/sqrt(K), 1/sqrt(K)) float32 (the range a
  Conv1d module with one input channel per group starts from); carried
  state [B, d, K-1] ~ N(0, 1) float32.
- Mamba-2 SSD layer (heads of P channels, one decay per head): x, dt_raw,
  z ~ N(0, 1) and B, C ~ N(0, 1) as above; A[h] = -U(1, 16) (the range
  Mamba-2's decay starts from); D[h] = 1; dt_bias per head as delta_bias
  per channel above.
- bf16 tensors are float32 draws rounded to nearest-even. On the host they
  are kept as uint16 bit patterns, so both sides see the exact same values.

Streams: every tensor is drawn in blocks of 4096 time steps (or rows), each
from ``np.random.default_rng([seed, stream, tensor_id, batch, block])``.
The values therefore do not depend on how the caller slices the work.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 4096
TID_DT, TID_U, TID_DELTA, TID_B, TID_C, TID_Z, TID_STATE = range(7)
TID_CONV_X, TID_CONV_W, TID_CONV_BIAS, TID_CONV_STATE = range(7, 11)
TID_SSD_A = 11


@dataclass(frozen=True)
class Workload:
    """A named workload: sizes, storage dtype and step-size range."""

    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    in_dtype: str              # "f32" or "bf16" for u, delta, B, C, z
    dt_range: tuple = (1e-3, 1e-1)
    gate: bool = True          # z present
    final_state: bool = False  # export h_final
    kind: str = "scan"         # "scan" or "decode"
    steps: int = 1             # decode: chained steps
    stream: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def updates(self) -> int:
        return self.batch * self.seqlen * self.dim * self.dstate


WORKLOADS = {
    0: Workload("tiny scan fp32", 1, 256, 64, 16, "f32", stream=0),
    1: Workload("mamba-130m-shaped layer scan", 8, 2048, 1536, 16, "bf16", stream=1),
    2: Workload("mamba-1.4b-shaped layer scan", 4, 8192, 4096, 16, "bf16",
                final_state=True, stream=2),
    3: Workload("long-sequence scan", 1, 262144, 2560, 16, "bf16",
                dt_range=(1e-4, 1e-1), stream=3),
    4: Workload("decode state update", 128, 1, 4096, 128, "f32", kind="decode",
                steps=1000, stream=4),
}


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    # No overflow for non-NaN inputs: the largest pattern, -inf, is 0xFF800000.
    out = ((b + np.uint32(0x7FFF) + ((b >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = (x.view(np.uint32)[nan] >> 16).astype(np.uint16) | np.uint16(0x0040)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_float64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Host array in its storage form (float32 or bf16 bits) -> exact float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- draws

def _rng(seed, stream, tid, b=0, block=0):
    return np.random.default_rng([seed, stream, tid, b, block])


def _normal_blocks(seed, stream, tid, batch, rows, cols, scale=1.0, dtype="f32"):
    """[batch, rows, cols] N(0, scale^2) in storage form, drawn per (batch, 4096-row block).

    Blocks are drawn (and rounded) on a thread pool; each block has its own
    generator, so the values do not depend on the scheduling.
    """
    out = np.empty((batch, rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(job):
        b, k = job
        n = min(BLOCK, rows - k)
        blk = _rng(seed, stream, tid, b, k // BLOCK).standard_normal((n, cols), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        out[b, k:k + n] = f32_to_bf16_bits(blk) if dtype == "bf16" else blk

    jobs = [(b, k) for b in range(batch) for k in range(0, rows, BLOCK)]
    if len(jobs) == 1 or batch * rows * cols < (1 << 20):
        for jb in jobs:
            one(jb)
    else:
        with ThreadPoolExecutor(max_workers=min(8, len(jobs), os.cpu_count() or 1)) as ex:
            list(ex.map(one, jobs))
    return out


def delta_bias_for(dim, dt_range, seed, stream):
    """Per-channel bias = softplus^-1(dt_d), dt_d log-uniform in dt_range."""
    lo, hi = dt_range
    r = _rng(seed, stream, TID_DT).uniform(np.log(lo), np.log(hi), size=dim)
    dt = np.exp(r)
    return (dt + np.log(-np.expm1(-dt))).astype(np.float32)


def s4d_real_A(dim, dstate):
    """A[d, n] = -(n + 1), float32."""
    return np.broadcast_to(-np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate)).copy()


def make_scan_inputs(batch, seqlen, dim, dstate, in_dtype="f32", dt_range=(1e-3, 1e-1),
                     gate=True, seed=0, stream=100):
    """Scan inputs in storage form.

    Returns a dict with u, delta, z ([B, L, d]), B, C ([B, L, N]) as float32
    or bf16 bits (``in_dtype``), and A [d, N], D [d], delta_bias [d] as
    float32. It also carries the keys in_dtype and delta_softplus (True).
    """
    u = _normal_blocks(seed, stream, TID_U, batch, seqlen, dim, dtype=in_dtype)
    dl = _normal_blocks(seed, stream, TID_DELTA, batch, seqlen, dim, dtype=in_dtype)
    Bm = _normal_blocks(seed, stream, TID_B, batch, seqlen, dstate, dtype=in_dtype)
    Cm = _normal_blocks(seed, stream, TID_C, batch, seqlen, dstate, dtype=in_dtype)
    z = _normal_blocks(seed, stream, TID_Z, batch, seqlen, dim, dtype=in_dtype) if gate else None
    return dict(u=u, delta=dl, B=Bm, C=Cm, z=z,
                A=s4d_real_A(dim, dstate), D=np.ones(dim, dtype=np.float32),
                delta_bias=delta_bias_for(dim, dt_range, seed, stream),
                in_dtype=in_dtype, delta_softplus=True)


def make_decode_inputs(batch, dim, dstate, in_dtype="f32", dt_range=(1e-3, 1e-1),
                       gate=True, seed=0, stream=200, state_scale=0.1):
    """Decode inputs: state [B, d, N] float32 ~ 0.1 N(0,1); one token x, delta,
    z [B, d] and B, C [B, N] in ``in_dtype``; A, D, delta_bias as for the scan."""
    state = _normal_blocks(seed, stream, TID_STATE, batch, dim, dstate, scale=state_scale)
    x = _normal_blocks(seed, stream, TID_U, 1, batch, dim, dtype=in_dtype)[0]
    dl = _normal_blocks(seed, stream, TID_DELTA, 1, batch, dim, dtype=in_dtype)[0]
    Bm = _normal_blocks(seed, stream, TID_B, 1, batch, dstate, dtype=in_dtype)[0]
    Cm = _normal_blocks(seed, stream, TID_C, 1, batch, dstate, dtype=in_dtype)[0]
    z = _normal_blocks(seed, stream, TID_Z, 1, batch, dim, dtype=in_dtype)[0] if gate else None
    return dict(state=state, x=x, delta=dl, B=Bm, C=Cm, z=z,
                A=s4d_real_A(dim, dstate), D=np.ones(dim, dtype=np.float32),
                delta_bias=delta_bias_for(dim, dt_range, seed, stream),
                in_dtype=in_dtype, delta_softplus=True)


def make_conv_inputs(batch, seqlen, dim, width, in_dtype="f32", seed=0, stream=400, with_state=True):
    """Inputs of the causal conv1d: x [B, L, d] in ``in_dtype``; weight [d, K],
    bias [d] and (optionally) state [B, d, K-1] float32."""
    x = _normal_blocks(seed, stream, TID_CONV_X, batch, seqlen, dim, dtype=in_dtype)
    bound = 1.0 / np.sqrt(width)
    w = _rng(seed, stream, TID_CONV_W).uniform(-bound, bound, size=(dim, width)).astype(np.float32)
    bias = _rng(seed, stream, TID_CONV_BIAS).uniform(-bound, bound, size=dim).astype(np.float32)
    state = None
    if with_state:
        state = _normal_blocks(seed, stream, TID_CONV_STATE, batch, dim, width - 1)
    return dict(x=x, weight=w, bias=bias, state=state, in_dtype=in_dtype)


def make_ssd_inputs(batch, seqlen, nheads, headdim, dstate, in_dtype="f32", dt_range=(1e-3, 1e-1),
                    gate=True, seed=0, stream=500):
    """SSD layer inputs: x, z [B, L, H, P], dt [B, L, H], B, C [B, L, N] in
    ``in_dtype`` (float32 or bf16 bits); A, D, dt_bias [H] float32. Also the
    keys in_dtype and dt_softplus (True)."""
    d = nheads * headdim
    x = _normal_blocks(seed, stream, TID_U, batch, seqlen, d, dtype=in_dtype).reshape(batch, seqlen, nheads, headdim)
    dt = _normal_blocks(seed, stream, TID_DELTA, batch, seqlen, nheads, dtype=in_dtype)
    Bm = _normal_blocks(seed, stream, TID_B, batch, seqlen, dstate, dtype=in_dtype)
    Cm = _normal_blocks(seed, stream, TID_C, batch, seqlen, dstate, dtype=in_dtype)
    z = (_normal_blocks(seed, stream, TID_Z, batch, seqlen, d, dtype=in_dtype).reshape(batch, seqlen, nheads, headdim)
         if gate else None)
    A = (-_rng(seed, stream, TID_SSD_A).uniform(1.0, 16.0, size=nheads)).astype(np.float32)
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=np.ones(nheads, np.float32), z=z,
                dt_bias=delta_bias_for(nheads, dt_range, seed, stream), in_dtype=in_dtype, dt_softplus=True)


def workload_inputs(i: int, seed: int = 0):
    """Inputs of the numbered workload (see WORKLOADS)."""
    w = WORKLOADS[i]
    if w.kind == "decode":
        return make_decode_inputs(w.batch, w.dim, w.dstate, w.in_dtype, w.dt_range,
                                  w.gate, seed, w.stream)
    return make_scan_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.in_dtype, w.dt_range,
                            w.gate, seed, w.stream)


def as_float64(inp: dict) -> dict:
    """Exact float64 view of every array in an input dict (for the oracle)."""
    dt = inp["in_dtype"]
    out = {}
    for k, v in inp.items():
        if isinstance(v, np.ndarray):
            if k in ("u", "delta", "B", "C", "z", "x", "dt"):
                out[k] = to_float64(v, dt)
            else:
                out[k] = v.astype(np.float64)
        else:
            out[k] = v
    return out
