"""GPU parity of the exact zero-order-hold option (SSM_FLAG_ZOH) of the scan
and of the decode update against the float64 oracle's ``zoh=True`` form,
through the C ABI.

The input coefficient k = (exp(dt A) - 1) / A takes two forms in the kernels
(a short series near dt A = 0, and (exp(dt A) - 1) / A elsewhere); the cases
below put A entries on both sides of the switch, at A = 0 (k = dt), and at
the magnitudes of the workloads (A = -(1..N), dt in [1e-3, 1e-1]).
"""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_87_amd import binding, synth
from tests.gpu_util import download, scan_inputs_to_device, tol_for, torch_dtype, upload
from tests.test_gpu_scan import check_scan, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def with_special_A(inp, grow=True):
    """A with a zero column, tiny entries (series side of the switch) and
    entries just either side of |dt A| = ln(2)/64 at dt = 0.01; with grow, a
    growing mode (for sequences short enough to stay within float32)."""
    inp = dict(inp)
    A = inp["A"].copy()
    N = A.shape[1]
    A[:, 0] = 0.0
    if N > 1:
        A[:, 1] = -1e-4
    if N > 2:
        A[:, 2] = np.float32(-np.log(2) / 64 / 0.01 * 0.98)
    if N > 3:
        A[:, 3] = np.float32(-np.log(2) / 64 / 0.01 * 1.02)
    if N > 4 and grow:
        A[:, 4] = 0.5          # a growing mode (A > 0): k = (e^x - 1) / A, x > 0
    inp["A"] = A
    return inp


SHAPES = [
    (1, 1, 1, 1, "f32"), (2, 67, 70, 16, "f32"), (1, 129, 130, 3, "bf16"), (3, 40, 64, 5, "f32"),
    (2, 100, 33, 64, "bf16"), (1, 64, 256, 8, "f32"), (2, 130, 300, 12, "f32"), (1, 150, 70, 32, "f32"),
    (1, 70, 96, 128, "f32"), (2, 50, 64, 100, "bf16"),
    # states split over two blocks per channel (65 to 128 channel blocks)
    (1, 40, 4160, 128, "bf16"), (2, 30, 4096, 64, "f32"),
]


@pytest.mark.parametrize("B,L,d,N,dt", SHAPES)
def test_zoh_shapes(B, L, d, N, dt):
    inp = with_special_A(synth.make_scan_inputs(B, L, d, N, dt, seed=31, stream=3100 + N))
    h0 = np.random.default_rng(N).standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"zoh {(B, L, d, N)} {dt}", inp, "f32", h0=h0, gpu_kwargs=dict(zoh=True))
    check_scan(f"zoh {(B, L, d, N)} {dt}", inp, "bf16", gpu_kwargs=dict(zoh=True))


@pytest.mark.parametrize("opts", [dict(softplus=False, use_bias=False), dict(use_D=False, use_z=False)])
def test_zoh_options(opts):
    inp = with_special_A(synth.make_scan_inputs(2, 150, 96, 16, "f32", seed=32, stream=3200))
    if opts.get("softplus") is False:
        inp = dict(inp)
        inp["delta"] = np.abs(inp["delta"]) * np.float32(0.05)
    check_scan(f"zoh options {opts}", inp, "f32", gpu_kwargs=dict(opts, zoh=True))


def test_zoh_differs_from_simplified_form():
    """The option changes the result by the expected amount: at these steps
    k / dt - 1 is about dt A / 2, far above the tolerance."""
    inp = synth.make_scan_inputs(1, 200, 64, 16, "f32", seed=33, stream=3300)
    dev = scan_inputs_to_device(inp)
    y0 = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"],
                                        z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True)
    y1 = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"],
                                        z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True, zoh=True)
    r0, _, m0, _ = oracle.selective_scan(**_oracle_args(inp), want_magnitude=True)
    r1, _, _, _ = oracle.selective_scan(**_oracle_args(inp), want_magnitude=True, zoh=True)
    gap = oracle.scaled_error(r1, r0, m0)
    assert gap > 100 * tol_for("f32", "f32"), gap
    report("zoh vs simplified, gpu gap against oracle gap",
           abs(oracle.scaled_error(download(y1), download(y0), m0) - gap) / gap, 0.01)


def _oracle_args(inp):
    f = synth.as_float64(inp)
    return dict(u=f["u"], delta=f["delta"], A=f["A"], B=f["B"], C=f["C"], D=f["D"], z=f["z"],
                delta_bias=f["delta_bias"], delta_softplus=True)


@pytest.mark.parametrize("B,L,d,N,dt", [(1, 4100, 64, 16, "bf16"), (2, 3000, 40, 8, "f32"), (1, 2100, 64, 128, "bf16"),
                                       (1, 2050, 40, 64, "f32")])
def test_zoh_chunked(B, L, d, N, dt):
    k = binding.ssm_scan_chunks(B, L, d, N)
    assert k > 1
    inp = with_special_A(synth.make_scan_inputs(B, L, d, N, dt, seed=34, stream=3400 + N), grow=False)
    h0 = np.random.default_rng(35).standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"zoh chunked x{k} {(B, L, d, N)} {dt}", inp, "f32", h0=h0, gpu_kwargs=dict(zoh=True))


def test_zoh_mamba14b_layer_sampled():
    inp = synth.workload_inputs(2)
    ch = np.r_[0:3, 62:67, 2047, 2048, 4093:4096]
    check_scan("zoh 1.4b layer (4,8192,4096,16) bf16 sampled", inp, "f32", channels=ch,
               gpu_kwargs=dict(zoh=True))


# ---------------------------------------------------------------- decode

def _decode_dev(inp):
    dt = inp["in_dtype"]
    d = {k: upload(inp[k], dt) for k in ("x", "delta", "B", "C", "z")}
    for k in ("A", "D", "delta_bias", "state"):
        d[k] = upload(inp[k], "f32")
    return d


@pytest.mark.parametrize("B,d,N,dt", [(3, 50, 3, "f32"), (5, 33, 16, "f32"), (4, 100, 128, "bf16"),
                                      (3, 17, 130, "f32"), (2, 64, 4, "bf16")])
def test_zoh_decode(B, d, N, dt):
    inp = with_special_A(synth.make_decode_inputs(B, d, N, dt, seed=36, stream=3600 + N))
    dev = _decode_dev(inp)
    f = synth.as_float64(inp)
    y = binding.ssm_selective_state_update(dev["state"], dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"],
                                           D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"],
                                           delta_softplus=True, out_dtype=torch_dtype("f32"), zoh=True)
    ref, sref, ymag, smag = oracle.selective_state_update(
        f["state"], f["x"], f["delta"], f["A"], f["B"], f["C"], D=f["D"], z=f["z"],
        delta_bias=f["delta_bias"], delta_softplus=True, want_magnitude=True, zoh=True)
    report(f"zoh decode {(B, d, N)} {dt} y", oracle.scaled_error(download(y), ref, ymag), tol_for(dt, "f32"))
    report(f"zoh decode {(B, d, N)} {dt} state", oracle.scaled_error(download(dev["state"]), sref, smag),
           tol_for(dt, "f32"))


def test_zoh_scan_then_decode_matches_longer_scan():
    inp = with_special_A(synth.make_scan_inputs(2, 41, 96, 16, "f32", seed=37, stream=3700))
    dev = scan_inputs_to_device(inp)
    first = {k: (v[:, :-1].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in dev.items()}
    _, h = binding.ssm_selective_scan_fwd(first["u"], first["delta"], dev["A"], first["B"], first["C"],
                                          D=dev["D"], z=first["z"], delta_bias=dev["delta_bias"],
                                          delta_softplus=True, return_final_state=True, zoh=True)
    yd = binding.ssm_selective_state_update(h, dev["u"][:, -1].contiguous(), dev["delta"][:, -1].contiguous(),
                                            dev["A"], dev["B"][:, -1].contiguous(), dev["C"][:, -1].contiguous(),
                                            D=dev["D"], z=dev["z"][:, -1].contiguous(),
                                            delta_bias=dev["delta_bias"], delta_softplus=True, zoh=True)
    ref, href, ymag, hmag = oracle.selective_scan(**_oracle_args(inp), want_magnitude=True, zoh=True)
    report("zoh scan+decode y", oracle.scaled_error(download(yd), ref[:, -1], ymag[:, -1]), 1e-4)
    report("zoh scan+decode state", oracle.scaled_error(download(h), href, hmag), 1e-4)
