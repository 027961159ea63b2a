"""The binding on a caller's stream other than torch's current one: the
outputs and workspace it allocates belong to that stream, so work that other
streams allocate meanwhile cannot be handed the same memory while the kernels
run. Checked against the float64 oracle, through the C ABI.
"""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_87_amd import binding, synth
from tests.gpu_util import download, oracle_scan, scan_inputs_to_device, tol_for, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def report(name, err, tol):
    print(f"[parity] {name}: scaled error {err:.3e} (tol {tol:.1e})", flush=True)
    assert err <= tol, f"{name}: scaled error {err:.3e} > {tol:.1e}"


def churn(n=8, mib=48):
    """Allocate, fill and free buffers on the current (default) stream."""
    for i in range(n):
        t = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
        t.fill_(i + 1)
        del t


def test_scan_fwd_and_bwd_on_a_side_stream():
    # chunked plan (few channel blocks, long sequence): the workspace holds
    # the packed B/C and the chunk summaries, all used by later launches
    inp = synth.make_scan_inputs(1, 4096, 128, 16, "f32", seed=3, stream=910)
    assert binding.ssm_scan_chunks(1, 4096, 128, 16) > 1
    dev = scan_inputs_to_device(inp)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        y, hf = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"],
                                               z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True,
                                               return_final_state=True, stream=side)
        churn()                    # default-stream allocations while the scan may still run
        outs.append((y, hf))
    side.synchronize()
    ref, href, ymag, hmag = oracle_scan(inp)
    tol = tol_for("f32", "f32")
    for i, (y, hf) in enumerate(outs):
        report(f"side-stream scan rep {i} y", oracle.scaled_error(download(y), ref, ymag), tol)
        report(f"side-stream scan rep {i} h_final", oracle.scaled_error(download(hf), href, hmag), tol)

    # backward on the same side stream, its workspace allocated by the binding
    small = synth.make_scan_inputs(2, 160, 96, 16, "f32", seed=4, stream=911)
    dsm = scan_inputs_to_device(small)
    dy = np.random.default_rng(5).standard_normal((2, 160, 96)).astype(np.float32)
    dy_dev = upload(dy, "f32")
    torch.cuda.synchronize()
    g = binding.ssm_selective_scan_bwd(dsm["u"], dsm["delta"], dsm["A"], dsm["B"], dsm["C"], dy_dev, D=dsm["D"],
                                       z=dsm["z"], delta_bias=dsm["delta_bias"], delta_softplus=True, stream=side)
    churn()
    side.synchronize()
    f = synth.as_float64(small)
    ref_g, mag_g = oracle.selective_scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], dy.astype(np.float64),
                                             D=f["D"], z=f["z"], delta_bias=f["delta_bias"], delta_softplus=True,
                                             want_magnitude=True)
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0"):
        report(f"side-stream bwd {k}", oracle.scaled_error(download(g[k]), ref_g[k], mag_g[k]), tol)
