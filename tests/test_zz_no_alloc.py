"""The allocation-free scan entry point (ssm_selective_scan_fwd_noalloc)
against the scan forward with a caller workspace, through the C ABI: two
calls in a row on the library's scratch array, the second on a smaller input
(a single-pass plan after a chunked one), each bitwise equal to the forward
with a workspace, and both within the oracle's tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_87_amd import binding, synth
from tests.gpu_util import download, oracle_scan, scan_inputs_to_device, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def run_both(inp, name, chunked):
    B, L, d = inp["u"].shape
    N = inp["A"].shape[1]
    assert (binding.ssm_scan_chunks(B, L, d, N) > 1) == chunked
    dev = scan_inputs_to_device(inp)
    out = torch.bfloat16 if inp["in_dtype"] == "bf16" else torch.float32
    kw = dict(D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True)
    y_ref, h_ref = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"],
                                                  out_dtype=out, return_final_state=True, **kw)
    y = torch.full_like(y_ref, float("nan"))
    h = torch.full_like(h_ref, float("nan"))
    binding.ssm_selective_scan_fwd_noalloc(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], y, h_final=h,
                                           **kw)
    torch.cuda.synchronize()
    print(f"[noalloc] {name}: shape {(B, L, d, N)} chunked={chunked}", flush=True)
    assert torch.equal(y.view(torch.int16) if out == torch.bfloat16 else y.view(torch.int32),
                       y_ref.view(torch.int16) if out == torch.bfloat16 else y_ref.view(torch.int32))
    assert torch.equal(h.view(torch.int32), h_ref.view(torch.int32))
    ref, href, ymag, hmag = oracle_scan(inp)
    ey = oracle.scaled_error(download(y), ref, ymag)
    eh = oracle.scaled_error(download(h), href, hmag)
    print(f"[noalloc] {name}: y err {ey:.2e}, h err {eh:.2e}", flush=True)
    assert ey <= tol_for(inp["in_dtype"], inp["in_dtype"]) and eh <= tol_for(inp["in_dtype"], "f32")


def test_noalloc_two_calls_second_smaller():
    big = synth.make_scan_inputs(1, 8192, 256, 16, "bf16", seed=1, stream=930)
    run_both(big, "first call (chunked plan)", True)
    small = synth.make_scan_inputs(2, 300, 96, 16, "f32", seed=2, stream=931)
    run_both(small, "second call (smaller, single pass)", False)


def test_noalloc_state_split_plans():
    """A scan whose states the plan splits over two blocks: bitwise equal to
    the forward with a workspace where the partial planes fit the scratch
    array; with one block per channel (equal to rounding) where they do not."""
    small = synth.make_scan_inputs(1, 64, 4160, 128, "bf16", seed=3, stream=932)
    assert binding.ssm_scan_workspace_bytes(1, 64, 4160, 128) <= 64 << 20
    run_both(small, "state split within the scratch array", False)
    B, L, d, N = 2, 8192, 4096, 128
    assert binding.ssm_scan_workspace_bytes(B, L, d, N) > 64 << 20
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=4, stream=933)
    dev = scan_inputs_to_device(inp)
    kw = dict(D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True)
    y_ref, h_ref = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"],
                                                  out_dtype=torch.float32, return_final_state=True, **kw)
    y = torch.empty_like(y_ref)
    h = torch.empty_like(h_ref)
    binding.ssm_selective_scan_fwd_noalloc(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], y, h_final=h,
                                           **kw)
    torch.cuda.synchronize()
    ch = np.r_[0, 63, 64, 4095]
    ref, href, ymag, hmag = oracle_scan(inp, channels=ch)
    tol = tol_for("bf16", "f32")
    ey = oracle.scaled_error(download(y)[:, :, ch], ref, ymag)
    eh = oracle.scaled_error(download(h)[:, ch], href, hmag)
    ea = oracle.scaled_error(download(y), download(y_ref), np.abs(download(y_ref)) + 1.0)
    print(f"[noalloc] state split too large for the scratch: y err {ey:.2e}, h err {eh:.2e}, "
          f"vs workspace entry {ea:.2e}", flush=True)
    assert ey <= tol and eh <= tol and ea <= tol
    assert torch.equal(h.view(torch.int32), h_ref.view(torch.int32))


def test_noalloc_refuses_oversized_workspace():
    limit = 64 << 20
    L = (limit // (2 * 16 * 4)) + 64
    assert binding.ssm_scan_workspace_bytes(1, L, 64, 16) > limit
    u = torch.zeros(1, L, 64, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(64, 16, dtype=torch.float32, device="cuda")
    Bm = torch.zeros(1, L, 16, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(u)
    with pytest.raises(binding.SSMError) as e:
        binding.ssm_selective_scan_fwd_noalloc(u, u, A, Bm, Bm, y)
    assert e.value.status == 5  # SSM_E_WORKSPACE
