"""GPU parity of the selective scan against the float64 oracle, through the C ABI.

Every case prints its name, shape and error before asserting, so a failing
run on the device names the case.
"""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_87_amd import binding, synth
from tests.gpu_util import (download, oracle_scan, run_scan, scan_inputs_to_device, tol_for, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def report(name, err, tol):
    print(f"[parity] {name}: scaled error {err:.3e} (tol {tol:.1e})", flush=True)
    assert err <= tol, f"{name}: scaled error {err:.3e} > {tol:.1e}"


def check_scan(name, inp, out_dtype="f32", channels=None, gpu_kwargs=None, ora_kwargs=None, h0=None):
    gpu_kwargs = gpu_kwargs or {}
    ora_kwargs = ora_kwargs or {}
    dev = scan_inputs_to_device(inp)
    h0_dev = None if h0 is None else upload(h0, "f32")
    y, hf = run_scan(dev, inp, out_dtype, h0=h0_dev, **gpu_kwargs)
    torch.cuda.synchronize()
    yg, hg = download(y), download(hf)
    if channels is not None:
        yg, hg = yg[:, :, channels], hg[:, channels]
    ref, href, ymag, hmag = oracle_scan(inp, channels=channels, h0=h0, **ora_kwargs, **gpu_kwargs)
    tol = tol_for(inp["in_dtype"], out_dtype)
    report(f"{name} y[{out_dtype}]", oracle.scaled_error(yg, ref, ymag), tol)
    report(f"{name} h_final", oracle.scaled_error(hg, href, hmag), tol_for(inp["in_dtype"], "f32"))
    return yg, hg


# ---------------------------------------------------------------- named workloads

def test_tiny_fp32_workload():
    inp = synth.workload_inputs(0)
    check_scan("tiny fp32 (1,256,64,16)", inp, "f32")
    check_scan("tiny fp32 (1,256,64,16)", inp, "bf16")


@pytest.fixture(scope="module")
def w1():
    return synth.workload_inputs(1)


def test_mamba130m_layer_full(w1):
    check_scan("130m layer (8,2048,1536,16) bf16", w1, "f32")


def test_mamba130m_layer_bf16_out_sampled(w1):
    ch = np.r_[0:5, 63:66, 700, 1020:1024, 1530:1536]
    check_scan("130m layer bf16-out sampled", w1, "bf16", channels=ch)


def test_mamba14b_layer_sampled():
    inp = synth.workload_inputs(2)
    ch = np.r_[0:3, 62:67, 255:258, 2047, 2048, 3000, 4093:4096]
    check_scan("1.4b layer (4,8192,4096,16) bf16 sampled", inp, "f32", channels=ch)
    check_scan("1.4b layer (4,8192,4096,16) bf16-out sampled", inp, "bf16", channels=ch)


def test_long_sequence_sampled():
    inp = synth.workload_inputs(3)
    ch = np.r_[0, 1, 63, 64, 1279, 2558, 2559]
    check_scan("long (1,262144,2560,16) bf16 sampled", inp, "f32", channels=ch)


# ---------------------------------------------------------------- shapes and options

SHAPES = [
    (1, 1, 1, 1, "f32"), (2, 67, 70, 16, "f32"), (1, 129, 130, 3, "bf16"), (3, 5, 64, 5, "f32"),
    (1, 300, 64, 33, "f32"), (2, 100, 33, 64, "bf16"), (1, 64, 256, 8, "f32"), (1, 17, 8, 2, "bf16"),
    (2, 200, 65, 16, "bf16"), (1, 1000, 3, 16, "f32"), (2, 130, 300, 12, "f32"), (4, 63, 128, 4, "bf16"),
    (1, 150, 70, 32, "f32"), (2, 90, 64, 24, "bf16"),
]


@pytest.mark.parametrize("B,L,d,N,dt", SHAPES)
def test_shapes(B, L, d, N, dt):
    inp = synth.make_scan_inputs(B, L, d, N, dt, seed=1, stream=1000 + N)
    rng = np.random.default_rng(N)
    h0 = rng.standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"shape {(B, L, d, N)} {dt}", inp, "f32", h0=h0)
    check_scan(f"shape {(B, L, d, N)} {dt}", inp, "bf16")


# From 64 padded states on, B and C are staged through LDS (no packing
# pre-pass); N = 128 runs sixteen states per lane.
LARGE_N = [
    (2, 100, 70, 128, "bf16"), (1, 67, 64, 128, "f32"), (1, 200, 130, 100, "f32"), (3, 40, 33, 65, "bf16"),
    (1, 129, 200, 64, "f32"), (2, 31, 64, 64, "bf16"), (1, 1, 1, 128, "f32"),
]


@pytest.mark.parametrize("B,L,d,N,dt", LARGE_N)
def test_large_state(B, L, d, N, dt):
    inp = synth.make_scan_inputs(B, L, d, N, dt, seed=4, stream=4000 + N)
    h0 = np.random.default_rng(N + 1).standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"large N {(B, L, d, N)} {dt}", inp, "f32", h0=h0)
    check_scan(f"large N {(B, L, d, N)} {dt}", inp, "bf16")


def test_large_state_chunked_by_plane_size():
    """N = 128 with a batch row's plane above 2^30 bytes (here 65,600 x 4,096
    x 4 bytes) at 64 channel blocks: the summary pass (its own short tiles)
    and the carry fold over sampled channels."""
    B, L, d, N = 1, 65600, 4096, 128
    assert binding.ssm_scan_chunks(2, 8192, 4096, N) == 1   # 128 blocks: one pass
    k = binding.ssm_scan_chunks(B, L, d, N)
    assert k > 1
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=5, stream=4500)
    ch = np.r_[0, 1, 63, 64, 2047, 4095]
    h0 = np.random.default_rng(45).standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"large N chunked x{k} {(B, L, d, N)} bf16 sampled", inp, "f32", h0=h0, channels=ch)


# N > 32 (64 or 128 padded states) at 65 to 128 channel blocks, single pass:
# each channel's states run in two blocks of half of them, whose float32
# partial readouts a combine pass adds (then the skip and the gate).
STATE_SPLIT = [(1, 64, 4160, 128, "bf16"), (2, 40, 4096, 100, "f32"), (1, 33, 4100, 65, "bf16"),
               (1, 70, 4160, 64, "f32"), (2, 35, 4000, 40, "bf16")]


@pytest.mark.parametrize("B,L,d,N,dt", STATE_SPLIT)
def test_state_split(B, L, d, N, dt):
    assert binding.ssm_scan_chunks(B, L, d, N) == 1
    assert binding.ssm_scan_workspace_bytes(B, L, d, N) >= 2 * B * L * d * 4
    inp = synth.make_scan_inputs(B, L, d, N, dt, seed=6, stream=4700 + N)
    h0 = np.random.default_rng(N + 7).standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"state split {(B, L, d, N)} {dt}", inp, "f32", h0=h0)
    check_scan(f"state split {(B, L, d, N)} {dt}", inp, "bf16")


@pytest.mark.parametrize("opts", [dict(use_D=False), dict(use_z=False), dict(use_bias=False, softplus=False)])
def test_state_split_optional_parts(opts):
    inp = synth.make_scan_inputs(1, 48, 4160, 128, "f32", seed=7, stream=4800)
    if opts.get("softplus") is False:
        inp = dict(inp)
        inp["delta"] = np.abs(inp["delta"]) * np.float32(0.05)   # positive raw steps
    check_scan(f"state split options {opts}", inp, "f32", gpu_kwargs=opts)


def test_state_split_in_place_deterministic_and_covering():
    """h_final over h0 in place, bitwise repeatable, every output written
    and nothing else (NaN guards around y), on a split plan."""
    B, L, d, N = 1, 40, 4150, 128
    assert binding.ssm_scan_workspace_bytes(B, L, d, N) >= 2 * B * L * d * 4
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=8, stream=4900)
    dev = scan_inputs_to_device(inp)
    h0 = np.random.default_rng(49).standard_normal((B, d, N)).astype(np.float32) * 0.5
    kw = dict(D=dev["D"], z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True)
    y1, h1 = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"],
                                            h0=upload(h0, "f32"), return_final_state=True,
                                            out_dtype=torch.float32, **kw)
    guard = torch.full((B * L * d + 2048,), float("nan"), dtype=torch.float32, device="cuda")
    y2 = guard[1024:1024 + B * L * d].view(B, L, d)
    hs = upload(h0, "f32")
    binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], h0=hs, y=y2,
                                   h_final=hs, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    print("[parity] state split: in place, repeat, guards", flush=True)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(h1.view(torch.int32), hs.view(torch.int32))
    assert torch.isnan(guard[:1024]).all() and torch.isnan(guard[1024 + B * L * d:]).all()
    assert not torch.isnan(y2).any()


def test_state_split_full_size_sampled():
    """(2, 8192, 4096, 128) bf16: 128 channel blocks, two blocks per channel."""
    B, L, d, N = 2, 8192, 4096, 128
    assert binding.ssm_scan_workspace_bytes(B, L, d, N) >= 2 * B * L * d * 4
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=9, stream=5000)
    ch = np.r_[0, 1, 63, 64, 2047, 4094, 4095]
    h0 = np.random.default_rng(50).standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"state split full size {(B, L, d, N)} bf16 sampled", inp, "bf16", h0=h0, channels=ch)


@pytest.mark.parametrize("opts", [
    dict(use_D=False), dict(use_z=False), dict(use_bias=False), dict(softplus=False, use_bias=False),
    dict(use_D=False, use_z=False, use_bias=False),
])
def test_optional_parts(opts):
    inp = synth.make_scan_inputs(2, 150, 96, 16, "f32", seed=2, stream=2000)
    if opts.get("softplus") is False:
        inp = dict(inp)
        inp["delta"] = np.abs(inp["delta"]) * np.float32(0.05)   # positive raw steps
    check_scan(f"options {opts}", inp, "f32", gpu_kwargs=opts)


def test_empty_sequence_writes_initial_state():
    inp = synth.make_scan_inputs(2, 0, 40, 16, "f32", seed=3, stream=3000)
    dev = scan_inputs_to_device(inp)
    h0 = torch.randn(2, 40, 16, device="cuda")
    y, hf = run_scan(dev, inp, "f32", h0=h0)
    assert y.shape == (2, 0, 40) and torch.equal(hf, h0)
    y, hf = run_scan(dev, inp, "f32", h0=None)
    assert torch.count_nonzero(hf) == 0


def test_final_state_in_place_over_h0():
    inp = synth.make_scan_inputs(2, 90, 70, 16, "bf16", seed=4, stream=4000)
    dev = scan_inputs_to_device(inp)
    h0_np = np.random.default_rng(0).standard_normal((2, 70, 16)).astype(np.float32)
    h = upload(h0_np, "f32")
    binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"],
                                   z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True,
                                   h0=h, h_final=h)
    _, href, _, hmag = oracle_scan(inp, h0=h0_np)
    report("h_final == h0 in place", oracle.scaled_error(download(h), href, hmag), tol_for("bf16", "f32"))


# ---------------------------------------------------------------- invariants (bitwise)

def test_zero_step_keeps_state_bitwise():
    inp = synth.make_scan_inputs(2, 77, 50, 16, "f32", seed=5, stream=5000)
    inp = dict(inp)
    inp["delta"] = np.zeros_like(inp["delta"])
    dev = scan_inputs_to_device(inp)
    h0 = torch.randn(2, 50, 16, device="cuda")
    y, hf = run_scan(dev, inp, "f32", h0=h0, use_bias=False, softplus=False)
    assert torch.equal(hf, h0)
    ref, _, ymag, _ = oracle_scan(inp, h0=download(h0), use_bias=False, softplus=False)
    report("zero step y", oracle.scaled_error(download(y), ref, ymag), 1e-4)


def test_causality_bitwise():
    inp = synth.make_scan_inputs(1, 200, 64, 16, "bf16", seed=6, stream=6000)
    dev = scan_inputs_to_device(inp)
    y1, _ = run_scan(dev, inp, "f32")
    t = 97
    for k in ("u", "delta", "z", "B", "C"):
        dev[k][:, t + 1:] = torch.randn_like(dev[k][:, t + 1:].float()).to(dev[k].dtype)
    y2, _ = run_scan(dev, inp, "f32")
    assert torch.equal(y1[:, :t + 1], y2[:, :t + 1])
    assert not torch.equal(y1[:, t + 1:], y2[:, t + 1:])


def test_deterministic_bitwise():
    inp = synth.make_scan_inputs(2, 500, 300, 16, "bf16", seed=7, stream=7000)
    dev = scan_inputs_to_device(inp)
    y1, h1 = run_scan(dev, inp, "bf16")
    y2, h2 = run_scan(dev, inp, "bf16")
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_split_invariance():
    inp = synth.make_scan_inputs(2, 300, 80, 16, "f32", seed=8, stream=8000)
    dev = scan_inputs_to_device(inp)
    y, h = run_scan(dev, inp, "f32")
    L1 = 131
    first = {k: (v[:, :L1].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in dev.items()}
    second = {k: (v[:, L1:].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in dev.items()}
    ya, ha = run_scan(first, inp, "f32")
    yb, hb = run_scan(second, inp, "f32", h0=ha)
    ref, href, ymag, hmag = oracle_scan(inp)
    report("split y", oracle.scaled_error(download(torch.cat([ya, yb], 1)), ref, ymag), 1e-4)
    report("split h", oracle.scaled_error(download(hb), href, hmag), 1e-4)


def test_scan_then_decode_equals_longer_scan():
    inp = synth.make_scan_inputs(3, 41, 96, 16, "f32", seed=9, stream=9000)
    dev = scan_inputs_to_device(inp)
    first = {k: (v[:, :-1].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in dev.items()}
    _, h = run_scan(first, inp, "f32")
    yd = binding.ssm_selective_state_update(h, dev["u"][:, -1].contiguous(), dev["delta"][:, -1].contiguous(),
                                            dev["A"], dev["B"][:, -1].contiguous(), dev["C"][:, -1].contiguous(),
                                            D=dev["D"], z=dev["z"][:, -1].contiguous(),
                                            delta_bias=dev["delta_bias"], delta_softplus=True)
    ref, href, ymag, hmag = oracle_scan(inp)
    report("scan+decode y", oracle.scaled_error(download(yd), ref[:, -1], ymag[:, -1]), 1e-4)
    report("scan+decode state", oracle.scaled_error(download(h), href, hmag), 1e-4)


def test_nan_stays_in_its_channel():
    inp = synth.make_scan_inputs(2, 120, 70, 16, "f32", seed=10, stream=10000)
    inp = dict(inp)
    u = inp["u"].copy()
    u[1, 30, 5] = np.nan
    inp["u"] = u
    dev = scan_inputs_to_device(inp)
    y, h = run_scan(dev, inp, "f32")
    yn = download(y)
    bad = np.isnan(yn)
    assert bad[1, 30:, 5].all() and bad.sum() == 90
    assert np.isnan(download(h)[1, 5]).all() and np.isnan(download(h)).sum() == 16


def test_guard_bands_and_full_coverage():
    B, L, d, N = 2, 70, 90, 16
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=11, stream=11000)
    dev = scan_inputs_to_device(inp)
    pad = 64
    ybuf = torch.full((2 * pad + B * L * d,), float("nan"), device="cuda")
    y = ybuf[pad:pad + B * L * d].view(B, L, d)
    hbuf = torch.full((2 * pad + B * d * N,), float("nan"), device="cuda")
    hf = hbuf[pad:pad + B * d * N].view(B, d, N)
    binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"], z=dev["z"],
                                   delta_bias=dev["delta_bias"], delta_softplus=True, y=y, h_final=hf,
                                   out_dtype=torch.float32)
    assert torch.isnan(ybuf[:pad]).all() and torch.isnan(ybuf[-pad:]).all()
    assert torch.isnan(hbuf[:pad]).all() and torch.isnan(hbuf[-pad:]).all()
    assert not torch.isnan(y).any() and not torch.isnan(hf).any()


# ---------------------------------------------------------------- sequence chunks
# Shapes with few 64-channel blocks and long sequences run as parallel chunks
# whose summaries are folded in order (ssm_scan_chunks > 1).

CHUNKED = [
    (1, 4096, 64, 16, "f32"), (2, 5000, 100, 16, "bf16"), (1, 3000, 64, 3, "f32"),
    (1, 2100, 130, 32, "bf16"), (1, 2048, 1, 1, "f32"), (3, 6000, 40, 8, "bf16"),
    # two states per lane with padding states (N padded to 16 and 32)
    (1, 2100, 64, 15, "bf16"), (1, 2050, 64, 24, "f32"),
    # from 33 states on: B/C through LDS, the summary pass in 2- or 4-step tiles
    (1, 2100, 64, 128, "bf16"), (1, 2050, 40, 64, "f32"), (2, 2064, 33, 100, "f32"), (1, 3000, 70, 33, "bf16"),
]


@pytest.mark.parametrize("B,L,d,N,dt", CHUNKED)
def test_chunked_shapes(B, L, d, N, dt):
    k = binding.ssm_scan_chunks(B, L, d, N)
    assert k > 1, (B, L, d, N, k)
    inp = synth.make_scan_inputs(B, L, d, N, dt, seed=12, stream=12000 + N)
    rng = np.random.default_rng(L)
    h0 = rng.standard_normal((B, d, N)).astype(np.float32) * 0.5
    check_scan(f"chunked x{k} {(B, L, d, N)} {dt}", inp, "f32", h0=h0)
    check_scan(f"chunked x{k} {(B, L, d, N)} {dt}", inp, "bf16")


@pytest.mark.parametrize("opts", [
    dict(use_D=False, use_z=False), dict(softplus=False, use_bias=False),
])
def test_chunked_optional_parts(opts):
    inp = synth.make_scan_inputs(1, 4100, 64, 16, "f32", seed=13, stream=13000)
    assert binding.ssm_scan_chunks(1, 4100, 64, 16) > 1
    if opts.get("softplus") is False:
        inp = dict(inp)
        inp["delta"] = np.abs(inp["delta"]) * np.float32(0.05)
    check_scan(f"chunked options {opts}", inp, "f32", gpu_kwargs=opts)


def test_chunked_final_state_in_place_over_h0():
    B, L, d, N = 1, 4500, 70, 16
    assert binding.ssm_scan_chunks(B, L, d, N) > 1
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=14, stream=14000)
    dev = scan_inputs_to_device(inp)
    h0_np = np.random.default_rng(1).standard_normal((B, d, N)).astype(np.float32)
    h = upload(h0_np, "f32")
    y = binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"],
                                       z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True,
                                       h0=h, h_final=h, out_dtype=torch.float32)
    ref, href, ymag, hmag = oracle_scan(inp, h0=h0_np)
    report("chunked y with h_final == h0", oracle.scaled_error(download(y[0]), ref, ymag), tol_for("bf16", "f32"))
    report("chunked h_final == h0 in place", oracle.scaled_error(download(h), href, hmag), tol_for("bf16", "f32"))


def test_chunked_guard_bands_causality_determinism():
    B, L, d, N = 2, 4200, 70, 16
    k = binding.ssm_scan_chunks(B, L, d, N)
    assert k > 1
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=15, stream=15000)
    dev = scan_inputs_to_device(inp)
    pad = 64
    ybuf = torch.full((2 * pad + B * L * d,), float("nan"), device="cuda")
    y = ybuf[pad:pad + B * L * d].view(B, L, d)
    hbuf = torch.full((2 * pad + B * d * N,), float("nan"), device="cuda")
    hf = hbuf[pad:pad + B * d * N].view(B, d, N)

    def run():
        binding.ssm_selective_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], D=dev["D"],
                                       z=dev["z"], delta_bias=dev["delta_bias"], delta_softplus=True, y=y,
                                       h_final=hf, out_dtype=torch.float32)
        return y.clone(), hf.clone()

    y1, h1 = run()
    assert torch.isnan(ybuf[:pad]).all() and torch.isnan(ybuf[-pad:]).all()
    assert torch.isnan(hbuf[:pad]).all() and torch.isnan(hbuf[-pad:]).all()
    assert not torch.isnan(y1).any() and not torch.isnan(h1).any()
    y2, h2 = run()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    t = 3 * L // 4   # inside a later chunk
    for key in ("u", "delta", "z", "B", "C"):
        dev[key][:, t + 1:] = torch.randn_like(dev[key][:, t + 1:].float()).to(dev[key].dtype)
    y3, _ = run()
    assert torch.equal(y1[:, :t + 1], y3[:, :t + 1])
    assert not torch.equal(y1[:, t + 1:], y3[:, t + 1:])


def test_chunked_nan_stays_in_its_channel():
    B, L, d, N = 1, 4096, 64, 16
    assert binding.ssm_scan_chunks(B, L, d, N) > 1
    inp = dict(synth.make_scan_inputs(B, L, d, N, "f32", seed=16, stream=16000))
    u = inp["u"].copy()
    u[0, 1500, 9] = np.nan
    inp["u"] = u
    dev = scan_inputs_to_device(inp)
    y, h = run_scan(dev, inp, "f32")
    yn = download(y)
    bad = np.isnan(yn)
    assert bad[0, 1500:, 9].all() and bad.sum() == L - 1500
    assert np.isnan(download(h)[0, 9]).all() and np.isnan(download(h)).sum() == N
