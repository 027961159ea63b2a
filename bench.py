#!/usr/bin/env python3
"""Benchmark: selective scan throughput on one MI355X, plus the decode state update.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one selective scan (all of: load/convert, softplus step size,
discretise, recurrence, readout, D skip, silu gate, bf16 store, final state)
over the Mamba-1.4B-shaped layer: B=4, L=8192, d_inner=4096, N=16, bf16
u/delta/B/C/z, float32 A/D/state, bf16 y, h_final exported. Inputs are
synthetic (seeded, see selective_state_space_87_amd/synth.py) and resident in
HBM before the timed region. Prints one JSON line.

Also reported in the same line: the scan kernel's roofline (VALU-bound: the
transition needs one transcendental per state update), the float64 CPU
oracle timed on a bounded sample of the same workload, and the decode state
update (128 x 4096 x 128 float32 state, 1000 chained steps).
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan G state-updates/s (B·L·d·N) + % HBM/VALU roofline, 1 MI355X"
UNIT = "G state-updates/s"

# MI355X constants (vendor figures): 256 CUs at 2.4 GHz, 8.0 TB/s HBM3E.
CUS, CLOCK_HZ, HBM_BPS = 256, 2.4e9, 8.0e12
# VALU issue model of gfx950: 4 SIMD x 16 lanes = 64 lane-slots per clock per CU
# for full-rate fp32 ops; transcendentals (exp, log, rcp) take 2 slots (half rate,
# no co-issue with FMA-pipe ops). Packed fp32 is not used.
SLOTS_PER_CLK_CU = 64
VALU_PEAK_SLOTS = CUS * SLOTS_PER_CLK_CU * CLOCK_HZ          # 3.93e13 lane-slots/s
TRANS_SLOTS = 2
# Algorithmic VALU work of the method (not of any implementation):
#   per state update (b,l,d,n): exp(dt*A) [trans], dt*A, (dt*u)*B, Abar*h + .., C*h + ..
#   per (b,l,d): softplus = exp, log [2 trans] + 2 adds; dt*u; D*u + y;
#                silu gate = exp, rcp [2 trans] + add, mul z, mul y.
SLOTS_PER_UPDATE = TRANS_SLOTS + 4
SLOTS_PER_BLD = 4 * TRANS_SLOTS + 2 + 1 + 1 + 3


def scan_alg_bytes(B, L, d, N, in_bytes, out_bytes, final_state):
    """Algorithmic HBM bytes of one scan: each input read once, each output written once."""
    b = B * L * d * in_bytes * 3            # u, delta, z
    b += B * L * N * in_bytes * 2           # B, C
    b += d * N * 4 + d * 4 * 2              # A, D, delta_bias
    b += B * L * d * out_bytes              # y
    if final_state:
        b += B * d * N * 4                  # h_final
    return b


def decode_alg_bytes(B, d, N, in_bytes=4, out_bytes=4):
    state = 2 * B * d * N * 4
    return state, state + B * d * in_bytes * 3 + B * d * out_bytes + 2 * B * N * in_bytes + d * N * 4 + 2 * d * 4


# The sources each kernel's counter summary depends on: a summary in
# profiles/ is used only while these files hash to the value it records.
KERNEL_SOURCES = {
    "scan": ["scan_fwd_impl.h", "scan_fwd.hip", "scan_fwd_bb.hip", "bc_pack.h", "device_math.h", "kernels.h",
             "plan.cpp"],
    "decode": ["state_update.hip", "device_math.h", "kernels.h"],
    "ssd": ["ssd.hip", "device_math.h", "kernels.h"],
    "conv": ["conv1d.hip", "device_math.h", "kernels.h"],
    "bwd": ["scan_bwd.hip", "scan_fwd_impl.h", "scan_ckpt_b.hip", "bc_pack.h", "device_math.h", "kernels.h",
            "plan.cpp"],
}


def kernel_source_hash(kernel="scan"):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "selective_state_space_87_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(profile_name, src_hash):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (same source hash); else None."""
    p = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m_hash = re.search(r"source_hash:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_hash and m_b) or m_hash.group(1) != src_hash:
        return None
    return float(m_b.group(1))


def valu_counters(profile_name, src_hash):
    """Issued / algorithmic VALU lane-slots and VALU busy of a kernel, from its
    committed rocprofv3 counter summary, if that was taken on the current
    kernel sources (same source hash); else None."""
    p = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m_hash = re.search(r"source_hash:\s*([0-9a-f]+)", txt)
    m_ratio = re.search(r"issued / algorithmic:\s*\**([0-9.]+)", txt)
    m_busy = re.search(r"VALU busy[^:]*:\s*([0-9.]+)", txt)
    if not (m_hash and m_ratio and m_busy) or m_hash.group(1) != src_hash:
        return None
    return {"issued_per_algorithmic_slot": float(m_ratio.group(1)), "valu_busy": float(m_busy.group(1)),
            "profile": profile_name}


# The engine clock takes tens of milliseconds of load to reach its steady
# state; a run that times its steps right after a few warm-up calls measures
# part of the ramp. Every timed region below is therefore preceded by this
# much wall time of the same launches (on top of the requested warm-up).
SETTLE_S = 0.5


def settle(torch, fn, seconds):
    """Launch fn back to back for `seconds` of wall time; return the count."""
    if seconds <= 0:
        return 0
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def timed_steps(torch, stream, fn, steps):
    """Time exactly `steps` calls of fn with an event between consecutive
    calls on `stream`: (wall ms per call, event ms per call, median event ms)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return wall_ms, ev[0].elapsed_time(ev[steps]) / steps, per[len(per) // 2]


def _oracle_block(args):
    """Pool worker: the float64 oracle on channels [c0, c1) of the scan inputs
    held in shared memory (storage form), single-threaded. Returns seconds."""
    import numpy as np
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits

    import oracle   # NumPy only (the package, which imports torch, is not loaded here)

    def widen(a):
        if dtype == "bf16":
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)

    names, shapes, dtype, c0, c1, steps, small = args
    shms = {k: shared_memory.SharedMemory(name=n) for k, n in names.items()}
    try:
        st = np.uint16 if dtype == "bf16" else np.float32
        arr = {k: np.ndarray(shapes[k], dtype=st, buffer=shms[k].buf) for k in names}
        sl = {k: widen(np.ascontiguousarray(arr[k][:, :steps, c0:c1])) for k in ("u", "delta", "z")}
        for k in ("B", "C"):
            sl[k] = widen(np.ascontiguousarray(arr[k][:, :steps]))
        A, D, bias = (np.asarray(v, dtype=np.float64) for v in small)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.selective_scan(sl["u"], sl["delta"], A[c0:c1], sl["B"], sl["C"], D=D[c0:c1], z=sl["z"],
                                  delta_bias=bias[c0:c1], delta_softplus=True)
            return time.perf_counter() - t0
    finally:
        for m in shms.values():
            m.close()


def cpu_pool_baseline(inp, cores):
    """The oracle over independent channel blocks on `cores` processes (all of
    the workload's steps): (seconds of wall time, state updates)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from multiprocessing import shared_memory

    import numpy as np

    dt = inp["in_dtype"]
    Bt, L, d = inp["u"].shape
    N = inp["A"].shape[1]
    names, shapes, shms = {}, {}, []
    try:
        for k in ("u", "delta", "z", "B", "C"):
            a = np.ascontiguousarray(inp[k])
            m = shared_memory.SharedMemory(create=True, size=a.nbytes)
            shms.append(m)
            np.ndarray(a.shape, dtype=a.dtype, buffer=m.buf)[...] = a
            names[k], shapes[k] = m.name, a.shape
        small = (inp["A"], inp["D"], inp["delta_bias"])
        blocks = 4 * cores
        edges = [d * i // blocks for i in range(blocks + 1)]
        tasks = [(names, shapes, dt, edges[i], edges[i + 1], L, small) for i in range(blocks) if edges[i + 1] > edges[i]]
        # Fresh interpreters (spawn): the workers hold no GPU state. A worker
        # that dies raises here (BrokenProcessPool) instead of being replaced.
        with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn")) as pool:
            list(pool.map(_oracle_block, [(names, shapes, dt, 0, 1, 16, small)] * cores, timeout=300))
            t0 = time.perf_counter()
            list(pool.map(_oracle_block, tasks, timeout=600))
            wall = time.perf_counter() - t0
    finally:
        for m in shms:
            m.close()
            m.unlink()
    return wall, Bt * L * d * N


def cpu_baseline(inp, sample_steps):
    """The float64 oracle, as it stands, on the first `sample_steps` time steps
    of the same workload (all batches, channels and states)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from selective_state_space_87_amd import synth

    dt = inp["in_dtype"]
    S = min(sample_steps, inp["u"].shape[1])
    sl = {k: synth.to_float64(np.ascontiguousarray(inp[k][:, :S]), dt) for k in ("u", "delta", "B", "C", "z")}
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.selective_scan(sl["u"], sl["delta"], inp["A"].astype(np.float64), sl["B"], sl["C"],
                              D=inp["D"].astype(np.float64), z=sl["z"],
                              delta_bias=inp["delta_bias"].astype(np.float64), delta_softplus=True)
        t = time.perf_counter() - t0
    Bt, _, d = inp["u"].shape
    N = inp["A"].shape[1]
    ups = Bt * S * d * N
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    one = {"value": ups / t / 1e9, "unit": UNIT, "cores": 1, "kind": "oracle",
           "sample": f"float64 NumPy oracle, first {S} of {inp['u'].shape[1]} time steps of the same "
                     f"workload (B={Bt}, d={d}, N={N}; {ups:.3e} state updates) in {t:.1f} s on one "
                     f"thread of {cpu}"}
    # All the cores this process may use (at most 16, the host share of one
    # GPU): a process pool over independent channel blocks, every time step.
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    wall, ups_all = cpu_pool_baseline(inp, cores)
    return {"value": ups_all / wall / 1e9, "unit": UNIT, "cores": cores, "kind": "oracle",
            "sample": f"float64 NumPy oracle over all {inp['u'].shape[1]} time steps of the same workload "
                      f"(B={Bt}, d={d}, N={N}; {ups_all:.3e} state updates), {4 * cores} channel blocks on a "
                      f"pool of {cores} single-threaded processes, {wall:.1f} s wall on {cpu}",
            "single_thread": one}


def bench_scan(args, torch, binding, synth):
    w = synth.WORKLOADS[args.workload]
    inp = synth.workload_inputs(args.workload)
    dev = torch.device("cuda:0")
    dt = inp["in_dtype"]

    def up(a, kind):
        import numpy as np
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: up(inp[k], dt) for k in ("u", "delta", "B", "C", "z")}
    for k in ("A", "D", "delta_bias"):
        t[k] = up(inp[k], "f32")
    out_dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    y = torch.empty(w.batch, w.seqlen, w.dim, dtype=out_dtype, device=dev)
    hf = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev)

    def step():
        binding.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                       delta_bias=t["delta_bias"], delta_softplus=True, y=y,
                                       h_final=hf if w.final_state else None, out_dtype=out_dtype)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settled = settle(torch, step, args.settle_s)
    wall_ms, kern_ms, kern_med_ms = timed_steps(torch, stream, step, args.steps)

    # Cold-cache kernel time: flush the 256 MB MALL and the L2s before each launch.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(3):
        flush.fill_(1)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        step()
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    del flush
    return w, inp, wall_ms, kern_ms, sorted(cold)[1], kern_med_ms, settled


def bench_decode(args, torch, binding, synth):
    w = synth.WORKLOADS[4]
    d = synth.workload_inputs(4)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(d[k]).to(dev) for k in ("state", "x", "delta", "B", "C", "z", "A", "D", "delta_bias")}
    y = torch.empty(w.batch, w.dim, dtype=torch.float32, device=dev)

    def step():
        binding.ssm_selective_state_update(t["state"], t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],
                                           z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, y=y)

    stream = torch.cuda.current_stream(dev)
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    settle(torch, step, 0.2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.decode_steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    state_b, alg_b = decode_alg_bytes(w.batch, w.dim, w.dstate)
    gbs = alg_b / (us * 1e-6) / 1e9
    traffic = counter_traffic("state_update_decode_counters.md", kernel_source_hash("decode"))
    return {
        "workload": f"{w.name} (batch={w.batch}, d_inner={w.dim}, N={w.dstate}, f32, "
                    f"{args.decode_steps} chained steps, same token)",
        "us_per_step": us,
        "state_GBps": state_b / (us * 1e-6) / 1e9,
        "G_updates_per_s": w.batch * w.dim * w.dstate / (us * 1e-6) / 1e9,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_BPS / 1e9, "unit": "GB/s",
                     "frac": gbs / (HBM_BPS / 1e9), "traffic": traffic,
                     "alg_bytes_per_launch": alg_b},
    }


def copy_calibration(torch, mib):
    """Three device-to-device copies of `mib` MiB (reads and writes mib MiB each)."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def conv_alg_bytes(B, L, d, K, in_bytes, out_bytes):
    """x read once, y written once, weight + bias, carried state read and written."""
    return B * L * d * (in_bytes + out_bytes) + d * K * 4 + d * 4 + 2 * B * d * (K - 1) * 4


def _timed(torch, fn, reps, warm, settle_s=0.2):
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    settle(torch, fn, settle_s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps  # microseconds


def hbm_roofline(alg_b, us, traffic=None):
    gbs = alg_b / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_BPS / 1e9, "unit": "GB/s",
            "frac": gbs / (HBM_BPS / 1e9), "traffic": traffic, "alg_bytes_per_launch": alg_b}


def bench_conv(args, torch, binding, synth):
    """The causal depthwise conv1d + SiLU before the scan (1.4B-shaped layer, width 4,
    bf16 in and out, state carried in and out) and its decode update (batch 128,
    d_inner 4096, width 4, float32)."""
    import numpy as np
    dev = torch.device("cuda:0")
    B, L, d, K = 4, 8192, 4096, 4
    ci = synth.make_conv_inputs(B, L, d, K, "bf16", seed=0, stream=700)
    x = torch.from_numpy(ci["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(ci["weight"]).to(dev)
    bias = torch.from_numpy(ci["bias"]).to(dev)
    s_in = torch.from_numpy(ci["state"]).to(dev)
    y = torch.empty_like(x)
    s_out = torch.empty_like(s_in)
    us = _timed(torch, lambda: binding.ssm_causal_conv1d_fwd(x, w, bias, s_in, y=y, state_out=s_out),
                args.conv_steps, 10)
    alg = conv_alg_bytes(B, L, d, K, 2, 2)
    fwd = {"workload": f"causal conv1d + SiLU (batch={B}, seqlen={L}, d_inner={d}, width={K}, bf16 in/out, "
                       f"state in/out)", "us_per_call": us,
           "roofline": hbm_roofline(alg, us, counter_traffic("conv1d_mamba14b_counters.md",
                                                             kernel_source_hash("conv")))}
    del x, y
    if args.no_conv_update:
        return fwd, None
    Bd = 128
    ui = synth.make_conv_inputs(Bd, 1, d, K, "f32", seed=0, stream=701)
    xs = torch.from_numpy(ui["x"][:, 0]).to(dev)
    st = torch.from_numpy(ui["state"]).to(dev)
    yu = torch.empty_like(xs)
    us_u = _timed(torch, lambda: binding.ssm_causal_conv1d_update(st, xs, w, bias, y=yu), 1000, 20)
    alg_u = Bd * d * 8 + d * K * 4 + d * 4 + 2 * Bd * d * (K - 1) * 4
    # The same chain with the host out of the loop: 100 steps captured in a
    # HIP graph, replayed 10 times. The graph's result is checked against
    # the same 100 steps launched one by one from the same state (bitwise).
    s0 = st.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.ssm_causal_conv1d_update(st, xs, w, bias, y=yu)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(100):
            binding.ssm_causal_conv1d_update(st, xs, w, bias, y=yu)
    st.copy_(s0)
    for _ in range(100):
        binding.ssm_causal_conv1d_update(st, xs, w, bias, y=yu)
    eager = st.clone()
    replay_ok = True
    for _ in range(3):                       # eager work and syncs between the replays
        st.copy_(s0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replay_ok = replay_ok and bool(torch.equal(st, eager))
    stream = torch.cuda.current_stream()
    settle(torch, graph.replay, 0.1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us_g = e0.elapsed_time(e1) * 1e3 / 1000
    del graph
    upd = {"workload": f"causal conv1d update (batch={Bd}, d_inner={d}, width={K}, float32, 1000 chained steps)",
           "us_per_step": us_g, "timing": "100 chained steps per captured graph, replayed 10 times",
           "graph_matches_eager": replay_ok, "roofline": hbm_roofline(alg_u, us_g),
           "launch_loop_us_per_step": us_u, "launch_loop_roofline": hbm_roofline(alg_u, us_u)}
    return fwd, upd


# Algorithmic VALU work of the backward, per state update: the transition
# exp(dt*A) [2 + 1 slots], the state and readout recomputed [2], the adjoint
# lam = dp*C + mu and mu = a*lam [2], dA [2], d(dt) [3], du [2], dB and dC
# contributions [2]; per (b,l,d): softplus and its derivative, silu and its
# derivative, dz, dD, bias and output scaling [~20].
BWD_SLOTS_PER_UPDATE = 16
BWD_SLOTS_PER_BLD = 20


# Exact zero-order hold: the input coefficient k = (exp(dt*A) - 1) / A costs,
# per state update, k itself [1: fma(Abar, 1/A, -1/A)] and one more product
# (u*B, then k*(u*B), in place of (dt*u)*B); dt*u per (b,l,d) is no longer
# needed. The series branch near dt*A = 0 that keeps k accurate there (3 ops,
# a compare and a select) is counted as implementation overhead, not here.
ZOH_SLOTS_PER_UPDATE = SLOTS_PER_UPDATE + 2
ZOH_SLOTS_PER_BLD = SLOTS_PER_BLD - 1


def bench_zoh(args, torch, binding, synth, inp):
    """The scan of the 1.4B-shaped layer with the exact zero-order-hold option."""
    import numpy as np
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dt = inp["in_dtype"]

    def up(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: up(inp[k], dt) for k in ("u", "delta", "B", "C", "z")}
    for k in ("A", "D", "delta_bias"):
        t[k] = up(inp[k], "f32")
    out_dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    y = torch.empty(w.batch, w.seqlen, w.dim, dtype=out_dtype, device=dev)
    hf = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev)
    fn = lambda: binding.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],  # noqa
                                                z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True,
                                                y=y, h_final=hf if w.final_state else None,
                                                out_dtype=out_dtype, zoh=True)
    us = _timed(torch, fn, args.zoh_steps, 20)
    ups = w.updates
    slots = ups * ZOH_SLOTS_PER_UPDATE + w.batch * w.seqlen * w.dim * ZOH_SLOTS_PER_BLD
    ach = slots / (us * 1e-6) / 1e12
    return {"workload": f"{w.name}, exact zero-order hold", "us_per_call": us,
            "G_updates_per_s": ups / (us * 1e-6) / 1e9,
            "roofline": {"bound": "alu", "achieved": ach, "peak": VALU_PEAK_SLOTS / 1e12, "unit": "Tslot/s",
                         "frac": ach / (VALU_PEAK_SLOTS / 1e12), "traffic": None, "alg_slots_per_launch": slots}}


def bench_large_state(args, torch, binding, synth, B=4, L=2048):
    """The scan at N = 128 (B and C staged through LDS), on the 1.4B layer's
    width: (4, 2048, 4096, 128), bf16 in and out, 256 channel blocks; or
    (2, 8192, 4096, 128), 128 blocks, where each channel's states run in two
    blocks (partial readouts through the workspace and a combine pass). For
    the latter, the allocation-free entry point, which keeps one block per
    channel at this size, is timed beside it."""
    import numpy as np
    d, N = 4096, 128
    inp = synth.make_scan_inputs(B, L, d, N, "bf16", seed=0, stream=4200)
    dev = torch.device("cuda:0")

    def up(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: up(inp[k], "bf16") for k in ("u", "delta", "B", "C", "z")}
    for k in ("A", "D", "delta_bias"):
        t[k] = up(inp[k], "f32")
    y = torch.empty(B, L, d, dtype=torch.bfloat16, device=dev)
    hf = torch.empty(B, d, N, dtype=torch.float32, device=dev)
    fn = lambda: binding.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"],  # noqa
                                                z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True,
                                                y=y, h_final=hf, out_dtype=torch.bfloat16)
    us = _timed(torch, fn, args.large_state_steps, 10)
    ups = B * L * d * N
    slots = ups * SLOTS_PER_UPDATE + B * L * d * SLOTS_PER_BLD
    ach = slots / (us * 1e-6) / 1e12
    split = binding.ssm_scan_workspace_bytes(B, L, d, N) >= 2 * B * L * d * 4
    out = {"workload": f"scan, N=128 (batch={B}, seqlen={L}, d_inner={d}, bf16 in/out, h_final)"
                       + (", states split over two blocks per channel" if split else ""),
           "us_per_call": us, "G_updates_per_s": ups / (us * 1e-6) / 1e9,
           "roofline": {"bound": "alu", "achieved": ach, "peak": VALU_PEAK_SLOTS / 1e12, "unit": "Tslot/s",
                        "frac": ach / (VALU_PEAK_SLOTS / 1e12), "traffic": None, "alg_slots_per_launch": slots}}
    if split and binding.ssm_scan_workspace_bytes(B, L, d, N) > (64 << 20):
        fn1 = lambda: binding.ssm_selective_scan_fwd_noalloc(t["u"], t["delta"], t["A"], t["B"], t["C"],  # noqa
                                                             y, D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                                             delta_softplus=True, h_final=hf)
        us1 = _timed(torch, fn1, max(3, args.large_state_steps // 2), 3)
        out["one_block_per_channel_us_per_call"] = us1
    return out


# Mamba-2 SSD layer, chunked matrix form with chunks of Q = 64 steps. Its
# algorithmic work per (batch, chunk): the scores C B^T once (2 Q^2 N, shared
# by every head), and per head S X (2 Q^2 P), the entering state's readout
# C H (2 Q N P) and the exit state B^T X (2 Q N P). With bfloat16 inputs the
# products run on the bfloat16 matrix cores (2.5 PFLOP/s dense), where these
# flops take a third of the time the algorithmic HBM bytes take at 8 TB/s:
# the layer's roofline is HBM.
SSD_Q = 64
MFMA_BF16_PEAK = 2.5e15


def ssd_alg_flops(B, L, H, P, N):
    chunks = -(-L // SSD_Q)
    return B * chunks * (2 * SSD_Q * SSD_Q * N + H * (2 * SSD_Q * SSD_Q * P + 4 * SSD_Q * N * P))


def bench_ssd(args, torch, binding, synth):
    """Mamba-2-shaped SSD layer: (4, 8192), 64 heads of 64 channels, N = 128, bf16 in and out."""
    import numpy as np
    B, L, H, P, N = 4, 8192, 64, 64, 128
    inp = synth.make_ssd_inputs(B, L, H, P, N, "bf16", seed=0, stream=4800)
    dev = torch.device("cuda:0")

    def up(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: up(inp[k], "bf16") for k in ("x", "dt", "B", "C", "z")}
    for k in ("A", "D", "dt_bias"):
        t[k] = up(inp[k], "f32")
    y = torch.empty(B, L, H, P, dtype=torch.bfloat16, device=dev)
    hf = torch.empty(B, H, P, N, dtype=torch.float32, device=dev)
    fn = lambda: binding.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],  # noqa
                                     dt_bias=t["dt_bias"], dt_softplus=True, y=y, h_final=hf,
                                     out_dtype=torch.bfloat16)
    us = _timed(torch, fn, args.ssd_steps, 5)
    flops = ssd_alg_flops(B, L, H, P, N)
    alg_b = 3 * B * L * H * P * 2 + B * L * H * 2 + 2 * B * L * N * 2 + B * H * P * N * 4 + 3 * H * 4
    tflops = flops / (us * 1e-6) / 1e12
    traffic = counter_traffic("ssd_mamba2_counters.md", kernel_source_hash("ssd"))
    rl = hbm_roofline(alg_b, us, traffic)
    rl.update({"alg_flops_per_launch": flops, "mfma_dtype": "bf16", "mfma_TFLOPs": tflops,
               "mfma_peak_TFLOPs": MFMA_BF16_PEAK / 1e12, "mfma_frac": tflops / (MFMA_BF16_PEAK / 1e12)})
    return {"workload": f"Mamba-2-shaped SSD layer (batch={B}, seqlen={L}, heads={H}, headdim={P}, "
                        f"d_state={N}, bf16 in/out, h_final), chunks of {SSD_Q}",
            "us_per_call": us, "G_updates_per_s": B * L * H * P * N / (us * 1e-6) / 1e9,
            "roofline": rl}


def bench_bwd(args, torch, binding, synth, inp):
    """Backward of the selective scan on the 1.4B-shaped layer (float32 dy)."""
    import numpy as np
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dt = inp["in_dtype"]

    def up(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: up(inp[k], dt) for k in ("u", "delta", "B", "C", "z")}
    for k in ("A", "D", "delta_bias"):
        t[k] = up(inp[k], "f32")
    dy = torch.from_numpy((np.random.default_rng(26).standard_normal(inp["u"].shape) * 0.1)
                          .astype(np.float32)).to(dev)
    ws = torch.empty(binding.ssm_scan_bwd_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate),
                     dtype=torch.uint8, device=dev)
    fn = lambda: binding.ssm_selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, D=t["D"],  # noqa
                                                z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True,
                                                workspace=ws)
    us = _timed(torch, fn, args.bwd_steps, 2)
    ups = w.updates
    slots = ups * BWD_SLOTS_PER_UPDATE + w.batch * w.seqlen * w.dim * BWD_SLOTS_PER_BLD
    ach = slots / (us * 1e-6) / 1e12
    out = {"workload": f"{w.name} backward (dy float32, all gradients float32)", "us_per_call": us,
           "G_updates_per_s": ups / (us * 1e-6) / 1e9,
           "roofline": {"bound": "alu", "achieved": ach, "peak": VALU_PEAK_SLOTS / 1e12, "unit": "Tslot/s",
                        "frac": ach / (VALU_PEAK_SLOTS / 1e12), "traffic": None, "alg_slots_per_launch": slots,
                        "valu_counters": valu_counters("scan_bwd_mamba14b_valu.md", kernel_source_hash("bwd"))}}
    # A training step that keeps the forward's states: the forward writes the
    # backward's checkpoints, the backward takes them (no recurrence pass of
    # its own). Timed beside the plain forward (bf16 y, as the headline).
    ck = torch.empty(binding.ssm_scan_checkpoint_bytes(w.batch, w.seqlen, w.dim, w.dstate) // 4,
                     dtype=torch.float32, device=dev)
    y = torch.empty(w.batch, w.seqlen, w.dim, dtype=t["u"].dtype, device=dev)
    hf = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev)
    fws = torch.empty(max(binding.ssm_scan_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate), 1),
                      dtype=torch.uint8, device=dev)
    fkw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, y=y, h_final=hf,
               workspace=fws)
    f_plain = lambda: binding.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **fkw)  # noqa
    f_ckpt = lambda: binding.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"],  # noqa
                                                    checkpoints=ck, **fkw)
    b_ckpt = lambda: binding.ssm_selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy,  # noqa
                                                    D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                                    delta_softplus=True, workspace=ws, checkpoints=ck)
    us_fp = _timed(torch, f_plain, args.bwd_steps, 2)
    us_fc = _timed(torch, f_ckpt, args.bwd_steps, 2)
    us_bc = _timed(torch, b_ckpt, args.bwd_steps, 2)
    out["with_forward_checkpoints"] = {
        "forward_us": us_fp, "forward_writing_checkpoints_us": us_fc, "backward_from_checkpoints_us": us_bc,
        "checkpoint_bytes": ck.numel() * 4,
        "training_step_us": {"recomputing": us_fp + us, "keeping_checkpoints": us_fc + us_bc},
        "backward_roofline": alu_roofline(slots, us_bc)}
    return out


def alu_roofline(slots, us):
    ach = slots / (us * 1e-6) / 1e12
    return {"bound": "alu", "achieved": ach, "peak": VALU_PEAK_SLOTS / 1e12, "unit": "Tslot/s",
            "frac": ach / (VALU_PEAK_SLOTS / 1e12), "traffic": None, "alg_slots_per_launch": slots}


def bench_workload(args, torch, binding, synth, wid, steps):
    """Another named scan workload (the 130M-shaped layer, the long sequence),
    timed like the headline: HIP events on the launch stream around each call
    (B/C pre-pass, and for a chunked plan the summary pass and carry fold too)."""
    import numpy as np
    w = synth.WORKLOADS[wid]
    inp = synth.workload_inputs(wid)
    dev = torch.device("cuda:0")
    dt = inp["in_dtype"]

    def up(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t = {k: up(inp[k], dt) for k in ("u", "delta", "B", "C", "z")}
    for k in ("A", "D", "delta_bias"):
        t[k] = up(inp[k], "f32")
    del inp
    out_dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    y = torch.empty(w.batch, w.seqlen, w.dim, dtype=out_dtype, device=dev)
    hf = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev) if w.final_state else None
    ws = torch.empty(max(1, binding.ssm_scan_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate)),
                     dtype=torch.uint8, device=dev)

    def step():
        binding.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                       delta_bias=t["delta_bias"], delta_softplus=True, y=y, h_final=hf,
                                       out_dtype=out_dtype, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    step()
    torch.cuda.synchronize()
    settle(torch, step, 0.3)
    _, us_ms, med_ms = timed_steps(torch, stream, step, steps)
    us = us_ms * 1e3
    ups = w.updates
    slots = ups * SLOTS_PER_UPDATE + w.batch * w.seqlen * w.dim * SLOTS_PER_BLD
    return {"workload": f"{w.name} (batch={w.batch}, seqlen={w.seqlen}, d_inner={w.dim}, d_state={w.dstate}, "
                        f"{w.in_dtype} in/out, softplus, gate)",
            "us_per_call": us, "median_us": med_ms * 1e3,
            "chunks": binding.ssm_scan_chunks(w.batch, w.seqlen, w.dim, w.dstate),
            "G_updates_per_s": ups / (us * 1e-6) / 1e9, "roofline": alu_roofline(slots, us),
            "hbm_frac": scan_alg_bytes(w.batch, w.seqlen, w.dim, w.dstate, 2, 2, w.final_state)
                        / (us * 1e-6) / HBM_BPS}


def valu_probe():
    """Issue rates the VALU roofline assumes, measured on this device by
    libssm_probe.so (include/ssm_probe.h)."""
    import ctypes

    class Rates(ctypes.Structure):
        _fields_ = [("exp", ctypes.c_double), ("fma", ctypes.c_double), ("mix", ctypes.c_double),
                    ("mix2", ctypes.c_double), ("copy", ctypes.c_double), ("cus", ctypes.c_int),
                    ("clock_khz", ctypes.c_int)]

    path = os.path.join(ROOT, "selective_state_space_87_amd", "lib", "libssm_probe.so")
    lib = ctypes.CDLL(path)
    lib.ssm_probe_valu.restype = ctypes.c_int
    r = Rates()
    rc = lib.ssm_probe_valu(ctypes.byref(r))
    if rc != 0:
        return {"error": f"ssm_probe_valu returned {rc}"}
    peak = r.cus * SLOTS_PER_CLK_CU * r.clock_khz * 1e3
    return {"cus": r.cus, "clock_GHz": r.clock_khz / 1e6, "peak_Tslot_per_s": peak / 1e12,
            "exp_T_per_s": r.exp / 1e12, "exp_frac_of_slot_peak": r.exp / peak,
            "fma_T_per_s": r.fma / 1e12, "fma_frac_of_slot_peak": r.fma / peak,
            "scan_mix_frac_8_waves_per_simd": r.mix / peak,
            "scan_mix_frac_2_waves_per_simd": r.mix2 / peak,
            "copy_GBps": r.copy / 1e9,
            "model": "64 lane-slots per clock per CU; v_exp_f32 2 slots, FMA-pipe ops 1; a 6-slot update "
                     "(2 mul, exp, 2 fma) reaches the peak at full occupancy"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: ~70 ms of warm-up lets the engine clock settle before the
    # timed steps (the first tens of milliseconds of a run are slower).
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2, choices=[0, 1, 2, 3])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the 130M-shaped and long-sequence scans")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of launches before the headline's timed steps (0 under a counter profiler)")
    ap.add_argument("--no-probe", action="store_true", help="skip the VALU / copy rate probes")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=5)
    ap.add_argument("--no-zoh", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--ssd-steps", type=int, default=20)
    ap.add_argument("--no-large-state", action="store_true")
    ap.add_argument("--large-state-steps", type=int, default=20)
    ap.add_argument("--zoh-steps", type=int, default=50)
    ap.add_argument("--conv-steps", type=int, default=50)
    ap.add_argument("--no-conv-update", action="store_true", help="time the conv1d but not its decode update")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=8192)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first copy a buffer of this many MiB device to device three times: a kernel "
                         "of known HBM traffic, against which hardware byte counters are scaled")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world > 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
                  "the scan shards channels with no communication, so only the one-GPU figure is measured.",
                  flush=True)
        sys.exit(2)

    import torch

    from selective_state_space_87_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration_mib > 0:
        copy_calibration(torch, args.copy_calibration_mib)
    w, inp, wall_ms, kern_ms, cold_ms, kern_med_ms, settled = bench_scan(args, torch, binding, synth)
    ups = w.updates
    value = ups / (wall_ms * 1e-3) / 1e9
    in_b = 2 if w.in_dtype == "bf16" else 4
    alg_bytes = scan_alg_bytes(w.batch, w.seqlen, w.dim, w.dstate, in_b, in_b, w.final_state)
    bld = w.batch * w.seqlen * w.dim
    alg_slots = ups * SLOTS_PER_UPDATE + bld * SLOTS_PER_BLD
    achieved = alg_slots / (kern_ms * 1e-3) / 1e12
    peak = VALU_PEAK_SLOTS / 1e12
    src_hash = kernel_source_hash("scan")
    traffic = counter_traffic("scan_fwd_mamba14b_counters.md", src_hash)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "d_inner": w.dim,
                   "d_state": w.dstate, "storage_dtype": w.in_dtype, "state_dtype": "f32",
                   "out_dtype": w.in_dtype, "delta_softplus": True, "gate": w.gate,
                   "final_state": w.final_state},
        "kernel_ms": kern_ms,
        "kernel_median_ms": kern_med_ms,
        "cold_kernel_ms": cold_ms,
        "clock_settle": {"seconds": args.settle_s, "calls": settled},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "Tslot/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "alg_slots_per_launch": alg_slots, "alg_bytes_per_launch": alg_bytes,
                     "hbm_GBps": alg_bytes / (kern_ms * 1e-3) / 1e9,
                     "hbm_frac": alg_bytes / (kern_ms * 1e-3) / HBM_BPS,
                     "source_hash": src_hash,
                     "valu_counters": valu_counters("scan_fwd_mamba14b_valu.md", src_hash)},
    }
    if not args.no_workloads:
        result["mamba130m"] = bench_workload(args, torch, binding, synth, 1, 50)
        result["long_sequence"] = bench_workload(args, torch, binding, synth, 3, 5)
    if not args.no_probe:
        result["valu_probe"] = valu_probe()
    if not args.no_decode:
        result["decode"] = bench_decode(args, torch, binding, synth)
    if not args.no_zoh:
        result["scan_zoh"] = bench_zoh(args, torch, binding, synth, inp)
    if not args.no_ssd:
        result["ssd"] = bench_ssd(args, torch, binding, synth)
    if not args.no_large_state:
        result["scan_n128"] = bench_large_state(args, torch, binding, synth)
        result["scan_n128_split"] = bench_large_state(args, torch, binding, synth, B=2, L=8192)
    if not args.no_bwd:
        result["scan_bwd"] = bench_bwd(args, torch, binding, synth, inp)
    if not args.no_conv:
        result["conv1d"], result["conv1d_update"] = bench_conv(args, torch, binding, synth)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_steps)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
