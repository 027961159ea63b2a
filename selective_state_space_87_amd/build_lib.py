"""Build libssm_scan.so (HIP, gfx950) in-tree with hipcc.

    python -m selective_state_space_87_amd.build_lib

Objects go to _build/ at the repository root; the library to
selective_state_space_87_amd/lib/libssm_scan.so, and the benchmark's rate
probes (include/ssm_probe.h) to selective_state_space_87_amd/lib/libssm_probe.so.
Always recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libssm_scan.so")
PROBE_LIB = os.path.join(LIBDIR, "libssm_probe.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 (v_pk_*_f32) is switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I", os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include")]
CXX = os.environ.get("CXX_HOST", "g++")

DEVICE_SOURCES = ["scan_fwd.hip", "scan_fwd_bb.hip", "scan_fwd_bf.hip", "scan_fwd_fb.hip", "scan_fwd_ff.hip",
                  "scan_ckpt_b.hip", "scan_ckpt_f.hip", "scan_bwd.hip", "state_update.hip", "conv1d.hip", "ssd.hip",
                  "scan_noalloc.hip"]
HOST_SOURCES = ["api.cpp", "plan.cpp"]
PROBE_SOURCES = ["probe.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = []
    for s in DEVICE_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append(([HIPCC] + DEVICE_FLAGS + ["-c", os.path.join(CSRC, s), "-o", o], o))
    for s in HOST_SOURCES:  # HIP-free host code: the C-ABI validation front end
        o = os.path.join(BUILD, s + ".o")
        jobs.append(([CXX] + HOST_FLAGS + ["-c", os.path.join(CSRC, s), "-o", o], o))
    probe_jobs = []
    for s in PROBE_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        probe_jobs.append(([HIPCC] + DEVICE_FLAGS + ["-c", os.path.join(CSRC, s), "-o", o], o))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs) + len(probe_jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs + probe_jobs))
    for lib, objs in ((LIB, jobs), (PROBE_LIB, probe_jobs)):
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for _, o in objs]
             + ["-Wl,-soname," + os.path.basename(lib)], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
