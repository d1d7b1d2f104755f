"""Build liblazyattn.so for gfx950 in-tree with hipcc.

Usage: python -m position_agnostic_kv_pool_amd.build [--resource-usage]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblazyattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["lazyattn_kernels.hip", "lazyattn_host.cpp", "lazyattn_pool.cpp", "lazyattn_runs.cpp"]
# peak probes for the benchmark (MFMA issue rate, HBM streaming read): a library of their own
PROBE_LIB_PATH = os.path.join(PKG, "liblazyattn_probe.so")
PROBE_SOURCES = ["lazyattn_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblazyattn)")


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    _build_one(SOURCES, LIB_PATH, resource_usage, verbose)
    _build_one(PROBE_SOURCES, PROBE_LIB_PATH, False, verbose)
    return LIB_PATH


def _build_one(sources, lib_path, resource_usage, verbose) -> None:
    out_tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed-FP32 instructions are kept out of generated code on this target
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC]
    if resource_usage:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    cmd += [os.path.join(CSRC, s) for s in sources] + ["-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if msgs.strip() and (verbose or resource_usage):
        print(msgs)
    os.replace(out_tmp, lib_path)


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
    print("built", LIB_PATH)
