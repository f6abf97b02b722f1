"""Build libmla_verify.so (gfx950) in-tree with hipcc.

    python -m mla_tree_verify_amd.build [--verbose]

The HIP source is compiled for gfx950 only, with packed-fp32 instruction
generation disabled (-target-feature -packed-fp32-ops), and linked into a
shared library that exports the C ABI of include/mla_verify.h.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "mla_verify.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_verify.so")
# the benchmark's MFMA peak probe (not part of the verify path)
PROBE_SRC = os.path.join(PKG, "csrc", "peak_probe.hip")
PROBE_LIB = os.path.join(PKG, "libmla_verify_probe.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(resource_usage: bool = False):
    flags = [
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-I", INCLUDE,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # latency-oriented machine scheduling: keeps several LDS reads in flight ahead of the MFMAs
        "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
        "-Wno-unused-result",
    ]
    if resource_usage:
        flags += ["-Rpass-analysis=kernel-resource-usage"]
    return flags


def _compile(src: str, lib: str, verbose: bool, resource_usage: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc()] + compile_flags(resource_usage) + [src, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature name; that warning is harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Builds libmla_verify.so and the benchmark's probe library; returns the former's path."""
    _compile(PROBE_SRC, PROBE_LIB, verbose, False)
    return _compile(SRC, LIB, verbose, resource_usage)


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv, resource_usage="--resource-usage" in sys.argv)
    print(path)
