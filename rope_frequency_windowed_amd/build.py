"""Builds librfw_atf.so (the HIP kernels and the C ABI) and librfw_probes.so
(the MFMA and HBM microbenchmarks) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librfw_atf.so")
SOURCES = [os.path.join(CSRC, "atf_api.cpp"), os.path.join(CSRC, "atf_kernels.hip")]
PROBE_LIB = os.path.join(PKG, "librfw_probes.so")
PROBE_SOURCES = [os.path.join(CSRC, "atf_probes.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build librfw_atf.so")
    return path


def _compile(out: str, sources, verbose: bool, resource_usage: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops are kept off for every kernel
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + list(sources)
    if resource_usage:
        cmd.insert(2, "-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose or resource_usage:
        print(res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile the attention library and the probe library; always recompiles."""
    _compile(PROBE_LIB, PROBE_SOURCES, verbose, resource_usage)
    return _compile(LIB, SOURCES, verbose, resource_usage)


if __name__ == "__main__":
    import sys
    print(build(verbose=True, resource_usage="--usage" in sys.argv))
