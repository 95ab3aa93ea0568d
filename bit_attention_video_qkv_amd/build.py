"""Builds libfp8attn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8attn.so")
SOURCES = ["fp8attn_api.hip", "fp8attn_quant.hip", "fp8attn_attn.hip", "fp8attn_cluster.hip", "fp8attn_sol.hip",
           "fp8attn_diag.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 instructions stay disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build_issue_rates() -> str:
    """The instruction-issue microbenchmark (csrc/issue_rates.hip), a stand-alone executable."""
    exe = os.path.join(HERE, "issue_rates")
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(CSRC, "issue_rates.hip"), "-o", exe + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building issue_rates")
    os.replace(exe + ".tmp", exe)
    return exe


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp8attn")
    if verbose:
        sys.stderr.write(res.stderr)
    # every kernel launch stub must resolve (a toolchain quirk can leave them undefined)
    import ctypes
    ctypes.CDLL(tmp, mode=ctypes.RTLD_GLOBAL | os.RTLD_NOW)
    os.replace(tmp, LIB)
    build_issue_rates()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
