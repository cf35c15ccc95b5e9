"""Build the HIP attention library for gfx950 into this package directory.

    python -m scaled_dot_product_qk_amd.build

Produces libattn_gfx950.so next to this file (hipcc, -O3, offload arch
gfx950).  Packed-fp32 instruction selection is switched off for all device
code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_gfx950.so"
SOURCES = ["attn_api.hip"]
HEADERS = ["device_common.h", "fwd_bf16.h", "fwd_f32.h", "fwd_fp8.h", "decode.h", "bwd_bf16.h"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra_flags=None) -> str:
    out = os.path.join(HERE, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if extra_flags:
        cmd[1:1] = list(extra_flags)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and (res.stdout or res.stderr):
        print((res.stdout + res.stderr)[-4000:])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
