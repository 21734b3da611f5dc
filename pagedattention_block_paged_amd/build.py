"""Build libpa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.cpp", "profile.cpp", "kv_manager.cpp", "kv_write.hip", "decode.hip", "prefill.hip", "noalloc.hip", "probe.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: str = LIB, extra=()) -> list:
    return [
        "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: the softmax works on them with VALU
        # instructions, and AGPR accumulators cost a copy each way per tile
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        # every atomic here is issued by one lane; the wave-level atomic
        # rewrite would read the result back at once and wait for it
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
        *extra,
        "-o", out,
        *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
