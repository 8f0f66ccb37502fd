"""Compile libv4moe.so (HIP, gfx950) in place with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libv4moe.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("v4moe_kernels.hip", "v4moe_bwd.hip", "v4moe_api.cpp",
                                                               "v4moe_noalloc.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("v4moe_device.h", "v4moe_internal.h")] + \
    [os.path.join(ROOT, "include", "v4moe.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                      # every fused multiply-add is written out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",     # MFMA results in VGPRs (no accvgpr copies)
    "-fvisibility=hidden",
]


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(SO):
        newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
        if os.path.getmtime(SO) >= newest:
            return SO
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
