"""Build libfp4idx.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["api.hip", "quantize.hip", "score.hip", "select.hip"]
OUT = os.path.join(HERE, "libfp4idx.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_fma/mul/add_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction results in ordinary VGPRs: the epilogue reads them without
    # v_accvgpr_read copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build_library(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_library(verbose=True))
