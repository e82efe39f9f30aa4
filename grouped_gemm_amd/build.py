"""Build the gfx950 HIP library libmoe.so in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32
instruction generation disabled, then linked into one shared library that
exports the C ABI of include/moe.h.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["route_dispatch.hip", "elementwise.hip", "gemm_stream.hip",
           "gemm_pipe.hip", "decode_layer.hip", "backward.hip", "moe_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-Wno-unused-result"]


# per-file code generation options: the pipelined GEMM keeps MFMA results in
# ordinary VGPRs, so its per-block scaling reads them without copies out of
# the accumulation registers
EXTRA = {"gemm_pipe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    # the rate probes (a standalone program; the library does not use it)
    diag = os.path.join(HERE, "diag_rates")
    cmd = [HIPCC, *FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form", os.path.join(CSRC, "diag_rates.hip"), "-o", diag + ".tmp"]
    cmd = [c for c in cmd if c not in ("-fPIC", "-fvisibility=hidden")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on diag_rates.hip")
    os.replace(diag + ".tmp", diag)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
