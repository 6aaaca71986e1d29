"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m sigmoid_top_routing_amd.build

Objects go to sigmoid_top_routing_amd/_build/, the library next to this
file. Every HIP source is compiled with fp contraction off (the router's
fma chain and the combine are bit-specified), correctly rounded fp32
division, and packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBPATH = os.path.join(HERE, "libmoe.so")
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["route.hip", "plan.hip", "gemm.hip", "grouped_gemm.hip", "grouped_gemm_f8.hip",
           "grouped_gemm_f4.hip", "stream.hip", "combine.hip", "norm.hip", "api.cpp"]
# Per-source flags: the FP8 grouped GEMM keeps its MFMA accumulators in VGPRs.
SOURCE_FLAGS = {"grouped_gemm_f8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source and link libmoe.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIBPATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIBPATH)
    if verbose:
        print(f"built {LIBPATH}")
    return LIBPATH


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
