"""Builds libqmoe.so (the HIP library behind include/qmoe.h) for gfx950.

Every source is compiled by hipcc for --offload-arch=gfx950 with packed
fp32 vector instructions disabled, then linked into one shared library next
to this file.  Object files go to _build/ (not committed).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
SO = os.path.join(HERE, "libqmoe.so")
HOST_SO = os.path.join(HERE, "libqmoe_host.so")  # host leg + residency policy (CPU only, g++)

SOURCES = ["abi.cpp", "route.hip", "batches.hip", "route_batches.hip", "ffn_decode.hip", "ffn_prefill.hip",
           "combine.hip", "layer_decode.hip", "hbm_probe.hip", "prefill_probe.hip", "ffn_prefill_i8.hip"]
# ffn_prefill.hip is compiled once more per block type with only that type's
# GEMM kernels (QMOE_PREFILL_FMT), so the types compile in parallel.
PREFILL_TYPES = [1, 2, 3, 4, 5]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(job) -> str:
    src, defines = job if isinstance(job, tuple) else (job, ())
    tag = "".join(f"_{d.split('=')[-1]}" for d in defines)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = [("ffn_prefill.hip", (f"QMOE_PREFILL_FMT={t}",)) for t in PREFILL_TYPES] + SOURCES
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, jobs_list))
    tmp = SO + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SO)
    build_host()
    return SO


def build_host() -> str:
    """The host library (the host leg and the residency policy): plain g++
    (the AVX2 kernels carry their own target attributes and run only after a
    CPU feature check), OpenMP."""
    tmp = HOST_SO + ".tmp"
    cmd = [os.environ.get("CXX", "g++"), "-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-Wall",
           "-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "host", "host_leg.cpp"),
           os.path.join(HERE, "host", "residency.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host leg build failed:\n{r.stderr}")
    os.replace(tmp, HOST_SO)
    return HOST_SO


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 8))
