"""Compile the HIP libraries for gfx950 (in-tree, next to this file).

libgemm_epilog.so is the epilogue library: each translation unit is compiled in
parallel (the HIP units by hipcc, the host-only plan arithmetic by g++), then linked
into one shared library that exports the C ABI of include/gemm_epilog.h.
libgemm_epilog_probe.so is a measurement aid kept apart from it: the MFMA-rate probe of
include/gemm_epilog_probe.h, which the benchmark loads.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgemm_epilog.so")
PROBE_LIB = os.path.join(HERE, "libgemm_epilog_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "inst_f32.hip", "inst_f16.hip", "inst_bf16.hip",
           "inst_f16_lay1.hip", "inst_f16_lay2.hip", "inst_f16_lay3.hip",
           "inst_bf16_lay1.hip", "inst_bf16_lay2.hip", "inst_bf16_lay3.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


PROBE_SOURCES = ["probe.hip"]

# Host-only C++ (the plan arithmetic): plain g++, no HIP.
HOST_SOURCES = ["plan_host.cpp"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    if src in HOST_SOURCES:
        obj = os.path.join(OBJ, src.replace(".cpp", ".o"))
        cmd = ["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Build both libraries; return the epilogue library's path."""
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), HOST_SOURCES + SOURCES + PROBE_SOURCES))
    n = len(HOST_SOURCES) + len(SOURCES)
    _link(objs[:n], LIB, verbose)
    _link(objs[n:], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
