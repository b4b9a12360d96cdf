"""Build libmla_absorb.so (gfx950) in-tree with hipcc.

Usage: python -m mla_latent_kv_absorb_amd.build_lib   (or call build()).
Every source is compiled on every call; objects go to _build/ next to this
file and the shared library lands in this package directory.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla_absorb.so")
# measurement helpers used by the benchmark only (a streaming read and a
# clock probe); not part of the decode library
BENCH_LIB = os.path.join(HERE, "libmla_bench.so")
BENCH_SOURCES = [("bench_kernels.hip", True)]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]
# Keep the compiler from forming packed fp32 VALU instructions.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    ("decode_attn_mfma.hip", True),
    ("decode_attn_bf16.hip", True),
    ("decode_attn_fp8.hip", True),
    ("decode_attn_f32.hip", True),
    ("combine.hip", True),
    ("head_gemm.hip", True),
    ("indexer.hip", True),
    ("cache_append.hip", True),
    ("prefill.hip", True),
    ("noalloc.hip", True),
    ("mla_api.cpp", False),
    ("indexer_api.cpp", False),
    ("host_checks.cpp", None),
]


def _compile(src: str, device) -> str:
    """device True: HIP source for gfx950; False: host C++ that includes the
    HIP runtime headers; None: plain C++ without HIP (built with g++)."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if device is None:
        cmd = [GXX, "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror"]
    else:
        cmd = [HIPCC, *COMMON]
    if device:
        cmd += [*DEVICE, "-x", "hip"]
    elif device is False:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {os.path.basename(lib)}:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(*s), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
