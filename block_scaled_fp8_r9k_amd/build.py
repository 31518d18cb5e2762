"""Build libr9k.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_scaled_fp8_r9k_amd.build

Every .hip file under csrc/ is compiled by hipcc in parallel and linked into
block_scaled_fp8_r9k_amd/libr9k.so; the benchmark's own kernels (bench_kernels/,
a plain read that gives the bandwidth ceiling) go into libr9k_bench.so, which
the library never loads.  Flags: the numerics need IEEE fp32
division and denormals and no contraction of a*b+c into fma behind the code's
back (the kernels write their fmas explicitly); packed-fp32 instructions are
turned off.  MFMA results go to ordinary VGPRs: every kernel promotes them with
VALU FMAs, and results in the accumulator registers would need a move each.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libr9k.so")
BENCH_SRC = os.path.join(HERE, "bench_kernels")
BENCH_LIB = os.path.join(HERE, "libr9k_bench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    bsrcs = sorted(glob.glob(os.path.join(BENCH_SRC, "*.hip")))
    if bsrcs:
        tmp = BENCH_LIB + ".tmp%d" % os.getpid()
        r = subprocess.run([HIPCC, *CFLAGS, "-shared", "-o", tmp, *bsrcs], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("benchmark kernels failed to build:\n" + r.stderr)
        os.replace(tmp, BENCH_LIB)
        if verbose:
            print(f"built {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build()
