"""Build libmq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in place, and
libmq_measure.so (a plain-read kernel the benchmark uses as its HBM read ceiling; the
product never loads it).

Usage: python -m block_quantized_matmul_mq_amd.build   (or build() from Python)

Flags: -O3, no fast-math (the activation quantizer needs IEEE f32 division and
round-half-even), packed-FP32 instructions disabled, f32 denormals kept.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmq.so")
MEASURE_SRC = os.path.join(HERE, "measure", "read_ceiling.hip")
MEASURE_LIB = os.path.join(HERE, "libmq_measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["mq_api.hip", "quantize_act.hip", "gemv.hip", "gemv_mfma.hip", "gemv_q8.hip", "mmq.hip", "mmq_kw.hip", "mmq_f6.hip", "repack.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src):
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fno-gpu-rdc", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [MEASURE_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], MEASURE_LIB)
    if verbose:
        print(f"built {LIB} and {MEASURE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
