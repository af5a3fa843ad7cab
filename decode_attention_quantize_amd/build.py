"""Build librq.so (the C-ABI HIP library) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librq.so")
# the benchmark's read-rate calibration kernel, a library of its own (not librq's interface)
CALIB_SRC = os.path.join(CSRC, "calib", "rq_calib_read.hip")
CALIB_LIB = os.path.join(PKG, "librq_calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# per-source extra flags: the append kernel takes its rounding decisions in fp64
# and must not contract products and sums into fused multiply-adds; its inputs
# are finite (rq.h), so min/max need not quiet NaN operands (IEEE mode off: one
# v_max_f64 instead of three)
SOURCES = {
    "rq_api.cpp": ["-x", "hip"],
    "rq_append.hip": ["-ffp-contract=off", "-fno-honor-nans", "-mno-amdgpu-ieee"],
    "rq_decode.hip": [],
    "rq_decode_paged.hip": [],
    "rq_decode_long.hip": [],
    "rq_decode_bf16.hip": [],
    "rq_prefill.hip": [],
}
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          # packed fp32 arithmetic is disabled on purpose for every kernel
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-result"]


def _compile(src: str, build_dir: str, extra: tuple) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC, *COMMON, *SOURCES[src], *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 6, out: str = LIB, extra_flags=(), build_dir: str = BUILD) -> str:
    """Compile every source and link `out` (default: the in-tree librq.so)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(extra_flags)), SOURCES))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if out == LIB:
        build_calib()
    return out


def build_calib(out: str = CALIB_LIB) -> str:
    """Compile and link the read-rate calibration library (used by bench.py only)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *COMMON, "-shared", CALIB_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CALIB_SRC}:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
