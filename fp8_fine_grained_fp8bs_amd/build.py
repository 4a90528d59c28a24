"""Build libfp8bs.so (gfx950 only) in-tree with hipcc.

    python -m fp8_fine_grained_fp8bs_amd.build

Flags: -O3, no fast-math (IEEE division, FP32 subnormals kept),
-ffp-contract=off (every fused multiply-add is written explicitly), and
packed-FP32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8bs.so")
# debug build for race checks: kernels fill their LDS with 0xFF before use
POISON_LIB = os.path.join(PKG, "libfp8bs_poison.so")
SOURCES = ["api.hip", "quant.hip", "requant.hip", "gemm.hip", "gemm_bf16a.hip", "e5m6.hip", "swiglu.hip"]
LDS_SOURCES = ["quant.hip", "requant.hip", "gemm.hip", "gemm_bf16a.hip"]   # the sources whose kernels use LDS
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfp8bs")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _compile(src: str, poison: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ("_poison.o" if poison else ".o"))
    extra = ["-DFP8BS_POISON_LDS"] if poison else []
    cmd = [hipcc()] + common_flags() + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfp8bs.so next to this file, and
    the LDS-poisoning debug build libfp8bs_poison.so (tests only)."""
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in LDS_SOURCES]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = dict(zip(SOURCES, objs[:len(SOURCES)]))
    poisoned = dict(zip(LDS_SOURCES, objs[len(SOURCES):]))
    _link([plain[s] for s in SOURCES], LIB)
    _link([poisoned.get(s, plain[s]) for s in SOURCES], POISON_LIB)
    if verbose:
        print("built", LIB, "and", POISON_LIB)
    return LIB


def asm(src: str) -> str:
    """AMD assembly of one source (for inspection of the gfx950 code)."""
    cmd = [hipcc()] + common_flags() + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", "-"]
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout


if __name__ == "__main__":
    build(verbose=True)
