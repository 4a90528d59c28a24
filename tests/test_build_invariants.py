"""Build invariants of every HIP source (CPU only: compiles to gfx950
assembly and reads it).

* Every kernel keeps FP32 denormals (`.amdhsa_float_denorm_mode_32 3`, no
  flush on input or output): tiles whose scale amax / 448 is an FP32
  subnormal must quantize exactly, and the oracle keeps subnormals too.
* No packed-FP32 arithmetic (`v_pk_fma_f32`, `v_pk_mul_f32`,
  `v_pk_add_f32`): the build disables it, and the kernels' FP32 arithmetic
  is written as scalar operations.
"""
import functools
import os
import re
import shutil

import pytest

from fp8_fine_grained_fp8bs_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


@functools.lru_cache(maxsize=None)
def _asm(src):
    return build.asm(src)


def _code_lines(asm):
    lines = [l.strip() for l in asm.splitlines()]
    return [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]


@pytest.mark.parametrize("src", build.SOURCES)
def test_kernels_keep_fp32_denormals(src):
    asm = _asm(src)
    modes = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", asm)
    if src == "api.hip":
        assert not modes or set(modes) == {"3"}
        return
    assert modes, f"{src}: no kernel descriptors found"
    assert set(modes) == {"3"}, f"{src}: FP32 denormal modes {sorted(set(modes))}"


@pytest.mark.parametrize("src", build.SOURCES)
def test_no_packed_fp32(src):
    code = _code_lines(_asm(src))
    packed = [l for l in code if re.match(r"v_pk_(fma|mul|add)_f32\b", l)]
    assert not packed, f"{src}: packed FP32 instructions: {packed[:3]}"
