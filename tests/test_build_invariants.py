"""Build invariants of every HIP source (CPU only: compiles to gfx950
assembly and reads it).

* Every kernel keeps FP32 denormals (`.amdhsa_float_denorm_mode_32 3`, no
  flush on input or output): tiles whose scale amax / 448 is an FP32
  subnormal must quantize exactly, and the oracle keeps subnormals too.
* No packed-FP32 arithmetic (`v_pk_fma_f32`, `v_pk_mul_f32`,
  `v_pk_add_f32`): the build disables it, and the kernels' FP32 arithmetic
  is written as scalar operations.
* Kernels whose grid assumes a number of resident waves fit the registers
  of that occupancy, and no kernel spills to scratch.
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


def _kernels(src):
    """name -> (VGPRs, private segment bytes) of every kernel in src."""
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", _asm(src), re.S):
        body = m.group(2)
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr\s+(\d+)", body).group(1))
        priv = int(re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", body).group(1))
        out[m.group(1)] = (vgpr, priv)
    return out


# (source, kernel-name fragment, waves per SIMD its launch assumes)
OCCUPANCY = [
    ("requant.hip", "requant_kernel", 4),       # four 256-thread workgroups per compute unit
    ("requant.hip", "transpose_w_kernel", 4),
    ("quant.hip", "quant_act_kernel", 8),       # 32 waves per compute unit walk the items
    ("gemm.hip", "gemm_kernel", 2),             # one 512-thread workgroup per compute unit
    ("gemm_bf16a.hip", "gemm_bf16a_kernel", 2),
]


@pytest.mark.parametrize("src,frag,waves", OCCUPANCY)
def test_register_budget_of_the_launch(src, frag, waves):
    """A kernel whose grid assumes a number of resident waves must fit their
    registers (512 per SIMD lane, allocated in granules of 8): one VGPR too
    many silently drops a workgroup per compute unit."""
    ks = {n: v for n, v in _kernels(src).items() if frag in n}
    assert ks, f"{src}: no kernel {frag}"
    for name, (vgpr, _) in ks.items():
        alloc = -(-vgpr // 8) * 8
        assert 512 // alloc >= waves, f"{name}: {vgpr} VGPRs allow {512 // alloc} waves per SIMD, launch assumes {waves}"


@pytest.mark.parametrize("src", [s for s in build.SOURCES if s != "api.hip"])
def test_no_register_spills(src):
    """No kernel spills to scratch.  In the persistent GEMM a reload from
    scratch waits for every copy and store in flight (a scratch load counts
    in the same vector-memory counter), so a spilled address costs a full
    memory round trip wherever it is reloaded."""
    for name, (_, priv) in _kernels(src).items():
        assert priv == 0, f"{name}: {priv} bytes of scratch"
