"""Race check: the LDS-poisoning debug build (`libfp8bs_poison.so`, built
with FP8BS_POISON_LDS) fills every kernel's LDS with 0xFF bytes -- NaN as
FP32, the NaN code as E4M3 -- before the kernel's first use of it.  A
kernel that reads LDS it has not written (a missing wait or barrier, a
stage read before its copy, an unwritten tail) would then produce NaNs or
wrong codes.  These parity cases run through that build and must still
match the oracle exactly as the library build does: ragged and strided
shapes, both B-scale modes, every output form, requant from every source,
the weight transpose, the grouped GEMM with empty experts, the BF16-A GEMM
(A quantized in place in LDS) and the one-launch activation and weight
quantizer.
"""
import os

import numpy as np
import pytest

import oracle
from fp8_fine_grained_fp8bs_amd import build, fp8bs, synth
from tests.gpu_common import announce, bf16_dev, check_quant_equal, host, native_loaded

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def poisoned_library():
    assert os.path.exists(build.POISON_LIB), "libfp8bs_poison.so is built with the library"
    prev = fp8bs.use_library(build.POISON_LIB)
    try:
        yield
    finally:
        fp8bs.use_library(prev)


def test_poisoned_build_is_loaded():
    lib = native_loaded()
    assert lib._name == build.POISON_LIB


@pytest.mark.parametrize("M,N,K", [(130, 264, 640), (1000, 9000, 384), (77, 1000, 1664)])
def test_gemm_poisoned(M, N, K):
    from tests.test_gpu_gemm import _full_check
    native_loaded()
    q = synth.tiny(M=M, N=N, K=K, seed=M + K)
    qa, sa = oracle.quant_act_1x128(q["A"])
    qb, sb = oracle.quant_w_128x128(q["W"])
    announce(f"poisoned gemm {M}x{N}x{K}")
    _full_check(f"poisoned {M}x{N}x{K}", qa, sa, qb, sb, pads=(16, 1, 0, 2, 8))
    qbr, sbr = oracle.quant_act_1x128(q["W"])
    _full_check(f"poisoned row {M}x{N}x{K}", qa, sa, qbr, sbr, oracle.BSCALE_ROW)


def test_gemm_quant_poisoned():
    from tests.test_gpu_gemm_quant import _gemm_quant_dev
    from tests.test_oracle_gemm import quant_output_closed_form_case
    native_loaded()
    rng = np.random.default_rng(31)
    a, sa, b, sbb, sbr, q_exp, s_exp = quant_output_closed_form_case(rng, 200, 640, G=7)
    for sb, mode in ((sbb, fp8bs.BSCALE_BLOCK_128x128), (sbr, fp8bs.BSCALE_ROW_1x128)):
        announce(f"poisoned gemm_quant bmode {mode}")
        q, s = _gemm_quant_dev(a, sa, b, sb, mode, pad_q=16, pad_s=1)
        check_quant_equal("poisoned gemm_quant", q, s, q_exp, s_exp)


def test_grouped_poisoned():
    from tests.gpu_common import check_gemm_outputs
    from tests.test_gpu_gemm import _grouped_dev
    native_loaded()
    counts = np.array([130, 0, 1, 127, 128, 0, 300])
    off = synth.offsets_from_counts(counts)
    T, E, N, K = int(off[-1]), len(counts), 256, 640
    x = synth.tiny(M=T, N=1, K=K, seed=7)["A"]
    w = synth.tiny(M=1, N=E * N, K=K, seed=8)["W"]
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_w_128x128(w)
    qb = qb.reshape(E, N, K); sb = sb.reshape(E, N // 128, K // 128)
    announce("poisoned grouped")
    ref = oracle.grouped_gemm(qa, sa, qb, sb, off)
    mag = oracle.grouped_gemm(qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), off)
    d32 = host(_grouped_dev(qa, sa, qb, sb, off, True))
    check_gemm_outputs("poisoned grouped", d32, host(_grouped_dev(qa, sa, qb, sb, off, False)), ref, mag)


@pytest.mark.parametrize("T", [1, 1000, 8200])
def test_requant_poisoned(T):
    from tests.test_gpu_requant import _run_requant
    native_loaded()
    d = synth.wgrad(T=T, C_in=384, C_out=256, seed=T + 1)
    q1, s1 = oracle.quant_act_1x128(d["X"])
    announce(f"poisoned requant T={T}")
    q, s = _run_requant(q1, s1, ld_in_pad=16, ld_out_pad=16, lds_out_pad=2)
    check_quant_equal(f"poisoned requant fp8 T={T}", q, s, *oracle.requant_T_128x1_fp8(q1, s1))
    q, s = _run_requant(d["dY"], ld_in_pad=8, ld_out_pad=32, lds_out_pad=1)
    check_quant_equal(f"poisoned requant bf16 T={T}", q, s, *oracle.requant_T_128x1_bf16(d["dY"]))


@pytest.mark.parametrize("T", [256, 300])
def test_requant_e5m6_poisoned(T):
    """The E5M6 source writes its decoded rows into LDS itself (no copies):
    every read of the tile must follow those writes and the barrier."""
    from tests.test_gpu_requant_e5m6 import run_requant_e5m6
    native_loaded()
    x = synth.wgrad(T=T, C_in=384, C_out=128, seed=T + 3)["X"]
    y = oracle.encode_e5m6(x)
    announce(f"poisoned requant e5m6 T={T}")
    q, s = run_requant_e5m6(y, 384, ld_in_pad=16, ld_out_pad=16, lds_out_pad=2)
    check_quant_equal(f"poisoned requant e5m6 T={T}", q, s, *oracle.requant_T_128x1_e5m6(y, 384))


def test_transpose_and_quant_w_poisoned():
    from tests.test_gpu_dgrad import _transpose_dev
    native_loaded()
    w = synth.wgrad(T=128, C_in=1152, C_out=640, seed=5, with_w=True)["W"]
    announce("poisoned quant_w and transpose_w")
    qg, sg = fp8bs.quant_w_128x128(bf16_dev(w))
    q, s = oracle.quant_w_128x128(w)
    check_quant_equal("poisoned quant_w", host(qg), host(sg), q, s)
    qt, st = _transpose_dev(q, s, pad_q=16, pad_s=3, pad_qt=32, pad_st=2)
    check_quant_equal("poisoned transpose_w", qt, st, *oracle.transpose_w_128x128(q, s))


@pytest.mark.parametrize("M,N,K", [(129, 264, 640), (300, 576, 128)])
def test_gemm_bf16a_poisoned(M, N, K):
    """The BF16-A GEMM quantizes A in place in its raw LDS stages and keeps
    the scales in the rows' free chunks: every code, scale and B stage it
    reads must have been written first."""
    from tests.test_gpu_gemm_bf16a import _full
    native_loaded()
    q = synth.tiny(M=M, N=N, K=K, seed=M + 5 * N)
    announce(f"poisoned gemm_bf16a {M}x{N}x{K}")
    _full(f"poisoned bf16a {M}x{N}x{K}", q["A"], q["W"], pads=(8, 16, 3, 8))


def test_quant_act_w_poisoned():
    from tests.test_gpu_quant import _run_act_w
    native_loaded()
    rng = np.random.default_rng(5)
    x = synth.bf16_bits(rng.standard_normal((70, 384)).astype(np.float32))
    w = synth.bf16_bits(rng.standard_normal((300, 384)).astype(np.float32))
    announce("poisoned quant_act_w 70x384 + 300x384")
    qx, sx, qw, sw = _run_act_w(x, w, pad=16)
    check_quant_equal("poisoned quant_act_w activation", qx, sx, *oracle.quant_act_1x128(x))
    check_quant_equal("poisoned quant_act_w weight", qw, sw, *oracle.quant_w_128x128(w))
