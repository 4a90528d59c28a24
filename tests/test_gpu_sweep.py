"""Sweeps over the number of 128-wide K groups, G = K / 128, on the GPU
against the CPU oracle.

The GEMM's main loop is unrolled by 12 groups (stages repeat every 3,
scale-block quarters every 4) and guards each iteration with g + i < G; its
scales travel in blocks of 4 groups.  The 1x128 activation quantizer picks
one of seven kernel shapes from ceil(G / 4) and the row count.  So every
G from 1 to 26 is run here: all residues of G modulo 12 and 4, with ragged
M and N, both B-scale modes, FP32 and BF16 outputs; and every G from 1 to
40 for the activation quantizer, at a row count that takes the persistent
kernel where it applies.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import announce, bf16_dev, check_quant_equal, host, native_loaded
from tests.test_gpu_gemm import _full_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G", list(range(1, 27)))
def test_gemm_every_group_count(G):
    native_loaded()
    M, N, K = 130, 264, 128 * G
    q = synth.tiny(M=M, N=N, K=K, seed=100 + G)
    qa, sa = oracle.quant_act_1x128(q["A"])
    announce(f"gemm sweep G={G}: {M}x{N}x{K}")
    if G % 2:
        qb, sb = oracle.quant_w_128x128(q["W"])
        _full_check(f"sweep G={G} block", qa, sa, qb, sb, pads=(16, 1, 0, 2, 8))
    else:
        qb, sb = oracle.quant_act_1x128(q["W"])
        _full_check(f"sweep G={G} row", qa, sa, qb, sb, oracle.BSCALE_ROW, pads=(0, 2, 16, 1, 0))


@pytest.mark.parametrize("G", list(range(1, 41)))
def test_quant_act_every_group_count(G):
    native_loaded()
    K = 128 * G
    for M in (33, 1000):
        x = synth.tiny(M=M, N=1, K=K, seed=200 + G)["A"]
        announce(f"quant_act sweep G={G}: {M}x{K}")
        q, s = fp8bs.quant_act_1x128(bf16_dev(x))
        qr, sr = oracle.quant_act_1x128(x)
        check_quant_equal(f"quant_act sweep {M}x{K}", host(q), host(s), qr, sr)


@pytest.mark.parametrize("M,G", [(11000, 41), (8300, 60)])
def test_quant_act_row_kernels_on_long_rows(M, G):
    """Many long rows: the one-wave-per-row kernels with 14 and 16 tile-quads
    in flight per wave (G = 41: 11 quads; G = 60: 15 quads)."""
    native_loaded()
    K = 128 * G
    x = synth.tiny(M=M, N=1, K=K, seed=300 + G)["A"]
    announce(f"quant_act long rows: {M}x{K}")
    q, s = fp8bs.quant_act_1x128(bf16_dev(x))
    qr, sr = oracle.quant_act_1x128(x)
    check_quant_equal(f"quant_act long rows {M}x{K}", host(q), host(s), qr, sr)


@pytest.mark.parametrize("case", range(8))
def test_grouped_random_expert_counts(case):
    """Seeded random expert counts (empty experts, counts below, at and just
    past a 128-row tile), expert counts 1 .. 16, several K and N: every
    output entry against the oracle."""
    from tests.gpu_common import check_gemm_outputs
    from tests.test_gpu_gemm import _grouped_dev
    native_loaded()
    rng = np.random.default_rng(400 + case)
    E = int(rng.choice([1, 2, 3, 5, 8, 16]))
    counts = rng.choice([0, 1, 5, 127, 128, 129, 200, 256, 300], size=E)
    if counts.sum() == 0:
        counts[0] = 129
    N = int(rng.choice([128, 256, 384]))
    K = 128 * int(rng.integers(1, 15))
    off = synth.offsets_from_counts(counts)
    T = int(off[-1])
    x = synth.tiny(M=T, N=1, K=K, seed=500 + case)["A"]
    w = synth.tiny(M=1, N=E * N, K=K, seed=600 + case)["W"]
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_w_128x128(w)
    qb = qb.reshape(E, N, K); sb = sb.reshape(E, N // 128, K // 128)
    announce(f"grouped sweep {case}: E={E} counts={counts.tolist()} N={N} K={K}")
    ref = oracle.grouped_gemm(qa, sa, qb, sb, off)
    mag = oracle.grouped_gemm(qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), off)
    d32 = host(_grouped_dev(qa, sa, qb, sb, off, True))
    d16 = host(_grouped_dev(qa, sa, qb, sb, off, False))
    check_gemm_outputs(f"grouped sweep {case}", d32, d16, ref, mag)


@pytest.mark.parametrize("G", [1, 2, 3, 5, 11, 12, 13, 25])
def test_gemm_quant_closed_form_group_counts(G):
    """The fused output quantization over several K-group counts, on
    operands whose FP32 result is exact: codes and scales bit-exact."""
    from tests.test_gpu_gemm_quant import _gemm_quant_dev
    from tests.test_oracle_gemm import quant_output_closed_form_case
    native_loaded()
    rng = np.random.default_rng(700 + G)
    a, sa, b, sbb, sbr, q_exp, s_exp = quant_output_closed_form_case(rng, 70, 384, G=G)
    for sb, mode in ((sbb, fp8bs.BSCALE_BLOCK_128x128), (sbr, fp8bs.BSCALE_ROW_1x128)):
        announce(f"gemm_quant closed form G={G} bmode {mode}")
        q_ref, s_ref = oracle.gemm_quant_1x128(a, sa, b, sb, mode)
        assert np.array_equal(q_ref, q_exp) and np.array_equal(s_ref, s_exp)
        q, s = _gemm_quant_dev(a, sa, b, sb, mode, pad_q=16, pad_s=1)
        check_quant_equal(f"gemm_quant closed form G={G}", q, s, q_ref, s_ref)
