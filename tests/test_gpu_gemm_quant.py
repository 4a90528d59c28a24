"""GPU parity of the GEMM with the next layer's 1x128 quantization fused into
its epilogue (fp8bs_gemm_quant_1x128).

* Operands whose FP32 result is exact (closed form): codes and scales
  bit-exact against the oracle.
* General data: the GPU's FP32 result may differ from the binary64 oracle
  within the GEMM tolerance, so a code may sit on the other side of an E4M3
  rounding midpoint.  Each tile's scale must match the oracle's tile max-abs
  within the GEMM allowance, each dequantized code must lie within half an
  E4M3 step of the oracle value plus that allowance, and the share of codes
  equal to the oracle's fused result is reported and bounded below.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.exact_ref import torch_e4m3_table
from tests.gpu_common import (announce, check_quant_equal, dev, f32_dev, gemm_mag, host,
                              native_loaded, u8_dev)
from tests.test_oracle_gemm import quant_output_closed_form_case

pytestmark = pytest.mark.gpu
TAB = torch_e4m3_table().astype(np.float64)


def _gemm_quant_dev(qa, sa, qb, sb, bmode, pad_q=0, pad_s=0):
    M, K = qa.shape
    N = qb.shape[0]
    q = torch.full((M, N + pad_q), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((M, N // 128 + pad_s), -5.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_gemm_quant_1x128(u8_dev(qa), f32_dev(sa), u8_dev(qb), f32_dev(sb), bmode,
                                 q[:, :N], s[:, :N // 128])
    qh, sh = host(q), host(s)
    assert (qh[:, N:] == 0x55).all(), "wrote past a code row"
    assert (sh[:, N // 128:] == -5.0).all(), "wrote past a scale row"
    return qh[:, :N], sh[:, :N // 128]


@pytest.mark.parametrize("M,N", [(1, 128), (300, 384), (129, 1024)])
def test_gemm_quant_closed_form_bit_exact(M, N):
    native_loaded()
    rng = np.random.default_rng(M + N)
    a, sa, b, sbb, sbr, q_exp, s_exp = quant_output_closed_form_case(rng, M, N)
    for sb, mode in ((sbb, fp8bs.BSCALE_BLOCK_128x128), (sbr, fp8bs.BSCALE_ROW_1x128)):
        announce(f"gemm_quant closed form {M}x{N} bmode {mode}")
        q_ref, s_ref = oracle.gemm_quant_1x128(a, sa, b, sb, mode)
        assert np.array_equal(q_ref, q_exp) and np.array_equal(s_ref, s_exp)
        q, s = _gemm_quant_dev(a, sa, b, sb, mode, pad_q=16, pad_s=3)
        check_quant_equal(f"gemm_quant closed form {M}x{N}", q, s, q_ref, s_ref)


def _check_against_f64(name, q, s, d_ref, mag):
    """q, s from the GPU; d_ref the binary64 oracle GEMM; mag = sum|a||b|."""
    R, N = d_ref.shape
    G = N // 128
    tol = 1e-3 * mag                                   # the GEMM acceptance allowance per entry
    amax_ref = np.abs(d_ref).reshape(R, G, 128).max(2)
    tol_t = tol.reshape(R, G, 128).max(2)
    s64 = s.astype(np.float64)
    bad = np.abs(s64 * 448.0 - amax_ref) > tol_t + amax_ref * 2.0 ** -21
    assert not bad.any(), f"{name}: {bad.sum()} tile scales off the oracle's max-abs"
    sr = np.repeat(s64, 128, 1)
    y = (np.abs(d_ref) + tol) / np.where(sr > 0, sr, 1.0)
    step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3), 2.0 ** -9) * sr
    err = np.abs(TAB[q] * sr - d_ref)
    over = err > 0.5 * step * (1 + 2.0 ** -10) + tol
    assert not over.any(), f"{name}: {over.sum()} codes farther than half a step (+ allowance)"


def test_gemm_quant_tiny_config_both_modes():
    """The small configuration (A 128x512 with outliers, W 256x512)."""
    native_loaded()
    d = synth.tiny()
    qa, sa = oracle.quant_act_1x128(d["A"])
    for mode in (fp8bs.BSCALE_BLOCK_128x128, fp8bs.BSCALE_ROW_1x128):
        if mode == fp8bs.BSCALE_BLOCK_128x128:
            qb, sb = oracle.quant_w_128x128(d["W"])
        else:
            qb, sb = oracle.quant_act_1x128(d["W"])
        announce(f"gemm_quant tiny bmode {mode}")
        q, s = _gemm_quant_dev(qa, sa, qb, sb, mode)
        d_ref = oracle.gemm(qa, sa, qb, sb, mode)
        _check_against_f64("tiny", q, s, d_ref, gemm_mag(qa, sa, qb, sb, mode))
        q_ref, s_ref = oracle.gemm_quant_1x128(qa, sa, qb, sb, mode)
        same = float((q == q_ref).mean())
        announce(f"tiny bmode {mode}: codes equal to the oracle's fused result {same:.5f}, "
                 f"scales equal {float((s == s_ref).mean()):.4f}")
        assert same >= 0.98


def test_gemm_quant_mlp_up_full_size_sampled_rows():
    """4096 x 18432 x 7168 with the fused output: 24 rows (every column)
    against the oracle."""
    native_loaded()
    announce("gemm_quant mlp_up 4096x18432x7168: inputs")
    d = synth.mlp_up()
    qa, sa = oracle.quant_act_1x128(d["X"])
    qb, sb = oracle.quant_w_128x128(d["W"])
    del d
    announce("gemm_quant mlp_up: gpu")
    q, s = fp8bs.gemm_quant_1x128(u8_dev(qa), f32_dev(sa), u8_dev(qb), f32_dev(sb))
    qh, sh = host(q), host(s)
    rows = np.unique(np.concatenate([[0, 4095, 2048], np.random.default_rng(3).integers(0, 4096, 21)]))
    N = qb.shape[0]
    mi = np.repeat(rows, N)
    ni = np.tile(np.arange(N), rows.size)
    announce(f"gemm_quant mlp_up: oracle on {rows.size} rows")
    d_ref = oracle.gemm_entries(qa, sa, qb, sb, mi, ni).reshape(rows.size, N)
    mag = gemm_mag(qa, sa, qb, sb, oracle.BSCALE_BLOCK, mi, ni).reshape(rows.size, N)
    _check_against_f64("mlp_up", qh[rows], sh[rows], d_ref, mag)
    q_ref, _ = oracle.quant_act_1x128_f32(d_ref.astype(np.float32))
    same = float((qh[rows] == q_ref).mean())
    announce(f"mlp_up: codes equal to the oracle's fused result on the sampled rows {same:.5f}")
    assert same >= 0.98
