"""GPU parity of the block-scaled FP8 GEMM and the grouped (MoE) GEMM
against the binary64 CPU oracle on the same quantized operands."""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import (announce, check_bf16_is_rounded_f32, check_gemm_outputs,
                              dev, f32_dev, gemm_mag, host, native_loaded, sampled_check,
                              u8_dev)

pytestmark = pytest.mark.gpu


def _gemm_dev(qa, sa, qb, sb, bmode, out_f32, pads=(0, 0, 0, 0, 0)):
    """Run fp8bs_gemm on host arrays (optionally with padded row strides)."""
    M, K = qa.shape
    N = qb.shape[0]
    pa, psa, pb, psb, pd = pads
    a = torch.zeros((M, K + pa), dtype=torch.uint8, device=dev()); a[:, :K] = u8_dev(qa)
    b = torch.zeros((N, K + pb), dtype=torch.uint8, device=dev()); b[:, :K] = u8_dev(qb)
    sa_d = torch.zeros((M, sa.shape[1] + psa), dtype=torch.float32, device=dev()); sa_d[:, :sa.shape[1]] = f32_dev(sa)
    sb_d = torch.zeros((sb.shape[0], sb.shape[1] + psb), dtype=torch.float32, device=dev()); sb_d[:, :sb.shape[1]] = f32_dev(sb)
    dt = torch.float32 if out_f32 else torch.bfloat16
    d = torch.full((M, N + pd), 7.0, dtype=dt, device=dev())
    fp8bs.fp8bs_gemm(a[:, :K], sa_d[:, :sa.shape[1]], b[:, :K], sb_d[:, :sb.shape[1]], bmode,
                     d[:, :N], fp8bs.OUT_F32 if out_f32 else fp8bs.OUT_BF16)
    dh = host(d)
    if pd:
        tail = dh[:, N:]
        assert (tail == (7.0 if out_f32 else 0x40E0)).all(), "wrote past the output row"
    return dh[:, :N]


def _full_check(name, qa, sa, qb, sb, bmode=oracle.BSCALE_BLOCK, pads=(0, 0, 0, 0, 0), **kw):
    ref = oracle.gemm(qa, sa, qb, sb, bmode)
    mag = gemm_mag(qa, sa, qb, sb, bmode)
    d32 = _gemm_dev(qa, sa, qb, sb, bmode, True, pads)
    d16 = _gemm_dev(qa, sa, qb, sb, bmode, False, pads)
    check_gemm_outputs(name, d32, d16, ref, mag, **kw)


def test_gemm_tiny_full():
    native_loaded()
    q = synth.tiny()
    qa, sa = oracle.quant_act_1x128(q["A"])
    qb, sb = oracle.quant_w_128x128(q["W"])
    announce("gemm tiny 128x256x512")
    _full_check("tiny", qa, sa, qb, sb, max_flip_share=0.04)   # measured 2.1 % (1 % of entries x50)


def test_gemm_probe_full():
    native_loaded()
    q = synth.probe()
    qa, sa = oracle.quant_act_1x128(q["A"])
    qb, sb = oracle.quant_w_128x128(q["W"])
    announce("gemm probe 1024x1024x4096")
    _full_check("probe", qa, sa, qb, sb, max_flip_share=0.015)   # measured 0.56 %


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (200, 136, 384), (129, 264, 256), (77, 1000, 640)])
def test_gemm_ragged_strided(M, N, K):
    native_loaded()
    rng = np.random.default_rng(M * 7 + N)
    q = synth.tiny(M=M, N=N, K=K, seed=M + N)
    qa, sa = oracle.quant_act_1x128(q["A"])
    qb, sb = oracle.quant_w_128x128(q["W"])
    announce(f"gemm ragged {M}x{N}x{K}")
    _full_check(f"ragged {M}x{N}x{K}", qa, sa, qb, sb, pads=(16, 3, 32, 1, 8))
    # row mode with per-row scales of B
    qbr, sbr = oracle.quant_act_1x128(q["W"])
    _full_check(f"ragged-row {M}x{N}x{K}", qa, sa, qbr, sbr, oracle.BSCALE_ROW, pads=(0, 0, 0, 2, 0))


def test_gemm_many_ragged_tiles():
    """More tiles than workgroups (each workgroup walks several tiles, the
    next tile's first copies overlapping the previous tile's output), with
    ragged M and N in both B-scale modes."""
    native_loaded()
    M, N, K = 1000, 9000, 384
    q = synth.tiny(M=M, N=N, K=K, seed=5)
    qa, sa = oracle.quant_act_1x128(q["A"])
    qb, sb = oracle.quant_w_128x128(q["W"])
    announce(f"gemm many tiles {M}x{N}x{K}")
    _full_check(f"many-tiles {M}x{N}x{K}", qa, sa, qb, sb)
    qbr, sbr = oracle.quant_act_1x128(q["W"])
    _full_check(f"many-tiles-row {M}x{N}x{K}", qa, sa, qbr, sbr, oracle.BSCALE_ROW)


def test_gemm_edge_scales_and_codes():
    """Zero, subnormal and huge scales; saturated codes; negative zeros."""
    native_loaded()
    rng = np.random.default_rng(12)
    M, N, K = 256, 256, 512
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E
    qb[(qb & 0x7F) == 0x7F] = 0xFE
    qa[:8] = 0x7E
    qb[:4] = 0x80
    sa = (rng.uniform(0.5, 2, (M, 4)) * 2.0 ** rng.integers(-20, 20, (M, 4))).astype(np.float32)
    sb = (rng.uniform(0.5, 2, (2, 4)) * 2.0 ** rng.integers(-20, 20, (2, 4))).astype(np.float32)
    sa[10:20, 1] = 0.0
    sa[20:30, 2] = np.float32(2.0 ** -140)
    sb[1, 3] = 0.0
    announce("gemm edge scales")
    _full_check("edge", qa, sa, qb, sb)


def test_gemm_mlp_up_full_size_sampled():
    """4096 x 18432 x 7168 (the K = 7168 dense up-projection), the launch
    configuration the benchmark times; sampled entries vs the oracle."""
    native_loaded()
    announce("gemm mlp_up 4096x18432x7168: inputs")
    d = synth.mlp_up()
    qa, sa = oracle.quant_act_1x128(d["X"])
    qb, sb = oracle.quant_w_128x128(d["W"])
    a, b = u8_dev(qa), u8_dev(qb)
    sad, sbd = f32_dev(sa), f32_dev(sb)
    out = fp8bs.gemm(a, sad, b, sbd)
    out32 = fp8bs.gemm(a, sad, b, sbd, out_f32=True)
    sampled_check("mlp_up", qa, sa, qb, sb, out32, out, max_flip_share=0.03)   # measured 0.9 %
    assert torch.isfinite(out32).all()


def test_gemm_wgrad_row_mode_full_size_sampled():
    """dW [7168][2048] = X^T dY over K = 8192 tokens, operands re-quantized
    to 128x1 tiles along tokens, FP32 output (row-mode B scales)."""
    native_loaded()
    announce("gemm wgrad 7168x2048x8192 row mode")
    d = synth.wgrad()
    q1, s1 = oracle.quant_act_1x128(d["X"])
    qa, sa = oracle.requant_T_128x1_fp8(q1, s1)          # [7168][8192]
    qb, sb = oracle.requant_T_128x1_bf16(d["dY"])        # [2048][8192]
    out = fp8bs.gemm(u8_dev(qa), f32_dev(sa), u8_dev(qb), f32_dev(sb), fp8bs.BSCALE_ROW_1x128, out_f32=True)
    sampled_check("wgrad", qa, sa, qb, sb, out, None, bmode=oracle.BSCALE_ROW)


def _grouped_dev(qa, sa, qb, sb, off, out_f32):
    d = fp8bs.grouped_gemm(u8_dev(qa), f32_dev(sa), u8_dev(qb), f32_dev(sb),
                           torch.from_numpy(off.astype(np.int32)).to(dev()), out_f32=out_f32)
    return d


def test_grouped_small_full_with_empty_and_tiny_experts():
    native_loaded()
    rng = np.random.default_rng(4)
    counts = np.array([130, 0, 1, 127, 128, 0, 300])
    off = synth.offsets_from_counts(counts)
    T, E, N, K = int(off[-1]), len(counts), 256, 384
    x = synth.tiny(M=T, N=1, K=K, seed=1)["A"]
    w = synth.tiny(M=1, N=E * N, K=K, seed=2)["W"]
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_w_128x128(w)
    qb = qb.reshape(E, N, K); sb = sb.reshape(E, N // 128, K // 128)
    ref = oracle.grouped_gemm(qa, sa, qb, sb, off)
    mag = oracle.grouped_gemm(qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), off)
    announce(f"grouped small E={E} T={T}")
    d32 = host(_grouped_dev(qa, sa, qb, sb, off, True))
    d16 = host(_grouped_dev(qa, sa, qb, sb, off, False))
    check_gemm_outputs("grouped small", d32, d16, ref, mag)


@pytest.mark.parametrize("which", ["up", "down"])
def test_grouped_moe_full_size_sampled(which):
    """One GPU's 8 experts, 16384 tokens with Zipf(1.1) counts; gate+up
    K=7168 -> N=4096 or down K=2048 -> N=7168; sampled entries in every
    expert, including each expert's first and last row."""
    native_loaded()
    announce(f"grouped moe {which}: inputs")
    parts = ("A_up", "W_up") if which == "up" else ("A_down", "W_down")
    m = synth.moe(parts=parts)
    x, w = m[parts[0]], m[parts[1]]
    E, N, K = w.shape
    off = m["offsets"]
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_w_128x128(w.reshape(E * N, K))
    qb = qb.reshape(E, N, K); sb = sb.reshape(E, N // 128, K // 128)
    out16 = _grouped_dev(qa, sa, qb, sb, off, False)
    out32 = _grouped_dev(qa, sa, qb, sb, off, True)
    rng = np.random.default_rng(1)
    nz = np.flatnonzero(np.diff(off) > 0)
    mi = np.concatenate([rng.integers(0, off[-1], 2000), off[nz], off[nz + 1] - 1])
    ni = np.concatenate([rng.integers(0, N, 2000), rng.integers(0, N, 2 * nz.size)])
    ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mi, ni)
    mag = oracle.grouped_gemm_entries(qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), off, mi, ni)
    check_gemm_outputs(f"grouped moe {which}", host(out32), host(out16), ref, mag, mi, ni,
                       max_flip_share=0.03)   # measured 1.1 % (up), 0.7 % (down)


def test_gemm_bf16_output_rounding_crafted_values():
    """The BF16 epilogue rounds every FP32 result once to nearest-even.  With
    a[m] = 1.0 at k = 0 (zero elsewhere), b[n] = 1.0 at k = 0 and sb = 1, the
    FP32 result of row m is exactly sa[m], so chosen scales put chosen FP32
    values through the epilogue: random bit patterns, bf16 ties with even
    and odd last bits, values next to ties, FP32 subnormals, and the top of
    the range (rounding up to infinity)."""
    native_loaded()
    rng = np.random.default_rng(21)
    rand = rng.integers(0, 0x7F800000, 40000, dtype=np.uint32) | (rng.integers(0, 2, 40000, dtype=np.uint32) << 31)
    hi = rng.integers(0x0001, 0x7F7F, 6000, dtype=np.uint32) << 16
    crafted = np.concatenate([
        hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi | 0x0001, hi | 0xFFFF,         # ties and neighbours
        rng.integers(1, 0x00800000, 4000, dtype=np.uint32),                      # FP32 subnormals
        np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F7EFFFF, 0x00000001, 0x00008000,
                  0x00018000, 0x007FFFFF, 0x00800000, 0x3F808000, 0x3F818000], np.uint32)])
    crafted = crafted | (rng.integers(0, 2, crafted.size, dtype=np.uint32) << 31)
    pats = np.concatenate([rand, crafted])
    pats = pats[pats != 0x80000000]           # -0 becomes +0 when added to the zero accumulator
    sa_vals = pats.view(np.float32)
    M, N, K = sa_vals.size, 48, 128
    qa = np.zeros((M, K), np.uint8); qa[:, 0] = 0x38
    qb = np.zeros((N, K), np.uint8); qb[:, 0] = 0x38
    sa = sa_vals.reshape(M, 1).copy()
    sb = np.ones((1, 1), np.float32)
    announce(f"bf16 epilogue rounding on {M} crafted FP32 values")
    d32 = _gemm_dev(qa, sa, qb, sb, oracle.BSCALE_BLOCK, True)
    assert np.array_equal(d32.view(np.uint32), np.repeat(pats.reshape(M, 1), N, 1)), "FP32 path is not exact"
    d16 = _gemm_dev(qa, sa, qb, sb, oracle.BSCALE_BLOCK, False)
    ref = oracle.round_to_bf16(sa_vals.astype(np.float64))
    bad = np.flatnonzero(d16[:, 0] != ref)
    assert bad.size == 0, f"{bad.size} wrong roundings, first {pats[bad[0]]:#010x} -> {d16[bad[0], 0]:#06x}, want {ref[bad[0]]:#06x}"
    assert (d16 == d16[:, :1]).all()


def test_gemm_deterministic():
    native_loaded()
    d = synth.mlp_up(T=512, K=1024, N=1024)
    qa, sa = oracle.quant_act_1x128(d["X"])
    qb, sb = oracle.quant_w_128x128(d["W"])
    a = _gemm_dev(qa, sa, qb, sb, oracle.BSCALE_BLOCK, True)
    b = _gemm_dev(qa, sa, qb, sb, oracle.BSCALE_BLOCK, True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
