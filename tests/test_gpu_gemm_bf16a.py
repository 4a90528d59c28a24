"""GPU parity of fp8bs_gemm_bf16a, the block-scaled GEMM that quantizes its
BF16 A operand in 1x128 tiles inside the GEMM ([p2] para 1: the FP8
activation then never crosses HBM; [p1] para 3: the 1x128 tile quantizer).

Three facts are checked for every case:
* the codes and scales it stores (the FP8 activation cache) are bit-exact
  with the oracle's 1x128 quantizer of the same BF16 rows;
* its D is bitwise the D of fp8bs_gemm on those codes (same arithmetic),
  in FP32 and BF16, with and without the code output;
* D is within the GEMM tolerance of the binary64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import (announce, bf16_dev, check_gemm_outputs, check_quant_equal, dev,
                              f32_dev, gemm_mag, host, native_loaded, sampled_check, u8_dev)
from tests.test_gpu_quant import _edge_rows

pytestmark = pytest.mark.gpu


def _run(x_u16, qb, sb, out_f32, codes, pads=(0, 0, 0, 0)):
    """fp8bs_gemm_bf16a on host arrays; pads = extra row elements of x, qx,
    sx and d (a sentinel past each row of d must survive)."""
    M, K = x_u16.shape
    N, G = qb.shape[0], K // 128
    px, pq, ps, pd = pads
    xd = torch.zeros((M, K + px), dtype=torch.bfloat16, device=dev()); xd[:, :K] = bf16_dev(x_u16)
    b = u8_dev(qb)
    sbd = f32_dev(sb)
    qx = sx = None
    if codes:
        qx = torch.full((M, K + pq), 0x5A, dtype=torch.uint8, device=dev())
        sx = torch.full((M, G + ps), -1.0, dtype=torch.float32, device=dev())
    dt = torch.float32 if out_f32 else torch.bfloat16
    d = torch.full((M, N + pd), 7.0, dtype=dt, device=dev())
    fp8bs.fp8bs_gemm_bf16a(xd[:, :K], qx[:, :K] if codes else None, sx[:, :G] if codes else None,
                           b, sbd, d[:, :N], fp8bs.OUT_F32 if out_f32 else fp8bs.OUT_BF16)
    dh = host(d)
    if pd:
        assert (dh[:, N:] == (7.0 if out_f32 else 0x40E0)).all(), "wrote past the output row"
    if not codes:
        return dh[:, :N], None, None
    qh, sh = host(qx), host(sx)
    if pq:
        assert (qh[:, K:] == 0x5A).all(), "wrote past the code row"
    if ps:
        assert (sh[:, G:] == -1.0).all(), "wrote past the scale row"
    return dh[:, :N], qh[:, :K], sh[:, :G]


def _gemm_on_codes(qa, sa, qb, sb, out_f32):
    M, N = qa.shape[0], qb.shape[0]
    dt = torch.float32 if out_f32 else torch.bfloat16
    d = torch.empty((M, N), dtype=dt, device=dev())
    fp8bs.fp8bs_gemm(u8_dev(qa), f32_dev(sa), u8_dev(qb), f32_dev(sb), fp8bs.BSCALE_BLOCK_128x128, d,
                     fp8bs.OUT_F32 if out_f32 else fp8bs.OUT_BF16)
    return host(d)


def _bitwise(name, got, want):
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.flatnonzero(g.ravel() != w.ravel())
    assert bad.size == 0, f"{name}: {bad.size} entries differ from fp8bs_gemm on the same codes, first {np.unravel_index(bad[0], got.shape)}"


def _full(name, x_u16, w_u16, pads=(0, 0, 0, 0), max_flip_share=0.03):
    qa, sa = oracle.quant_act_1x128(x_u16)
    qb, sb = oracle.quant_w_128x128(w_u16)
    d32, qx, sx = _run(x_u16, qb, sb, True, True, pads)
    check_quant_equal(f"{name} codes", qx, sx, qa, sa)
    d16, qx16, sx16 = _run(x_u16, qb, sb, False, True, pads)
    check_quant_equal(f"{name} codes (bf16 run)", qx16, sx16, qa, sa)
    d32n, _, _ = _run(x_u16, qb, sb, True, False)
    d16n, _, _ = _run(x_u16, qb, sb, False, False)
    g32, g16 = _gemm_on_codes(qa, sa, qb, sb, True), _gemm_on_codes(qa, sa, qb, sb, False)
    for tag, got, want in [("f32", d32, g32), ("bf16", d16, g16), ("f32 no codes", d32n, g32),
                           ("bf16 no codes", d16n, g16)]:
        _bitwise(f"{name} {tag}", got, want)
    ref = oracle.gemm(qa, sa, qb, sb, oracle.BSCALE_BLOCK)
    check_gemm_outputs(name, d32, d16, ref, gemm_mag(qa, sa, qb, sb), max_flip_share=max_flip_share)


def test_bf16a_tiny():
    native_loaded()
    q = synth.tiny()
    announce("gemm_bf16a tiny 128x256x512")
    _full("bf16a tiny", q["A"], q["W"], max_flip_share=0.04)


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (200, 136, 384), (129, 264, 256), (77, 1000, 640),
                                   (65, 576, 1024), (300, 256, 128)])
def test_bf16a_ragged_strided(M, N, K):
    """Ragged tiles in M (64-row tiles) and N (256-column tiles), K from
    one to ten groups (the copies run up to three groups ahead), padded
    rows of every operand."""
    native_loaded()
    q = synth.tiny(M=M, N=N, K=K, seed=M + 3 * N)
    announce(f"gemm_bf16a ragged {M}x{N}x{K}")
    _full(f"bf16a ragged {M}x{N}x{K}", q["A"], q["W"], pads=(8, 16, 3, 8))


def test_bf16a_edge_tiles():
    """The in-GEMM quantizer on the edge tiles of the standalone quantizer's
    tests (zeros, subnormals, tiny and huge scales, E4M3 midpoints)."""
    native_loaded()
    rng = np.random.default_rng(11)
    K = 768
    x = _edge_rows(K, rng)
    x = np.concatenate([x, x[::-1], x], axis=0)                  # more than one 64-row tile
    w = synth.bf16_bits(rng.standard_normal((320, K)).astype(np.float32))
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_w_128x128(w)
    announce(f"gemm_bf16a edge tiles M={x.shape[0]} K={K}")
    d32, qx, sx = _run(x, qb, sb, True, True)
    check_quant_equal("bf16a edge codes", qx, sx, qa, sa)
    _bitwise("bf16a edge f32", d32, _gemm_on_codes(qa, sa, qb, sb, True))
    d16, _, _ = _run(x, qb, sb, False, False)
    _bitwise("bf16a edge bf16", d16, _gemm_on_codes(qa, sa, qb, sb, False))


@pytest.mark.parametrize("N", [576, 1536])
def test_bf16a_projection_shapes(N):
    """The low-rank projections of the model family (7168 -> 576 and
    7168 -> 1536) on 4096 tokens: codes and scales bit-exact everywhere,
    D bitwise fp8bs_gemm on the same codes, and sampled entries within
    tolerance of the oracle."""
    native_loaded()
    M, K = 4096, 7168
    rng = np.random.default_rng(N)
    x = synth.mlp_up(T=M, K=K, N=N, seed=1, with_w=False)["X"]
    w = synth.bf16_bits((rng.standard_normal((N, K)) * 0.006).astype(np.float32))
    qa, sa = oracle.quant_act_1x128(x)
    qb, sb = oracle.quant_w_128x128(w)
    announce(f"gemm_bf16a projection {M}x{N}x{K}")
    xd = bf16_dev(x)
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev())
    sx = torch.empty((M, K // 128), dtype=torch.float32, device=dev())
    d32 = torch.empty((M, N), dtype=torch.float32, device=dev())
    d16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    b, sbd = u8_dev(qb), f32_dev(sb)
    fp8bs.fp8bs_gemm_bf16a(xd, qx, sx, b, sbd, d32, fp8bs.OUT_F32)
    fp8bs.fp8bs_gemm_bf16a(xd, None, None, b, sbd, d16, fp8bs.OUT_BF16)
    check_quant_equal(f"projection {N} codes", host(qx), host(sx), qa, sa)
    _bitwise(f"projection {N} f32", host(d32), _gemm_on_codes(qa, sa, qb, sb, True))
    _bitwise(f"projection {N} bf16", host(d16), _gemm_on_codes(qa, sa, qb, sb, False))
    sampled_check(f"bf16a projection {N}", qa, sa, qb, sb, d32, d16)
