"""Parity at the largest row strides the library accepts.

The GEMM addresses a tile's code and scale rows with 32-bit offsets from
the tile's first row (a 256-row tile of codes spans less than 4 GiB while
lda, ldb < 2^24 bytes; of scales while ldsa, ldsb < 2^22 floats), and the
re-quantization addresses a 128-token tile the same way (ld_in < 2^25
bytes).  These cases run at the largest strides below those limits, with
ragged row counts so that the descriptors' row bounds are exercised too,
and compare against the oracle.  The buffers are a few GiB of device
memory, most of it never touched.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import (announce, check_gemm_outputs,
                              check_quant_equal, dev, f32_dev, gemm_mag, host, native_loaded, u8_dev)

pytestmark = pytest.mark.gpu

MAX_CODE_LD = (1 << 24) - 16      # bytes per code row, 16-byte multiple
MAX_SCALE_LD = (1 << 22) - 1      # floats per scale row
MAX_REQUANT_LD = (1 << 25) - 16   # bytes per requant input row


def _strided(rows, cols, ld, dtype, host_data):
    buf = torch.empty((rows, ld), dtype=dtype, device=dev())
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(host_data)).to(dev())
    return buf[:, :cols]


@pytest.mark.parametrize("bmode", [oracle.BSCALE_BLOCK, oracle.BSCALE_ROW])
def test_gemm_at_the_largest_strides(bmode):
    native_loaded()
    M, N, K = 130, 264, 384
    q = synth.tiny(M=M, N=N, K=K, seed=77)
    qa, sa = oracle.quant_act_1x128(q["A"])
    if bmode == oracle.BSCALE_BLOCK:
        qb, sb = oracle.quant_w_128x128(q["W"])
    else:
        qb, sb = oracle.quant_act_1x128(q["W"])
    announce(f"gemm at max strides, bmode {bmode}: lda = ldb = {MAX_CODE_LD}, ldsa = ldsb = {MAX_SCALE_LD}")
    a = _strided(M, K, MAX_CODE_LD, torch.uint8, qa)
    b = _strided(N, K, MAX_CODE_LD, torch.uint8, qb)
    sa_d = _strided(M, sa.shape[1], MAX_SCALE_LD, torch.float32, sa)
    sb_d = _strided(sb.shape[0], sb.shape[1], MAX_SCALE_LD, torch.float32, sb)
    mode = fp8bs.BSCALE_ROW_1x128 if bmode == oracle.BSCALE_ROW else fp8bs.BSCALE_BLOCK_128x128
    d32 = torch.empty((M, N), dtype=torch.float32, device=dev())
    d16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    fp8bs.fp8bs_gemm(a, sa_d, b, sb_d, mode, d32, fp8bs.OUT_F32)
    fp8bs.fp8bs_gemm(a, sa_d, b, sb_d, mode, d16, fp8bs.OUT_BF16)
    ref = oracle.gemm(qa, sa, qb, sb, bmode)
    check_gemm_outputs("max strides", host(d32), host(d16), ref, gemm_mag(qa, sa, qb, sb, bmode))
    del a, b, sa_d, sb_d
    torch.cuda.empty_cache()


def test_requant_at_the_largest_input_stride():
    native_loaded()
    T, C = 130, 256
    d = synth.wgrad(T=T, C_in=C, C_out=128, seed=78)
    q1, s1 = oracle.quant_act_1x128(d["X"])
    announce(f"requant at max input stride: ld_in = {MAX_REQUANT_LD}, lds_in = {MAX_SCALE_LD}")
    x = _strided(T, C, MAX_REQUANT_LD, torch.uint8, q1)
    si = _strided(T, C // 128, MAX_SCALE_LD, torch.float32, s1)
    TB = (T + 127) // 128
    q = torch.empty((C, 144), dtype=torch.uint8, device=dev())
    s = torch.empty((C, TB), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_FP8_1x128, x, si, q[:, :T], s)
    qr, sr = oracle.requant_T_128x1_fp8(q1, s1)
    check_quant_equal("requant max stride", host(q)[:, :T], host(s), qr, sr)
    del x, si
    torch.cuda.empty_cache()
