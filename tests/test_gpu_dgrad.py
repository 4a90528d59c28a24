"""GPU parity of the backward pass for the input, dX = dY W: the transpose of
the 128x128-block-quantized weight (bit-exact codes and scale grid against
the CPU oracle) and the whole input-gradient path at full size (quant_act of
dY, quant_w of W, the transpose and the block-scaled GEMM, all on the GPU)
against the oracle on sampled entries."""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import (announce, bf16_dev, check_quant_equal, dev, f32_dev, host,
                              native_loaded, sampled_check, u8_dev)

pytestmark = pytest.mark.gpu


def _transpose_dev(q, s, pad_q=0, pad_s=0, pad_qt=0, pad_st=0):
    """fp8bs_transpose_w_128x128 on host arrays with padded row strides;
    checks that nothing past a row (or past the scale grid) is written."""
    N, K = q.shape
    qd = torch.zeros((N, K + pad_q), dtype=torch.uint8, device=dev()); qd[:, :K] = u8_dev(q)
    sd = torch.zeros((N // 128, K // 128 + pad_s), dtype=torch.float32, device=dev())
    sd[:, :K // 128] = f32_dev(s)
    qt = torch.full((K, N + pad_qt), 0x55, dtype=torch.uint8, device=dev())
    st = torch.full((K // 128, N // 128 + pad_st), -3.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_transpose_w_128x128(qd[:, :K], sd[:, :K // 128], qt[:, :N], st[:, :N // 128])
    qth, sth = host(qt), host(st)
    assert (qth[:, N:] == 0x55).all(), "wrote past an output row"
    assert (sth[:, N // 128:] == -3.0).all(), "wrote past a scale row"
    return qth[:, :N], sth[:, :N // 128]


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (640, 1152)])
def test_transpose_w_bit_exact_strided(N, K):
    native_loaded()
    announce(f"transpose_w {N}x{K} strided")
    w = synth.wgrad(T=128, C_in=K, C_out=N, seed=N + K, with_w=True)["W"]
    q, s = oracle.quant_w_128x128(w)
    q_ref, s_ref = oracle.transpose_w_128x128(q, s)
    qt, st = _transpose_dev(q, s, pad_q=16, pad_s=3, pad_qt=32, pad_st=2)
    check_quant_equal(f"transpose_w {N}x{K}", qt, st, q_ref, s_ref)


@pytest.mark.parametrize("which", ["wgrad_W_2048x7168", "mlp_up_W_18432x7168"])
def test_transpose_w_full_size(which):
    """The weights of the two dense layers: W [2048][7168] of the backward
    shapes and the up-projection W [18432][7168]."""
    native_loaded()
    announce(f"transpose_w {which}: inputs")
    if which.startswith("wgrad"):
        w = synth.wgrad(with_w=True)["W"]
    else:
        w = synth.mlp_up(T=128)["W"]
    q, s = oracle.quant_w_128x128(w)
    del w
    q_ref, s_ref = oracle.transpose_w_128x128(q, s)
    announce(f"transpose_w {which}: gpu")
    qt, st = fp8bs.transpose_w_128x128(u8_dev(q), f32_dev(s))
    check_quant_equal(f"transpose_w {which}", host(qt), host(st), q_ref, s_ref)


def test_input_gradient_full_size_sampled():
    """dX [8192][7168] = dY [8192][2048] W [2048][7168]: dY quantized 1x128
    along C_out, W quantized in 128x128 blocks and transposed, both on the
    GPU; BF16 and FP32 outputs; sampled entries vs the oracle."""
    native_loaded()
    announce("input gradient 8192x7168x2048: inputs")
    d = synth.wgrad(with_w=True)
    qdy, sdy = oracle.quant_act_1x128(d["dY"])
    qw, sw = oracle.quant_w_128x128(d["W"])
    qwt, swt = oracle.transpose_w_128x128(qw, sw)
    announce("input gradient: gpu quantization and transpose")
    gq, gs = fp8bs.quant_act_1x128(bf16_dev(d["dY"]))
    gw, gsw = fp8bs.quant_w_128x128(bf16_dev(d["W"]))
    gwt, gswt = fp8bs.transpose_w_128x128(gw, gsw)
    check_quant_equal("dY quant_act", host(gq), host(gs), qdy, sdy)
    check_quant_equal("W^T", host(gwt), host(gswt), qwt, swt)
    announce("input gradient: gpu gemm")
    out = fp8bs.gemm(gq, gs, gwt, gswt)
    out32 = fp8bs.gemm(gq, gs, gwt, gswt, out_f32=True)
    sampled_check("input gradient", qdy, sdy, qwt, swt, out32, out, max_flip_share=0.03)   # measured 1.0 %
    assert torch.isfinite(out32).all()
