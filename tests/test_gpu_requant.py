"""GPU parity of the backward 1x128 -> 128x1 re-quantization (FP8 and bf16
sources): bit-exact codes and scales against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import (announce, bf16_dev, check_quant_equal, dev, f32_dev,
                              host, native_loaded, u8_dev)

pytestmark = pytest.mark.gpu


def _run_requant(src_u8_or_u16, s_in=None, ld_in_pad=0, ld_out_pad=0, lds_out_pad=0):
    T, C = src_u8_or_u16.shape
    TB = (T + 127) // 128
    if s_in is not None:
        x = torch.zeros((T, C + ld_in_pad), dtype=torch.uint8, device=dev())
        x[:, :C] = u8_dev(src_u8_or_u16)
        si = f32_dev(s_in)
        src = fp8bs.SRC_FP8_1x128
    else:
        x = torch.zeros((T, C + ld_in_pad), dtype=torch.bfloat16, device=dev())
        x[:, :C] = bf16_dev(src_u8_or_u16)
        si = None
        src = fp8bs.SRC_BF16
    Tp = (T + 15) // 16 * 16 + ld_out_pad
    q = torch.full((C, Tp), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((C, TB + lds_out_pad), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_requant_T_128x1(src, x[:, :C], si, q[:, :T], s[:, :TB])
    qh, sh = host(q), host(s)
    assert (qh[:, T:] == 0x55).all(), "wrote past the output row"
    if lds_out_pad:
        assert (sh[:, TB:] == -1.0).all()
    return qh[:, :T], sh[:, :TB]


def test_requant_fp8_wgrad_X_full():
    native_loaded()
    announce("requant fp8 wgrad X 8192x7168")
    x = synth.wgrad()["X"]
    q1, s1 = oracle.quant_act_1x128(x)
    q, s = _run_requant(q1, s1)
    qr, sr = oracle.requant_T_128x1_fp8(q1, s1)
    check_quant_equal("requant X", q, s, qr, sr)


def test_requant_bf16_wgrad_dY_full():
    native_loaded()
    announce("requant bf16 wgrad dY 8192x2048")
    dy = synth.wgrad()["dY"]
    q, s = _run_requant(dy)
    qr, sr = oracle.requant_T_128x1_bf16(dy)
    check_quant_equal("requant dY", q, s, qr, sr)


@pytest.mark.parametrize("T", [1, 100, 1000, 8200])
def test_requant_ragged_strided(T):
    native_loaded()
    announce(f"requant ragged T={T}")
    d = synth.wgrad(T=T, C_in=384, C_out=256, seed=T)
    q1, s1 = oracle.quant_act_1x128(d["X"])
    q, s = _run_requant(q1, s1, ld_in_pad=16, ld_out_pad=16, lds_out_pad=2)
    qr, sr = oracle.requant_T_128x1_fp8(q1, s1)
    check_quant_equal(f"requant fp8 T={T}", q, s, qr, sr)
    q, s = _run_requant(d["dY"], ld_in_pad=8, ld_out_pad=32, lds_out_pad=1)
    qr, sr = oracle.requant_T_128x1_bf16(d["dY"])
    check_quant_equal(f"requant bf16 T={T}", q, s, qr, sr)


def test_requant_edge_scales():
    """Source tiles with zero, subnormal and huge scales, and a channel of
    all-zero codes."""
    native_loaded()
    rng = np.random.default_rng(8)
    T, C = 384, 256
    q1 = rng.integers(0, 256, (T, C)).astype(np.uint8)
    q1[(q1 & 0x7F) == 0x7F] = 0x01
    q1[:, 5] = 0x00
    q1[:, 6] = 0x80
    s1 = (rng.uniform(0.5, 2, (T, 2)) * 2.0 ** rng.integers(-60, 60, (T, 2))).astype(np.float32)
    s1[:50, 0] = 0.0
    s1[50:100, 0] = np.float32(2.0 ** -140)          # subnormal scale: subnormal values
    s1[100:130, 1] = np.float32(2.0 ** -149)
    s1[130:200, 1] = np.float32(3.0e35)              # dec * s up to ~1.3e38
    announce("requant edge scales")
    q, s = _run_requant(q1, s1)
    qr, sr = oracle.requant_T_128x1_fp8(q1, s1)
    check_quant_equal("requant edge", q, s, qr, sr)


def test_requant_deterministic():
    native_loaded()
    d = synth.wgrad(T=1024, C_in=1024, C_out=128)
    q1, s1 = oracle.quant_act_1x128(d["X"])
    a = _run_requant(q1, s1)
    b = _run_requant(q1, s1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
