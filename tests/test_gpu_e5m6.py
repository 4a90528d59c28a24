"""GPU parity of the E5M6 cached-activation format: encoding bit-exact over
every finite bf16 value and at the backward shapes, decoding exact, and the
backward re-quantization of decoded rows equal to the oracle's.  Also the
accuracy of the weight gradient with activations cached in E5M6 against
activations cached as 1x128 FP8 (the pages keep E5M6 for activations that
the backward pass re-quantizes)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import announce, bf16_dev, check_quant_equal, dev, host, native_loaded, u8_dev

pytestmark = pytest.mark.gpu


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    b[((b >> 7) & 0xFF) == 0xFF] = 0            # infinities and NaNs are out of contract
    return b.astype(np.uint16).reshape(512, 128)


def _encode_dev(x_u16, pad_x=0, pad_y=0):
    T, C = x_u16.shape
    xd = torch.zeros((T, C + pad_x), dtype=torch.bfloat16, device=dev())
    xd[:, :C] = bf16_dev(x_u16)
    y = torch.full((T, C // 2 * 3 + pad_y), 0x5A, dtype=torch.uint8, device=dev())
    fp8bs.fp8bs_encode_e5m6(xd[:, :C], y[:, :C // 2 * 3])
    yh = host(y)
    assert (yh[:, C // 2 * 3:] == 0x5A).all(), "wrote past a packed row"
    return yh[:, :C // 2 * 3]


def _decode_dev(y_u8, C, pad_x=0):
    T = y_u8.shape[0]
    x = torch.full((T, C + pad_x), 3.0, dtype=torch.bfloat16, device=dev())
    fp8bs.fp8bs_decode_e5m6(u8_dev(y_u8), x[:, :C])
    xh = host(x)
    assert (xh[:, C:] == 0x4040).all(), "wrote past a bf16 row"
    return xh[:, :C]


def test_e5m6_every_finite_bf16_value():
    native_loaded()
    x = _all_finite_bf16()
    announce("e5m6 encode/decode, every finite bf16 value")
    ref = oracle.encode_e5m6(x)
    y = _encode_dev(x, pad_x=16, pad_y=16)
    assert np.array_equal(y, ref), f"{int((y != ref).sum())} packed bytes differ"
    back = _decode_dev(ref, 128, pad_x=8)
    assert np.array_equal(back, oracle.decode_e5m6(ref, 128))


def _pack_codes(codes):
    """12-bit codes [T][C] -> packed rows (value i in bits 12 i .. 12 i + 11)."""
    T, C = codes.shape
    c = codes.astype(np.uint16)
    y = np.empty((T, C // 2 * 3), np.uint8)
    y[:, 0::3] = (c[:, 0::2] & 0xFF).astype(np.uint8)
    y[:, 1::3] = ((c[:, 0::2] >> 8) | ((c[:, 1::2] & 0xF) << 4)).astype(np.uint8)
    y[:, 2::3] = (c[:, 1::2] >> 4).astype(np.uint8)
    return y


def test_e5m6_decode_every_code():
    """All 4096 codes, NaN codes with every payload and both signs included:
    the oracle's bf16 patterns bit for bit (a NaN code decodes to the quiet
    NaN 0x7FC0 of its sign), in two orders so every code sits at every
    position of an 8-value group."""
    native_loaded()
    codes = np.arange(4096, dtype=np.uint16).reshape(32, 128)
    # the helper packs as the oracle's encoder does (rows of finite codes)
    fin = ~(((codes >> 6) & 31) == 31).any(axis=1)
    y = _pack_codes(codes)
    assert np.array_equal(oracle.encode_e5m6(oracle.decode_e5m6(y, 128))[fin], y[fin])
    for shift in (0, 3):
        c = np.roll(codes.ravel(), shift).reshape(32, 128)
        y = _pack_codes(c)
        announce(f"e5m6 decode, every code, shift {shift}")
        got = _decode_dev(y, 128, pad_x=8)
        ref = oracle.decode_e5m6(y, 128)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (f"{bad.size} values differ, first code {int(c.ravel()[bad[0]]):#05x}: "
                               f"{int(got.ravel()[bad[0]]):#06x} vs {int(ref.ravel()[bad[0]]):#06x}")
    nan = ((codes >> 6) & 31 == 31) & (codes & 63 != 0)
    ref = oracle.decode_e5m6(_pack_codes(codes), 128)
    assert set(np.unique(ref[nan])) == {0x7FC0, 0xFFC0}


def test_e5m6_backward_shape_and_requant_of_decoded_rows():
    """X [8192][7168] cached in E5M6, decoded, re-quantized to 128x1 tiles:
    every step bit-exact against the oracle."""
    native_loaded()
    announce("e5m6 X 8192x7168: inputs")
    x = synth.wgrad()["X"]
    ref_y = oracle.encode_e5m6(x)
    ref_x = oracle.decode_e5m6(ref_y, x.shape[1])
    q_ref, s_ref = oracle.requant_T_128x1_bf16(ref_x)
    announce("e5m6 X 8192x7168: gpu")
    y = fp8bs.encode_e5m6(bf16_dev(x))
    assert np.array_equal(host(y), ref_y)
    xd = fp8bs.decode_e5m6(y, x.shape[1])
    assert np.array_equal(host(xd), ref_x)
    q, s = fp8bs.requant_T_128x1(xd)
    check_quant_equal("requant of decoded E5M6 rows", host(q), host(s), q_ref, s_ref)


def test_weight_gradient_accuracy_e5m6_cache_vs_fp8_cache():
    """dW = X^T dY with X cached as 1x128 FP8 (re-quantized 1x128 -> 128x1)
    and with X cached in E5M6 (decoded, quantized once to 128x1), both on the
    GPU, against the binary64 product of the unquantized inputs."""
    native_loaded()
    d = synth.wgrad(T=2048, C_in=1024, C_out=256)
    X, dY = bf16_dev(d["X"]), bf16_dev(d["dY"])
    qdy, sdy = fp8bs.requant_T_128x1(dY)                         # [256][2048]
    qx, sx = fp8bs.quant_act_1x128(X)                            # FP8 cache
    qa1, sa1 = fp8bs.requant_T_128x1(qx, sx)
    dw_fp8 = host(fp8bs.gemm(qa1, sa1, qdy, sdy, fp8bs.BSCALE_ROW_1x128, out_f32=True)).astype(np.float64)
    xe = fp8bs.decode_e5m6(fp8bs.encode_e5m6(X), X.shape[1])     # E5M6 cache
    qa2, sa2 = fp8bs.requant_T_128x1(xe)
    dw_e5m6 = host(fp8bs.gemm(qa2, sa2, qdy, sdy, fp8bs.BSCALE_ROW_1x128, out_f32=True)).astype(np.float64)
    exact = oracle.gemm_bf16_f64(np.ascontiguousarray(d["X"].T), np.ascontiguousarray(d["dY"].T))
    e1 = np.linalg.norm(dw_fp8 - exact) / np.linalg.norm(exact)
    e2 = np.linalg.norm(dw_e5m6 - exact) / np.linalg.norm(exact)
    announce(f"weight gradient rel-Frobenius: FP8 cache {e1:.3e}, E5M6 cache {e2:.3e}")
    assert e2 < e1
