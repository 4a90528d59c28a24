"""GPU parity of the re-quantization from E5M6-cached activations
(fp8bs_requant_T_128x1 with FP8BS_SRC_E5M6; [p1] para 3: E5M6 for some
activations cached for the backward pass, and the 1x128 -> 128x1
re-quantization in the backward pass) against oracle.requant_T_128x1_e5m6
(the exact decode, then the bf16-source re-quantization): codes and scales
bit-exact, at the weight-gradient shape, ragged and strided, and equal to
the two-kernel path (decode to bf16, then re-quantize the bf16 rows)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import announce, check_quant_equal, dev, host, native_loaded, u8_dev

pytestmark = pytest.mark.gpu


def run_requant_e5m6(y, C, ld_in_pad=0, ld_out_pad=0, lds_out_pad=0):
    """Packed rows y [T][1.5 C] (host) through the fused re-quantization,
    with optional padding of every row stride; returns (q [C][T], s)."""
    T = y.shape[0]
    TB = (T + 127) // 128
    W = C // 2 * 3
    x = torch.zeros((T, W + ld_in_pad), dtype=torch.uint8, device=dev())
    x[:, :W] = u8_dev(y)
    Tp = (T + 15) // 16 * 16 + ld_out_pad
    q = torch.full((C, Tp), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((C, TB + lds_out_pad), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_E5M6, x[:, :W], None, q[:, :T], s[:, :TB])
    qh, sh = host(q), host(s)
    assert (qh[:, T:] == 0x55).all(), "wrote past the output row"
    if lds_out_pad:
        assert (sh[:, TB:] == -1.0).all(), "wrote past the scale row"
    return qh[:, :T], sh[:, :TB]


def test_requant_e5m6_wgrad_X_full():
    """X [8192][7168] of the weight-gradient configuration, cached as E5M6."""
    native_loaded()
    x = synth.wgrad()["X"]
    y = oracle.encode_e5m6(x)
    C = x.shape[1]
    announce("requant e5m6 8192x7168")
    q, s = run_requant_e5m6(y, C)
    check_quant_equal("requant e5m6 full", q, s, *oracle.requant_T_128x1_e5m6(y, C))
    # the same as decoding to bf16 and re-quantizing those rows on the GPU
    yd = u8_dev(y)
    xb = fp8bs.decode_e5m6(yd, C)
    q2, s2 = fp8bs.requant_T_128x1(xb)
    check_quant_equal("requant e5m6 vs decode + requant bf16", q, s, host(q2), host(s2))


@pytest.mark.parametrize("T", [1, 127, 300, 4097])
def test_requant_e5m6_ragged_strided(T):
    """Ragged token counts (rows past T read as zeros), padded input rows,
    output rows and scale rows with sentinels."""
    native_loaded()
    d = synth.wgrad(T=T, C_in=640, C_out=128, seed=T)
    y = oracle.encode_e5m6(d["X"])
    announce(f"requant e5m6 ragged T={T}")
    q, s = run_requant_e5m6(y, 640, ld_in_pad=32, ld_out_pad=16, lds_out_pad=2)
    check_quant_equal(f"requant e5m6 T={T}", q, s, *oracle.requant_T_128x1_e5m6(y, 640))


def test_requant_e5m6_special_values():
    """Codes at the edges of the format: zeros of both signs, subnormals,
    the largest finite value 65024 and mixed magnitudes in one tile."""
    native_loaded()
    rng = np.random.default_rng(11)
    T, C = 256, 256
    codes = rng.integers(0, 0x7C0, (T, C)) | (rng.integers(0, 2, (T, C)) << 11)   # finite codes
    codes[0:128, 0:64] = rng.integers(0, 64, (128, 64))          # subnormal (exponent 0) only
    codes[128:256, 64:128] = 0x7BF                               # 65024 everywhere
    codes[:, 128:192] = 0x800                                    # -0 tiles
    codes[5, 200] = 0x7BF | 0x800                                # -65024 in a mixed tile
    flat = codes.astype(np.uint64).reshape(T, C // 8, 8)
    words = np.zeros((T, C // 8), dtype=np.uint64)
    for i in range(8):
        words |= flat[:, :, i] << np.uint64(12 * i)
    y = np.zeros((T, C // 8, 12), np.uint8)
    for b in range(12):
        y[:, :, b] = ((words >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
    y = y.reshape(T, C // 2 * 3)
    assert (oracle.encode_e5m6(oracle.decode_e5m6(y, C)) == y).all()   # the packing above is the format's
    announce("requant e5m6 special values")
    q, s = run_requant_e5m6(y, C)
    check_quant_equal("requant e5m6 special", q, s, *oracle.requant_T_128x1_e5m6(y, C))
