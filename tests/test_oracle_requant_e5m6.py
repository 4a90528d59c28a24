"""Pin of the oracle's re-quantization from E5M6-cached activations
(oracle.requant_T_128x1_e5m6 = the exact E5M6 decode, then the bf16-source
re-quantization) to the bf16 path and to the FP8-source path, through
values the format holds exactly."""
import numpy as np

import oracle


def test_requant_from_e5m6_is_the_bf16_requant_where_e5m6_is_exact():
    """bf16 values with at most 6 mantissa bits in the E5M6 range survive
    the encoding unchanged, so re-quantizing their E5M6 rows gives the codes
    and scales of re-quantizing the bf16 rows directly."""
    rng = np.random.default_rng(5)
    T, C = 300, 256
    mant = rng.integers(0, 64, (T, C)).astype(np.uint32)
    exp = rng.integers(127 - 14, 127 + 15, (T, C)).astype(np.uint32)   # E5M6 normal range
    sign = rng.integers(0, 2, (T, C)).astype(np.uint32)
    x = ((sign << 15) | (exp << 7) | (mant << 1)).astype(np.uint16)
    y = oracle.encode_e5m6(x)
    assert (oracle.decode_e5m6(y, C) == x).all()
    q1, s1 = oracle.requant_T_128x1_e5m6(y, C)
    q2, s2 = oracle.requant_T_128x1_bf16(x)
    assert (q1 == q2).all() and (s1.view(np.uint32) == s2.view(np.uint32)).all()


def test_requant_from_e5m6_is_the_fp8_requant_of_power_of_two_scaled_codes():
    """Rows of E4M3 values times a power-of-two 1x128 scale: the FP8-source
    re-quantization dequantizes them exactly (one FP32 multiply by a power
    of two), and E5M6 holds them exactly (3 mantissa bits, exponents kept in
    the format's range), so both re-quantizations see the same values and
    must give the same codes and scales."""
    rng = np.random.default_rng(6)
    T, C = 260, 384
    q = rng.integers(0, 256, (T, C)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3A                       # no NaN codes
    e = rng.integers(-6, 7, (T, C // 128))             # E4M3 2^-9..448 times 2^e stays in E5M6 range
    s1 = np.ldexp(np.ones((T, C // 128)), e).astype(np.float32)
    v = oracle.e4m3_table()[q] * np.repeat(s1, 128, axis=1).astype(np.float64)
    x = oracle.round_to_bf16(v)
    back = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert (back == v).all()                           # bf16 holds them exactly
    y = oracle.encode_e5m6(x)
    assert (oracle.decode_e5m6(y, C) == x).all()       # and so does E5M6
    q1, sc1 = oracle.requant_T_128x1_e5m6(y, C)
    q2, sc2 = oracle.requant_T_128x1_fp8(q, s1)
    assert (q1 == q2).all() and (sc1.view(np.uint32) == sc2.view(np.uint32)).all()
