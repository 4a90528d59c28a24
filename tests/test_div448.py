"""The quantizers compute a tile's scale fl32(amax / 448) as
q0 = fl32(amax * c), r = fma(-q0, 448, amax), q = fma(r, c, q0) with
c = fl32(1 / 448), and keeps q when q >= 2^-100 (smaller and non-finite
quotients take the IEEE division).  The first test runs every positive
finite BF16 value (the amax of a BF16 tile is one) through exact rational
arithmetic (each operation rounded once to binary32, nearest-even, as
v_mul_f32 and v_fma_f32 round) and checks q against the correctly rounded
quotient wherever q >= 2^-100; the second covers every binary32 amax (the
FP8-source re-quantization, SwiGLU and the GEMM's quantized output take the
max of FP32 values) through the 2^23 significands.  The scale is
the definition of [p1] para 3 (xn--9g3bo1gtkw0l8ubf92bgle.kr post
wr_id=32373): s = amax / 448 per 1x128 tile."""
from fractions import Fraction as F

import numpy as np


def rn32(x: F) -> F:
    """x rounded to the nearest binary32 value, ties to even (normal and
    subnormal range; no overflow in this test)."""
    if x == 0:
        return F(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    quantum = F(2) ** (max(e, -126) - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return (fl * quantum) * (1 if x > 0 else -1)


def test_rn32_agrees_with_numpy():
    rng = np.random.default_rng(0)
    for v in rng.standard_normal(200) * 10.0 ** rng.integers(-40, 38, 200):
        assert rn32(F(float(v))) == F(float(np.float32(v)))


def test_fast_division_by_448_is_exact_for_every_bf16():
    c = rn32(F(1, 448))
    assert c == F(float(np.float32(1) / np.float32(448)))
    checked = 0
    for bits in range(0x0001, 0x7F80):          # every positive finite BF16 value
        a = F(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))
        q0 = rn32(a * c)
        r = rn32(a - q0 * 448)
        q = rn32(r * c + q0)
        if q >= F(2) ** -100:
            assert q == rn32(a / 448), hex(bits)
            checked += 1
    assert checked == 28064          # all BF16 values from about 2^-91.2 up


def _rne_div(n, d):
    """Round to nearest, ties to even, of n / d for int64 arrays n >= 0 and a
    positive integer d."""
    q, r = np.divmod(n, d)
    return q + ((2 * r > d) | ((2 * r == d) & (q % 2 == 1)))


def test_fast_division_by_448_is_exact_for_every_fp32_significand():
    """The same three operations for every binary32 significand, in exact
    integer arithmetic.  Scaling a by a power of two scales q0, r and q
    exactly while all of them stay normal, which holds for quotients of at
    least 2^-100 (r is about 2^-15 q), so the significands of one binade
    cover every such input.  With a = A 2^-23 (A in [2^23, 2^24)) and
    c = C 2^-32, every quantity is an integer multiple of a power of two:
    q0 in units of 2^-32 (2^-31 at and above 2^-8), r = A 2^9 - 448 Q0 in
    units of 2^-32 (exact), r c + q0 in units of 2^-64, and the exact
    quotient a / 448 = (8 A / 7) 2^-32."""
    A = np.arange(1 << 23, 1 << 24, dtype=np.int64)
    C = int(rn32(F(1, 448)) * 2 ** 32)
    assert (1 << 23) <= C < (1 << 24)
    P = A * C                                                   # a c, units of 2^-55
    Q0 = np.where(P < (1 << 47), _rne_div(P, 1 << 23), 2 * _rne_div(P, 1 << 24))
    NR = A * 512 - 448 * Q0                                     # r, units of 2^-32
    assert np.abs(NR).max() < (1 << 24)                         # r is a binary32 value
    V = NR * C + Q0 * (1 << 32)                                 # r c + q0, units of 2^-64
    Q = np.where(V < (1 << 56), _rne_div(V, 1 << 32), 2 * _rne_div(V, 1 << 33))
    X = A * 8                                                   # exact quotient: X / 7
    QX = np.where(X < 7 * (1 << 24), _rne_div(X, 7), 2 * _rne_div(X, 14))
    assert (Q == QX).all(), f"{int((Q != QX).sum())} significands differ"
    # the correction step matters: q0 alone is wrong for about half of them
    assert (Q0 != QX).sum() > (1 << 21)
    # spot checks of the integer model against the rational one above
    for a_int in (A[0], A[12345], A[-1], 0x924925):
        a = F(int(a_int), 1 << 23)
        q0 = rn32(a * rn32(F(1, 448)))
        q = rn32(rn32(a - q0 * 448) * rn32(F(1, 448)) + q0)
        i = int(a_int) - (1 << 23)
        assert q == F(int(Q[i]), 1 << 32) and q == rn32(a / 448)
