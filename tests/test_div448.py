"""The BF16-A GEMM computes a 1x128 tile's scale fl32(amax / 448) as
q0 = fl32(amax * c), r = fma(-q0, 448, amax), q = fma(r, c, q0) with
c = fl32(1 / 448), and keeps q when q >= 2^-100 (smaller and non-finite
quotients take the IEEE division).  amax is the largest magnitude of BF16
values, so it is itself a BF16 value: this test runs every positive finite
BF16 value through exact rational arithmetic (each operation rounded once to
binary32, nearest-even, as v_mul_f32 and v_fma_f32 round) and checks q
against the correctly rounded quotient wherever q >= 2^-100.  The scale is
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
