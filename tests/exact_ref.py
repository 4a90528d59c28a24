"""Independent brute-force references used to pin the oracle.

Nothing here calls the oracle.  The E4M3 value table comes from PyTorch's
``float8_e4m3fn`` dtype (a library decoder written by others), quotients are
exact rationals (``fractions.Fraction``), FP32 scale arithmetic is numpy's
IEEE binary32 arithmetic, and the nearest code is found by scanning.
Slow on purpose; used on small inputs only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def torch_e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 codes, decoded by PyTorch."""
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


_TAB = torch_e4m3_table()
# non-negative finite codes and their magnitudes (exact rationals)
_POS_CODES = [c for c in range(128) if np.isfinite(_TAB[c])]
_POS_VALS = [Fraction(float(_TAB[c])) for c in _POS_CODES]
_MAXV = max(_POS_VALS)


_POS_FLOATS = np.array([float(v) for v in _POS_VALS])


def nearest_code(q: Fraction, negative: bool) -> int:
    """Nearest E4M3 code to the exact rational q (sign given separately so
    that -0 keeps its sign); ties to the even code; saturating.  The exact
    comparison runs over the few codes whose float value is closest."""
    a = abs(q)
    sign = 0x80 if negative else 0x00
    if a >= _MAXV:
        return sign | _POS_CODES[_POS_VALS.index(_MAXV)]
    i = int(np.searchsorted(_POS_FLOATS, float(a)))
    cands = range(max(0, i - 2), min(len(_POS_CODES), i + 2))
    best = None
    best_d = None
    for j in cands:
        c, v = _POS_CODES[j], _POS_VALS[j]
        d = abs(a - v)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return sign | best


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_scale(amax: np.float32) -> np.float32:
    """IEEE binary32 amax / 448 (numpy float32 division)."""
    with np.errstate(all="ignore"):
        return np.float32(amax) / np.float32(448.0)


def quantize_group_exact(vals_f32: np.ndarray):
    """Quantize one group of float32 values: (codes, scale) with
    s = fl32(amax/448) and code = nearest-even E4M3 of the exact x/s."""
    vals = np.asarray(vals_f32, dtype=np.float32).ravel()
    amax = np.float32(np.max(np.abs(vals))) if vals.size else np.float32(0)
    s = f32_scale(amax)
    codes = []
    for x in vals:
        neg = bool(np.signbit(x))
        if s == 0:
            codes.append(0x80 if neg else 0x00)
        else:
            codes.append(nearest_code(Fraction(float(x)) / Fraction(float(s)), neg))
    return np.array(codes, dtype=np.uint8), s


def e4m3_dec_f32(codes) -> np.ndarray:
    return _TAB[np.asarray(codes, dtype=np.int64)].astype(np.float32)


def bf16_round_exact(v: Fraction) -> int:
    """Nearest-even bf16 bit pattern of an exact rational (finite, within
    range), by scanning the two bracketing bf16 values."""
    neg = v < 0
    a = abs(v)
    if a == 0:
        return 0x8000 if neg else 0
    # find exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    k = a / quantum
    fl = k.numerator // k.denominator
    frac = k - fl
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = float(fl * quantum)
    bits = int(np.array([val], dtype=np.float32).view(np.uint32)[0] >> 16)
    return bits | (0x8000 if neg else 0)
