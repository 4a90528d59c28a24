"""Pins of the oracle's E4M3 and bf16 codecs against sources other than
itself: the OCP format facts (golden file), PyTorch's float8_e4m3fn decoder
and encoder, exhaustive scans and exact rationals."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.exact_ref import bf16_round_exact, torch_e4m3_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_golden_facts():
    facts = json.load(open(os.path.join(GOLDEN, "e4m3_ocp_facts.json")))
    tab = oracle.e4m3_table()
    for c in facts["nan_codes"]:
        assert np.isnan(tab[c])
    assert int(np.isfinite(tab).sum()) == facts["finite_codes"]
    for c, v in facts["zero_codes"].items():
        assert tab[int(c)] == 0.0 and np.signbit(tab[int(c)]) == np.signbit(v)
    for c, v in facts["values"].items():
        assert tab[int(c)] == v, (c, tab[int(c)], v)
    fin = tab[np.isfinite(tab)]
    assert fin.max() == facts["max_normal"]
    pos = fin[fin > 0]
    assert pos.min() == facts["min_subnormal"]
    assert pos[pos >= facts["min_normal"]].min() == facts["min_normal"]
    assert pos[pos < facts["min_normal"]].max() == facts["max_subnormal"]


def test_e4m3_decode_matches_torch_all_codes():
    ours = oracle.e4m3_table()
    ref = torch_e4m3_table()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))


def test_e4m3_positive_codes_strictly_increasing():
    tab = oracle.e4m3_table()
    pos = tab[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(tab[128:255], -pos)


def test_encode_roundtrip_all_finite_codes():
    tab = oracle.e4m3_table()
    for c in range(256):
        if np.isfinite(tab[c]):
            assert oracle.e4m3_encode(tab[c]) == c


def test_encode_midpoints_ties_to_even_and_neighbours():
    tab = oracle.e4m3_table()
    for c in range(126):
        lo, hi = tab[c], tab[c + 1]
        mid = 0.5 * (lo + hi)
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even
        assert oracle.e4m3_encode(-mid) == (0x80 | even)
        assert oracle.e4m3_encode(np.nextafter(mid, -np.inf)) == c
        assert oracle.e4m3_encode(np.nextafter(mid, np.inf)) == c + 1


def test_encode_saturates_and_keeps_sign_of_zero():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.9) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00       # tie with 0 -> 0
    assert oracle.e4m3_encode(2.0 ** -10 * 1.0000001) == 0x01


def test_encode_exhaustive_bf16_against_linear_scan():
    """Every finite bf16 pattern (scale 1) against nearest-by-scan over the
    PyTorch value table."""
    bits = np.arange(65536, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]   # finite patterns only
    vals = (bits << 16).view(np.float32).astype(np.float64)
    tab = torch_e4m3_table()[:127]            # non-negative finite magnitudes
    a = np.minimum(np.abs(vals), tab.max())
    d = np.abs(a[:, None] - tab[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # tie -> even code; codes == column index
    even_ok = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(even_ok.any(axis=1), even_ok.argmax(axis=1), cand.argmax(axis=1))
    ref = pick.astype(np.uint8) | np.where(np.signbit(vals), 0x80, 0).astype(np.uint8)
    lib = oracle._load()
    ours = np.array([lib.orc_e4m3_encode(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def test_encode_matches_torch_in_range():
    """PyTorch's float32 -> float8_e4m3fn cast (round to nearest even) on
    random and near-midpoint values below 464 (above that torch gives NaN
    where the adopted reading saturates)."""
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.uniform(-460, 460, 20000),
        np.exp(rng.uniform(np.log(1e-5), np.log(460), 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    tab = oracle.e4m3_table()
    mids = 0.5 * (tab[:126] + tab[1:127])
    near = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    v = np.concatenate([v, near, -near])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    lib = oracle._load()
    ours = np.array([lib.orc_e4m3_encode(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def test_bf16_round_against_exact_and_torch():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(300) * 10.0 ** rng.uniform(-30, 30, 300))
    # exact bf16 midpoints and their neighbours in binary64
    for _ in range(200):
        b = int(rng.integers(0x0080, 0x7F00))
        lo = float((np.array([b], np.uint32) << 16).view(np.float32)[0])
        hi = float((np.array([b + 1], np.uint32) << 16).view(np.float32)[0])
        mid = 0.5 * (lo + hi)
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    vals += [2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -134, 2.0 ** -135]  # bf16 subnormal range
    for v in vals:
        assert oracle.bf16_round(v) == bf16_round_exact(Fraction(v)), v
    # float32-exact inputs: torch's float32 -> bfloat16 cast is RNE
    f = (rng.standard_normal(5000) * 10.0 ** rng.uniform(-20, 20, 5000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.round_to_bf16(f.astype(np.float64))
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# E5M6 (12-bit cached-activation format): codec pins
# ---------------------------------------------------------------------------

def _e5m6_table():
    return np.array([oracle.e5m6_value(c) for c in range(4096)])


def test_e5m6_code_space():
    """Sign, 5-bit exponent (bias 15), 6-bit mantissa, IEEE conventions:
    +-0, 2 x 63 subnormals, 2 x 1920 normals, 2 infinities, 2 x 63 NaNs;
    the non-negative finite codes ordered by value; closed-form anchors."""
    tab = _e5m6_table()
    assert np.isnan(tab).sum() == 126
    assert np.isinf(tab).sum() == 2 and tab[0x7C0] == np.inf and tab[0xFC0] == -np.inf
    pos = tab[:0x7C0]
    assert pos[0] == 0.0 and np.all(np.diff(pos) > 0)
    assert np.array_equal(tab[0x800:0x800 + 0x7C0], -pos)
    assert tab[1] == 2.0 ** -20 and tab[63] == 63 * 2.0 ** -20      # subnormals
    assert tab[64] == 2.0 ** -14                                    # smallest normal
    assert tab[15 << 6] == 1.0 and tab[(15 << 6) | 1] == 1.0 + 1 / 64
    assert tab[0x7BF] == (2 - 1 / 64) * 2.0 ** 15 == 65024.0          # largest finite


def test_e5m6_encode_roundtrip_and_every_value_is_bf16():
    tab = _e5m6_table()
    for c in list(range(0x7C0)) + list(range(0x800, 0xFC0)):
        assert oracle.e5m6_encode(tab[c]) == c
    # every finite E5M6 value is exact in bf16 (6 <= 7 mantissa bits, range inside bf16's)
    fin = tab[np.isfinite(tab)]
    b = np.array([oracle.bf16_round(v) for v in fin], np.uint16)
    assert np.array_equal(np.array([oracle.bf16_value(int(x)) for x in b]), fin)


def test_e5m6_encode_exhaustive_bf16_against_linear_scan():
    """Every finite bf16 value against the nearest of the finite magnitudes
    and 2^16 (standing for infinity under IEEE overflow), ties to the even
    code, sign copied."""
    tab = _e5m6_table()
    cand = np.concatenate([tab[:0x7C0], [65536.0]])          # codes 0 .. 0x7C0
    bits = np.arange(65536, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    vals = (bits << 16).view(np.float32).astype(np.float64)
    a = np.abs(vals)
    hi = np.searchsorted(cand, a, side="left").clip(1, len(cand) - 1)
    lo = hi - 1
    exact_hi = cand[hi] == a
    dlo, dhi = a - cand[lo], cand[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(exact_hi, hi, pick)
    pick = np.where(a >= 65536.0, 0x7C0, pick)
    want = pick | ((bits >> 15) << 11)
    got = np.array([oracle.e5m6_encode(v) for v in vals])
    assert np.array_equal(got, want)


def test_e5m6_pack_unpack_rows():
    """Packed rows (value i in bits 12 i .. 12 i + 11) decode to the values
    encoded; the packing of a known pair is spelled out."""
    rng = np.random.default_rng(5)
    tab = _e5m6_table()
    codes = rng.integers(0, 4096, (3, 256))
    codes[~np.isfinite(tab[codes])] = 0x3C0
    x = np.array([[oracle.bf16_round(tab[c]) for c in row] for row in codes], np.uint16)
    y = oracle.encode_e5m6(x)
    assert y.shape == (3, 384)
    assert np.array_equal(oracle.decode_e5m6(y, 256), x)
    c0, c1 = int(codes[0, 0]), int(codes[0, 1])
    assert y[0, 0] == c0 & 0xFF and y[0, 1] == (c0 >> 8) | ((c1 & 0xF) << 4) and y[0, 2] == c1 >> 4
