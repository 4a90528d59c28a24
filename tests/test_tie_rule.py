"""CPU model of the BF16 quantizers' E4M3 encoding (encode4_bf16 and the
BF16-A GEMM's in-LDS quantizer) against the oracle's quantizer.

The kernels compute, per value x of a tile with scale s = fl32(amax / 448)
and r within one unit in the last place of 1/s (v_rcp_f32):
  lo = E4M3(x * fl32(r (1 - 2^-20))), hi = E4M3(x * fl32(r (1 + 2^-20)))
(hardware conversion: nearest-even, saturating at 448), and where lo and hi
differ they take, per tile, the upper code if 448 s < amax (the scale was
rounded down), the even code if 448 s = amax (exact scale), the lower code
otherwise.  The claim behind it (for BF16 values and a BF16 amax, differing
brackets mean 448 x / amax is exactly the midpoint between the two codes,
so the rounding direction of s decides the side) is checked here
exhaustively: every amax significand (128 BF16 values) at three binades,
with every BF16 magnitude of both signs from 2^-24 amax up to amax in its
tiles, for three reciprocals (the correctly rounded one and its two
neighbours).  The oracle is the exact nearest-even E4M3 of x / s ([p1]
para 3, xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=32373: 1x128 tiles scaled
by their max-abs).
"""
import numpy as np
import pytest
import torch

import oracle


def _bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def _e4m3_rne_sat(y: np.ndarray) -> np.ndarray:
    """Codes of float32 values, nearest-even, saturated to +-448 (the
    hardware conversion's behaviour on [-464, 464])."""
    t = torch.from_numpy(np.clip(y, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _tiles(amax_bits: int):
    """Rows of 128 BF16 values: amax first, then every BF16 magnitude below
    it down to 2^-24 amax, with alternating signs."""
    e_amax = (amax_bits >> 7) & 0xFF
    mags = np.arange(max(e_amax - 24, 1) << 7, amax_bits + 1, dtype=np.uint32)
    vals = np.concatenate([mags, mags | 0x8000])
    n_rows = -(-vals.size // 127)
    rows = np.zeros((n_rows, 128), np.uint16)
    rows[:, 0] = amax_bits
    flat = np.full(n_rows * 127, amax_bits, np.uint16)
    flat[:vals.size] = vals
    rows[:, 1:] = flat.reshape(n_rows, 127)
    return rows


@pytest.mark.parametrize("binade", [127, 120, 134])
def test_side_rule_matches_the_oracle(binade):
    differing = {"up": 0, "down": 0, "even": 0}
    for mant in range(128):
        amax_bits = (binade << 7) | mant
        amax = np.float32(_bf16_bits_to_f32(amax_bits))
        rows = _tiles(amax_bits)
        q_ref, s_ref = oracle.quant_act_1x128(rows)
        x = _bf16_bits_to_f32(rows)
        s = np.float32(s_ref[0, 0])
        assert (s_ref[:, 0] == s).all() and s == amax / np.float32(448)
        # sign of 448 s - amax (exact in binary64: 448 s has 27 bits)
        d = 448.0 * float(s) - float(amax)
        side = "up" if d < 0 else ("even" if d == 0 else "down")
        r0 = np.float32(1) / s
        for r in (r0, np.nextafter(r0, np.float32(0)), np.nextafter(r0, np.float32(np.inf))):
            rlo = np.float32(r * np.float32(1 - 2 ** -20))
            rhi = np.float32(r * np.float32(1 + 2 ** -20))
            lo = _e4m3_rne_sat((x * rlo).astype(np.float32))
            hi = _e4m3_rne_sat((x * rhi).astype(np.float32))
            differ = lo != hi
            if differ.any():
                # differing codes are adjacent magnitudes of the same sign
                assert ((hi[differ] & 0x7F).astype(int) - (lo[differ] & 0x7F) == 1).all()
                assert (hi[differ] >> 7 == lo[differ] >> 7).all()
            pick = {"up": hi, "down": lo, "even": np.where((lo & 1) == 0, lo, hi)}[side]
            model = np.where(differ, pick, lo)
            bad = model != q_ref
            assert not bad.any(), (hex(amax_bits), side, x[bad][:4], model[bad][:4], q_ref[bad][:4])
            differing[side] += int(differ.sum())
    # all three sides occur in this sweep
    assert min(differing.values()) > 0, differing


def test_exact_scales_are_multiples_of_7():
    """448 s = amax exactly (the even-code side) for the amax significands
    that are multiples of 7, and only for those."""
    for mant in range(128):
        a = np.float32(_bf16_bits_to_f32((127 << 7) | mant))
        s = a / np.float32(448)
        exact = 448.0 * float(s) == float(a)
        assert exact == ((128 + mant) % 7 == 0), mant
