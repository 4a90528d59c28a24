"""The E4M3 encoder on every FP32 bit pattern, on the GPU
(fp8bs_cast_e4m3: the quantizers' encoder run with a unit scale after
saturation to +-448), against the oracle's encoder.

Non-negative FP32 bit patterns order like their values, and nearest-even
encoding is a non-decreasing step function of the value, so on the
2^31 - 2^23 finite non-negative patterns (and +inf, which saturates) the
device agrees with the oracle everywhere iff
  * its codes are non-decreasing in the bit pattern and never above 0x7E, and
  * at each of the oracle's 126 steps (the first pattern b_c the oracle
    encodes to c) it gives c at b_c and c - 1 at b_c - 1.
Every negative pattern must give the code of its magnitude with the sign bit
set.  The steps come from the oracle by bisection; the sweep runs the device
over all 2^32 - 2^24 + 2 finite-or-infinite patterns in 16 chunks.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs
from tests.gpu_common import announce, dev, host, native_loaded

pytestmark = pytest.mark.gpu

POS_INF = 0x7F800000
SIGN = -(1 << 31)        # int32 bit pattern of the sign bit


def _f32(u: int) -> float:
    return float(np.array([u], np.uint32).view(np.float32)[0])


def _oracle_steps() -> np.ndarray:
    """b[c - 1] = the smallest non-negative finite pattern the oracle encodes
    to a code >= c, for c = 1 .. 126."""
    steps = []
    for c in range(1, 127):
        lo, hi = 0, POS_INF - 1
        while lo < hi:
            mid = (lo + hi) // 2
            if oracle.e4m3_encode(_f32(mid)) >= c:
                hi = mid
            else:
                lo = mid + 1
        steps.append(lo)
    return np.array(steps, np.int64)


def _cast(x: torch.Tensor) -> torch.Tensor:
    q = torch.empty(x.numel(), dtype=torch.uint8, device=x.device)
    fp8bs.fp8bs_cast_e4m3(x, q)
    return q


def test_cast_every_fp32_pattern_against_the_oracle_steps():
    native_loaded()
    announce("cast_e4m3: oracle steps")
    b = _oracle_steps()
    assert np.all(np.diff(b) > 0)
    assert oracle.e4m3_encode(_f32(int(b[-1]))) == 0x7E and oracle.e4m3_encode(_f32(POS_INF - 1)) == 0x7E
    pts = np.concatenate([b, b - 1]).astype(np.uint32)
    want = np.concatenate([np.arange(1, 127), np.arange(0, 126)]).astype(np.uint8)
    assert [oracle.e4m3_encode(_f32(int(u))) for u in pts] == want.tolist()
    announce("cast_e4m3: device at the steps")
    got = host(_cast(torch.from_numpy(pts.view(np.float32)).to(dev())))
    assert np.array_equal(got, want), np.nonzero(got != want)
    chunk = 1 << 27
    last = 0
    for start in range(0, POS_INF + 1, chunk):
        end = min(start + chunk, POS_INF + 1)
        announce(f"cast_e4m3: patterns {start:#010x} .. {end - 1:#010x} and their negatives")
        u = torch.arange(start, end, dtype=torch.int32, device=dev())
        qp = _cast(u.view(torch.float32))
        qn = _cast(torch.bitwise_or(u, SIGN).view(torch.float32))
        assert torch.equal(qn, qp | 0x80), "a negative pattern is not the sign-flipped code"
        qi = qp.to(torch.int16)
        assert int(qi[0]) >= last and bool((qi[1:] >= qi[:-1]).all()), "codes decrease"
        assert int(qi.max()) <= 0x7E
        last = int(qi[-1])
        del u, qp, qn, qi
    assert last == 0x7E, "+inf must saturate to 448"


@pytest.mark.parametrize("n", [1, 7, 8, 13, 1000, 4099])
def test_cast_ragged_lengths_and_special_values(n):
    """Lengths with a tail (n % 8 != 0), random patterns of every exponent,
    zeros of both signs, subnormals, values at and past 448: each code equal
    to the oracle's, nothing written past n."""
    native_loaded()
    rng = np.random.default_rng(n)
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x43E00000, 0xC3E00000,
                        0x43E80000, 0x43F00000, 0x7F7FFFFF, 0xFF7FFFFF, 0x3B800000, 0x3B000000],
                       np.uint32)
    u[:min(n, special.size)] = special[:n]
    exp_bits = (u >> 23) & 0xFF
    u[exp_bits == 0xFF] &= 0x807FFFFF            # NaN and inf patterns -> finite ones
    x = u.view(np.float32)
    want = np.array([oracle.e4m3_encode(float(v)) for v in x], np.uint8)
    announce(f"cast_e4m3: {n} values")
    xd = torch.from_numpy(x.copy()).to(dev())
    q = torch.full((n + 32,), 0x5A, dtype=torch.uint8, device=dev())
    fp8bs.fp8bs_cast_e4m3(xd, q[:n])
    qh = host(q)
    assert (qh[n:] == 0x5A).all(), "wrote past n"
    assert np.array_equal(qh[:n], want), np.nonzero(qh[:n] != want)
