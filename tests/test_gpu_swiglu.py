"""GPU parity of fp8bs_swiglu_quant_1x128: h = silu(g) u of the cached BF16
gate and up halves ([p1] para 4, [p4] para 3), quantized in 1x128 tiles for
the down-projection ([p1] para 3), against oracle.swiglu_quant_1x128.

The kernel computes h in FP32 (exp, one reciprocal, two products), a few
units in the last place from the oracle's binary64 value rounded once, so:

- where h is exact on both sides (gates of 90 or more make sigma exactly 1
  in FP32 and in binary64 after rounding: h = g u), codes, scales and the
  BF16 h are bit-exact;
- elsewhere every scale is within 2^-19 of the oracle's, every BF16 h within
  one bf16 step of the oracle's, every code the oracle's or its neighbour
  where the oracle's quotient lies within 2^-17 of the midpoint between the
  two, and the share of codes or BF16 values that differ stays below 0.5%.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import announce, bf16_dev, dev, host, native_loaded

pytestmark = pytest.mark.gpu

TAB = oracle.e4m3_table()


def _run(g, u, codes=True, hout=True, pad=0):
    T, I = g.shape
    G = I // 128
    gd = torch.zeros((T, I + pad), dtype=torch.bfloat16, device=dev()); gd[:, :I] = bf16_dev(g)
    ud = torch.zeros((T, I + pad), dtype=torch.bfloat16, device=dev()); ud[:, :I] = bf16_dev(u)
    q = torch.full((T, I + pad), 0x5A, dtype=torch.uint8, device=dev()) if codes else None
    s = torch.full((T, G + pad // 16), -1.0, dtype=torch.float32, device=dev()) if codes else None
    h = torch.full((T, I + pad), 7.0, dtype=torch.bfloat16, device=dev()) if hout else None
    fp8bs.fp8bs_swiglu_quant_1x128(gd[:, :I], ud[:, :I], q[:, :I] if codes else None,
                                   s[:, :G] if codes else None, h[:, :I] if hout else None)
    out = {}
    if codes:
        qh, sh = host(q), host(s)
        if pad:
            assert (qh[:, I:] == 0x5A).all() and (sh[:, G:] == -1.0).all(), "wrote past a row"
        out["q"], out["s"] = qh[:, :I], sh[:, :G]
    if hout:
        hh = host(h)
        if pad:
            assert (hh[:, I:] == 0x40E0).all(), "wrote past an h row"
        out["h"] = hh[:, :I]
    return out


def _check(name, out, ref):
    q_ref, s_ref, h32, h16_ref = ref
    T, I = h32.shape
    if "s" in out:
        s, q = out["s"], out["q"]
        zero = s_ref == 0
        assert (s[zero] == 0).all(), f"{name}: zero tiles"
        rel = np.abs(s[~zero].astype(np.float64) / s_ref[~zero] - 1.0)
        assert rel.size == 0 or rel.max() <= 2.0 ** -19, f"{name}: scale off by {rel.max():.3g}"
        diff = q != q_ref
        share = diff.mean()
        if diff.any():
            # only neighbours, only near a midpoint of the oracle's quotient
            mq, mr = (q[diff] & 0x7F).astype(int), (q_ref[diff] & 0x7F).astype(int)
            assert (np.abs(mq - mr) == 1).all(), f"{name}: a code more than one step away"
            assert ((q[diff] >> 7) == (q_ref[diff] >> 7)).all(), f"{name}: sign"
            srow = np.repeat(s_ref, 128, axis=1)[diff].astype(np.float64)
            y = np.abs(h32[diff].astype(np.float64)) / srow
            mid = 0.5 * (TAB[np.minimum(mq, mr)] + TAB[np.maximum(mq, mr)])
            assert (np.abs(y - mid) <= mid * 2.0 ** -17).all(), f"{name}: a differing code away from a midpoint"
        assert share <= 0.005, f"{name}: {share:.2%} codes differ"
        announce(f"{name}: codes differing from the oracle {diff.sum()} ({share:.3%})")
    if "h" in out:
        h = out["h"].astype(np.int64)
        hr = h16_ref.astype(np.int64)

        def key(b):  # bf16 bits ordered like their values
            return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
        d = np.abs(key(h) - key(hr))
        assert d.max() <= 1, f"{name}: a BF16 h more than one step away"
        assert (d != 0).mean() <= 0.005, f"{name}: {(d != 0).mean():.2%} BF16 h differ"


def test_swiglu_exact_when_sigma_is_one():
    """Gates of 90 and more: e^-g is below half an ulp of 1 in both
    precisions, so h = g u exactly and everything is bit-exact."""
    native_loaded()
    rng = np.random.default_rng(3)
    g = synth.bf16_bits(rng.uniform(90.0, 300.0, (70, 512)).astype(np.float32))
    u = synth.bf16_bits((rng.standard_normal((70, 512)) * 10.0 ** rng.integers(-3, 3, (70, 1))).astype(np.float32))
    ref = oracle.swiglu_quant_1x128(g, u)
    announce("swiglu exact 70x512")
    out = _run(g, u, pad=16)
    assert (out["q"] == ref[0]).all() and (out["s"].view(np.uint32) == ref[1].view(np.uint32)).all()
    assert (out["h"] == ref[3]).all()


@pytest.mark.parametrize("T,I", [(1, 128), (300, 2048), (129, 640)])
def test_swiglu_general(T, I):
    native_loaded()
    rng = np.random.default_rng(T + I)
    g = synth.bf16_bits((rng.standard_normal((T, I)) * 2.0).astype(np.float32))
    u = synth.bf16_bits(rng.standard_normal((T, I)).astype(np.float32))
    ref = oracle.swiglu_quant_1x128(g, u)
    announce(f"swiglu {T}x{I}")
    _check(f"swiglu {T}x{I}", _run(g, u, pad=16), ref)
    # each output alone
    _check(f"swiglu {T}x{I} codes only", _run(g, u, hout=False), ref)
    _check(f"swiglu {T}x{I} h only", _run(g, u, codes=False), ref)


def test_swiglu_edge_gates():
    """Gates near zero (tiny h), strongly negative (h down to about 1e-24 of
    g u), large positive, zero rows and signed zeros."""
    native_loaded()
    rng = np.random.default_rng(9)
    T, I = 64, 384
    g = np.empty((T, I), np.float32)
    g[0:16] = rng.standard_normal((16, I)) * 1e-6
    g[16:32] = -rng.uniform(10.0, 55.0, (16, I))
    g[32:48] = rng.uniform(20.0, 80.0, (16, I))
    g[48:56] = 0.0
    g[56:64] = rng.standard_normal((8, I)) * 8.0
    u = rng.standard_normal((T, I)).astype(np.float32)
    u[52:56] = -0.0
    g16, u16 = synth.bf16_bits(g), synth.bf16_bits(u)
    ref = oracle.swiglu_quant_1x128(g16, u16)
    announce("swiglu edge gates 64x384")
    _check("swiglu edge gates", _run(g16, u16), ref)


def test_swiglu_moe_down_input():
    """The MoE down-projection's input at full size: 16384 tokens x 2048
    (the halves of the 16384 x 4096 up-projection output)."""
    native_loaded()
    rng = np.random.default_rng(4)
    T, I = 16384, 2048
    g = synth.bf16_bits((rng.standard_normal((T, I)) * 1.5).astype(np.float32))
    u = synth.bf16_bits(rng.standard_normal((T, I)).astype(np.float32))
    ref = oracle.swiglu_quant_1x128(g, u)
    announce("swiglu moe down input 16384x2048")
    _check("swiglu 16384x2048", _run(g, u), ref)
