"""Pins of the oracle's quantizers (1x128 activation tiles, 128x128 weight
blocks, backward 1x128 -> 128x1 re-quantization) against hand-worked cases,
exact-rational brute force, closed forms and invariants."""
import json
import os

import numpy as np
import pytest

import oracle
from fp8_fine_grained_fp8bs_amd import synth
from tests.exact_ref import (e4m3_dec_f32, quantize_group_exact,
                             torch_e4m3_table)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TAB = torch_e4m3_table()


def _bf16(a):
    return synth.bf16_bits(np.asarray(a, dtype=np.float32))


def test_quant_act_hand_cases():
    cases = json.load(open(os.path.join(GOLDEN, "quant_hand.json")))["cases"]
    for case in cases:
        row = np.full(128, case["fill"], dtype=np.float32)
        row[: len(case["x"])] = np.array(case["x"], dtype=np.float32)
        q, s = oracle.quant_act_1x128(_bf16(row[None, :]))
        assert s[0, 0] == np.float32(case["scale"]), case["note"]
        assert list(q[0, : len(case["codes"])]) == case["codes"], case["note"]


def _crafted_rows(rng, rows, K):
    """Rows whose values sit on, and one bf16 step beside, E4M3 rounding
    midpoints of their own tile scale, plus plain normal draws."""
    x = rng.standard_normal((rows, K)).astype(np.float32)
    for r in range(rows):
        for g in range(K // 128):
            amax = np.float32(2.0 ** rng.integers(-20, 20))
            s = amax / np.float32(448.0)
            seg = x[r, g * 128:(g + 1) * 128]
            seg[0] = amax
            mids = 0.5 * (TAB[rng.integers(0, 126, 40)] + TAB[rng.integers(0, 126, 40)])
            seg[1:41] = (mids * float(s)).astype(np.float32)
            seg[41:] *= amax / np.float32(4.0)
    return _bf16(np.clip(x, -3e38, 3e38))


def test_quant_act_exact_bruteforce_tiny_and_crafted():
    data = synth.tiny(M=6, N=1, K=512)
    rng = np.random.default_rng(11)
    x = np.concatenate([data["A"], _crafted_rows(rng, 6, 512)])
    q, s = oracle.quant_act_1x128(x)
    xf = synth.bf16_to_f32(x)
    for r in range(x.shape[0]):
        for g in range(4):
            cq, cs = quantize_group_exact(xf[r, g * 128:(g + 1) * 128])
            assert s[r, g] == cs
            assert np.array_equal(q[r, g * 128:(g + 1) * 128], cq), (r, g)


def test_quant_act_subnormal_scale_and_zero_tiles():
    rng = np.random.default_rng(3)
    rows = []
    # amax spanning bf16 subnormals up to the FP32-subnormal-scale boundary
    for e in [-133, -131, -128, -126, -124, -120, -118, -117, -116, -110]:
        r = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** e)
        rows.append(r)
    rows.append(np.zeros(128, np.float32))
    z = np.zeros(128, np.float32); z[::2] = -0.0
    rows.append(z)
    x = _bf16(np.stack(rows))
    q, s = oracle.quant_act_1x128(x)
    xf = synth.bf16_to_f32(x)
    for r in range(x.shape[0]):
        cq, cs = quantize_group_exact(xf[r])
        assert s[r, 0] == cs and np.array_equal(q[r], cq), r
    assert s[-1, 0] == 0 and s[-2, 0] == 0
    assert np.array_equal(q[-1], np.where(np.signbit(xf[-1]), 0x80, 0).astype(np.uint8))


def test_quant_roundtrip_exact_codes():
    """x = dec(c) * s0 with s0 of <= 4 significant bits and a +-448 code in
    each tile: the codes come back unchanged and the scale is s0."""
    rng = np.random.default_rng(1)
    M, K = 16, 512
    codes = rng.integers(0, 256, (M, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes
    codes[:, ::128] = 0x7E                        # one 448 per tile
    s0 = np.array([m * 2.0 ** e for m, e in zip(rng.choice([8, 9, 11, 13, 15], (M, 4)).ravel(),
                                                 rng.integers(-20, 10, M * 4))], dtype=np.float32).reshape(M, 4)
    vals = e4m3_dec_f32(codes).astype(np.float64) * np.repeat(s0, 128, axis=1)
    x = _bf16(vals)
    assert np.array_equal(synth.bf16_to_f32(x).astype(np.float64), vals)  # exact in bf16
    q, s = oracle.quant_act_1x128(x)
    assert np.array_equal(s, s0)
    assert np.array_equal(q, codes)


def test_quant_power_of_two_invariance():
    x = synth.tiny(M=32, N=1, K=512)["A"]
    q0, s0 = oracle.quant_act_1x128(x)
    xf = synth.bf16_to_f32(x)
    for k in (-40, -3, 1, 7, 60):
        xk = _bf16(xf * np.float32(2.0 ** k))
        assert np.array_equal(synth.bf16_to_f32(xk), xf * np.float32(2.0 ** k))
        qk, sk = oracle.quant_act_1x128(xk)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk, s0 * np.float32(2.0 ** k))


def _check_error_bound_and_448(x_f32, q, s, groups):
    """|x - s*dec(q)| <= half an E4M3 ulp of x/s, times s, for every element
    of a tile with a normal scale; each such non-zero tile holds +-448."""
    for idx, sc in groups:
        if sc == 0 or sc < np.float32(2.0 ** -126):
            continue
        xv = x_f32[idx].astype(np.float64).ravel()
        dq = TAB[q[idx].ravel()]
        y = np.abs(xv / float(sc))
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        ulp = 2.0 ** (e - 3)
        assert np.all(np.abs(xv - float(sc) * dq) <= 0.5 * ulp * float(sc) * (1 + 1e-12))
        assert np.any((q[idx] & 0x7F) == 0x7E)


def test_quant_act_error_bound_and_full_range_code():
    d = synth.mlp_up(T=64, K=1024, with_w=False)
    x = d["X"]
    q, s = oracle.quant_act_1x128(x)
    xf = synth.bf16_to_f32(x)
    groups = [((r, slice(g * 128, (g + 1) * 128)), s[r, g]) for r in range(64) for g in range(8)]
    _check_error_bound_and_448(xf, q, s, groups)


def test_quant_w_bruteforce_ragged_and_bounds():
    w = synth.tiny(M=1, N=200, K=256)["W"]             # 200 rows: one partial block
    q, s = oracle.quant_w_128x128(w)
    assert s.shape == (2, 2)
    wf = synth.bf16_to_f32(w)
    for nb in range(2):
        for g in range(2):
            blk = wf[nb * 128:min(200, nb * 128 + 128), g * 128:(g + 1) * 128]
            cq, cs = quantize_group_exact(blk)
            assert s[nb, g] == cs
            assert np.array_equal(q[nb * 128:min(200, nb * 128 + 128), g * 128:(g + 1) * 128].ravel(), cq)
    groups = [((slice(nb * 128, min(200, nb * 128 + 128)), slice(g * 128, (g + 1) * 128)), s[nb, g])
              for nb in range(2) for g in range(2)]
    _check_error_bound_and_448(wf, q, s, groups)


def test_quant_w_transpose_invariance():
    w = synth.mlp_up(T=384, K=256, with_w=False)["X"]     # 384 x 256, heavy channels
    q, s = oracle.quant_w_128x128(w)
    qt, st = oracle.quant_w_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(qt, q.T)
    assert np.array_equal(st, s.T)


def test_transpose_w_equals_quantization_of_transposed_weight():
    """The quantized W^T of the input-gradient pass is the quantization of
    the bf16 W^T: transposing the codes and the scale grid must give the
    same bits as quantizing W^T block by block."""
    w = synth.wgrad(T=256, C_in=384, C_out=256, with_w=True)["W"]       # [256][384]
    rng = np.random.default_rng(11)
    w = w.copy()
    w[rng.random(w.shape) < 0.01] ^= 0x0100       # perturb exponents: varied block max-abs
    q, s = oracle.quant_w_128x128(w)
    qt, st = oracle.transpose_w_128x128(q, s)
    q2, s2 = oracle.quant_w_128x128(np.ascontiguousarray(w.T))
    assert qt.shape == (384, 256) and st.shape == (3, 2)
    assert np.array_equal(qt, q2) and np.array_equal(st.view(np.uint32), s2.view(np.uint32))
    # and it is an involution
    q3, s3 = oracle.transpose_w_128x128(qt, st)
    assert np.array_equal(q3, q) and np.array_equal(s3, s)


def test_quant_per_tensor_is_one_group_over_the_tensor():
    """Per-tensor scaling is the tile quantization with the whole tensor as
    one group: brute force over every value, and equal to quant_act_1x128
    when the tensor is a single 1x128 row."""
    x = synth.tiny(M=64, N=128, K=256)["A"]                  # with x50 outliers
    q, s = oracle.quant_per_tensor(x)
    cq, cs = quantize_group_exact(synth.bf16_to_f32(x).ravel())
    assert s == cs and np.array_equal(q.ravel(), cq)
    row = x[:1, :128]
    q1, s1 = oracle.quant_per_tensor(np.ascontiguousarray(row))
    qa, sa = oracle.quant_act_1x128(np.ascontiguousarray(row))
    assert s1 == sa[0, 0] and np.array_equal(q1, qa)


def test_requant_fp8_composition_bruteforce():
    """requant_T(q, s1) equals the exact 128-token quantization of the FP32
    dequantized values fl32(dec(q) * s1), transposed; ragged T."""
    T, C = 200, 256
    x = synth.wgrad(T=T, C_in=C, C_out=128)["X"]
    q1, s1 = oracle.quant_act_1x128(x)
    q2, s2 = oracle.requant_T_128x1_fp8(q1, s1)
    assert q2.shape == (C, T) and s2.shape == (C, 2)
    v = e4m3_dec_f32(q1) * np.repeat(s1, 128, axis=1)     # numpy float32 multiply
    for c in range(0, C, 7):
        for tg in range(2):
            seg = v[tg * 128:min(T, tg * 128 + 128), c]
            cq, cs = quantize_group_exact(seg)
            assert s2[c, tg] == cs
            assert np.array_equal(q2[c, tg * 128:min(T, tg * 128 + 128)], cq), (c, tg)
    # the same identity through the oracle's FP32-input quantizer (T = 128k)
    qa, sa = oracle.quant_act_1x128_f32(np.ascontiguousarray(v[:128].T))
    assert np.array_equal(qa, q2[:, :128]) and np.array_equal(sa[:, 0], s2[:, 0])


def test_requant_bf16_source_bruteforce():
    T, C = 130, 128
    dy = synth.wgrad(T=T, C_in=128, C_out=C)["dY"]
    q2, s2 = oracle.requant_T_128x1_bf16(dy)
    df = synth.bf16_to_f32(dy)
    for c in range(0, C, 5):
        for tg in range(2):
            seg = df[tg * 128:min(T, tg * 128 + 128), c]
            cq, cs = quantize_group_exact(seg)
            assert s2[c, tg] == cs
            assert np.array_equal(q2[c, tg * 128:min(T, tg * 128 + 128)], cq)
