"""Shared helpers of the GPU parity tests: device transfer, the GEMM
comparison rules, and cached synthetic inputs with their oracle results.

Comparison rules (from the acceptance bar of the method):
* quantized codes and scales: bit-exact;
* FP32 GEMM outputs: relative Frobenius error <= 1e-4 and, per entry,
  |err| <= 1e-3 * sum_k |a_k||b_k|, against the binary64 oracle;
* BF16 GEMM outputs, two rules:
  - bitwise equal to the same kernel's FP32 result rounded once to
    nearest-even (that FP32 result meeting the bounds above);
  - against the oracle: within half a bf16 step plus the GEMM allowance
    1e-3 * sum|a||b| everywhere; where that allowance is below one bf16
    step of the oracle value, an entry differing from the oracle rounded to
    bf16 is one bf16 step away with a bf16 rounding midpoint between the
    oracle value and the kernel's FP32 value, within the allowance of the
    oracle value; the share of differing entries stays below a bound.
  The gfx950 FP8 matrix instruction drops the bits of each product that lie
  more than 13 binary orders below the largest product of its 8-product
  chunk (tests/test_gpu_mfma_chunks.py measures this), so the FP32 result
  sits a little off the binary64 value and can land on the other side of a
  bf16 midpoint; the rules bound where and how often that may happen.

Accuracy records: with FP8BS_ACCURACY_JSON set, every GEMM comparison
appends one JSON line (configuration, error figures, flip share) to that
file.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(a_u16: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16)
    return t.to(dev())


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def abs_codes(q: np.ndarray) -> np.ndarray:
    return (q & 0x7F).astype(np.uint8)


def check_quant_equal(name, q_gpu, s_gpu, q_ref, s_ref):
    assert q_gpu.shape == q_ref.shape and s_gpu.shape == s_ref.shape, name
    bad_s = np.flatnonzero(s_gpu.view(np.uint32) != s_ref.view(np.uint32))
    assert bad_s.size == 0, f"{name}: {bad_s.size} scale mismatches, first at {np.unravel_index(bad_s[0], s_ref.shape)}: gpu {s_gpu.flat[bad_s[0]]!r} ref {s_ref.flat[bad_s[0]]!r}"
    bad_q = np.flatnonzero(q_gpu != q_ref)
    assert bad_q.size == 0, f"{name}: {bad_q.size} code mismatches, first at {np.unravel_index(bad_q[0], q_ref.shape)}: gpu {q_gpu.flat[bad_q[0]]:#04x} ref {q_ref.flat[bad_q[0]]:#04x}"


def check_f32_gemm(name, d_gpu, d_ref, mag):
    """d_gpu float32, d_ref binary64 oracle, mag = sum |a||b| per entry."""
    err = d_gpu.astype(np.float64) - d_ref
    fro = np.linalg.norm(err) / max(np.linalg.norm(d_ref), 1e-300)
    assert fro <= 1e-4, f"{name}: relative Frobenius {fro:.3e}"
    ratio = np.abs(err) / np.maximum(mag, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1e-3, f"{name}: max |err| / sum|a||b| = {worst:.3e}"
    return fro, worst


def bf16_val(u16: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(u16).astype(np.float64)


def check_bf16_is_rounded_f32(name, d_bf16_u16, d_f32):
    """The BF16 output must be the kernel's FP32 result rounded once to
    nearest-even (checked with the oracle's independent bf16 rounding)."""
    ref = oracle.round_to_bf16(np.asarray(d_f32, dtype=np.float64))
    bad = np.flatnonzero(d_bf16_u16.ravel() != ref.ravel())
    assert bad.size == 0, (f"{name}: {bad.size} bf16 outputs differ from RNE(fp32 result); "
                           f"first idx {bad[0]}: {d_bf16_u16.ravel()[bad[0]]:#06x} vs {ref.ravel()[bad[0]]:#06x}")


def record(kind, name, **fields):
    """Append one accuracy record (JSON line) if FP8BS_ACCURACY_JSON is set."""
    path = os.environ.get("FP8BS_ACCURACY_JSON")
    if not path:
        return
    rec = {"kind": kind, "name": name}
    rec.update({k: (float(v) if isinstance(v, (np.floating, float)) else v) for k, v in fields.items()})
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (2^-133 at zero and for subnormals)."""
    _, e = np.frexp(np.abs(np.asarray(v, np.float64)))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def check_bf16_vs_oracle(name, d_bf16_u16, d_f32, d_ref, mag, max_flip_share):
    """BF16 output against the binary64 oracle.

    * every entry: |bf16 - oracle| <= half a bf16 step of the output plus the
      GEMM allowance 1e-3 * sum|a||b|;
    * an entry that differs from the oracle rounded to bf16, where that
      allowance is smaller than one bf16 step of the oracle value (no heavy
      cancellation): exactly one bf16 step away, with the bf16 midpoint
      between the two lying between the oracle value and the kernel's FP32
      value (inclusive) and within the allowance of the oracle value;
    * the share of differing entries at most max_flip_share.
    Returns (flips, share, multi_step) where multi_step counts differing
    entries more than one step away (cancellation entries only)."""
    d16 = np.asarray(d_bf16_u16, np.uint16).ravel()
    f32 = np.asarray(d_f32, np.float64).ravel()
    ref = np.asarray(d_ref, np.float64).ravel()
    mag = np.broadcast_to(np.asarray(mag, np.float64), np.shape(d_ref)).ravel()
    allow = 1e-3 * mag
    dv = bf16_val(d16)
    far = np.flatnonzero(np.abs(dv - ref) > 0.5 * bf16_ulp(dv) + allow)
    assert far.size == 0, (f"{name}: bf16 output {dv[far[0]]!r} farther than half a bf16 step plus "
                           f"1e-3 sum|a||b| from the oracle {ref[far[0]]!r} at flat index {far[0]}")
    ref16 = oracle.round_to_bf16(ref).ravel()
    bad = np.flatnonzero(d16 != ref16)
    multi = 0
    if bad.size:
        def key(u):  # bf16 values ordered like their sign-magnitude bit patterns
            u = u.astype(np.int64)
            return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
        steps = np.abs(key(d16[bad]) - key(ref16[bad]))
        plain = allow[bad] < bf16_ulp(ref[bad])
        multi = int((steps > 1).sum())
        i0 = np.flatnonzero(plain & (steps > 1))
        assert i0.size == 0, (f"{name}: bf16 output {d16[bad[i0[0]]]:#06x} is {steps[i0[0]]} steps from the "
                              f"rounded oracle {ref16[bad[i0[0]]]:#06x} at flat index {bad[i0[0]]}")
        one = np.flatnonzero(steps == 1)
        g, r = bf16_val(d16[bad[one]]), bf16_val(ref16[bad[one]])
        mid = 0.5 * (g + r)
        fb, rb, ab = f32[bad[one]], ref[bad[one]], allow[bad[one]]
        between = ((rb <= mid) & (mid <= fb)) | ((fb <= mid) & (mid <= rb))
        i1 = np.flatnonzero(~between)
        assert i1.size == 0, (f"{name}: no bf16 midpoint between oracle {rb[i1[0]]!r} and the kernel's "
                              f"FP32 value {fb[i1[0]]!r} at flat index {bad[one[i1[0]]]}")
        i2 = np.flatnonzero(np.abs(rb - mid) > ab)
        assert i2.size == 0, f"{name}: bf16 midpoint farther than 1e-3 sum|a||b| from the oracle at {bad[one[i2[0]]]}"
    share = bad.size / max(d16.size, 1)
    assert share <= max_flip_share, (f"{name}: {bad.size} of {d16.size} bf16 outputs ({share:.2%}) differ "
                                     f"from the rounded oracle, bound {max_flip_share:.2%}")
    return int(bad.size), share, multi


def bf16_flips(d_bf16_u16, d_ref):
    """Entries whose bf16 output differs from the oracle rounded to bf16."""
    return int((d_bf16_u16.ravel() != oracle.round_to_bf16(d_ref).ravel()).sum())


def gemm_mag(qa, sa, qb, sb, bmode=oracle.BSCALE_BLOCK, mi=None, ni=None):
    """sum_k |a_k||b_k| per output entry (from the oracle on |codes|, |scales|)."""
    aa, ab = abs_codes(qa), abs_codes(qb)
    if mi is None:
        return oracle.gemm(aa, np.abs(sa), ab, np.abs(sb), bmode)
    return oracle.gemm_entries(aa, np.abs(sa), ab, np.abs(sb), mi, ni, bmode)


def native_loaded():
    """The HIP library is the code under test: fail loudly if absent."""
    lib = fp8bs.load()
    assert lib.fp8bs_version() >= 100
    return lib


def sample_idx(M, N, n=3000, seed=0):
    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, M, n), [0, M - 1, 0, M - 1], np.full(64, M // 2)])
    ni = np.concatenate([rng.integers(0, N, n), [0, 0, N - 1, N - 1], np.arange(64) * (N // 64)])
    return mi, ni


# Bound on the share of bf16 outputs that differ from the rounded oracle
# (each one a single bf16 step at a midpoint, see check_bf16_vs_oracle),
# unless a test states its own; measured shares are in the accuracy records.
DEFAULT_FLIP_SHARE = 0.05


def check_gemm_outputs(name, d32, d16, ref, mag, mi=None, ni=None, max_flip_share=DEFAULT_FLIP_SHARE):
    """Every rule of the GEMM comparison on host arrays: d32 (FP32 output,
    full), d16 (BF16 output of the same inputs, full, or None), ref and mag
    the oracle value and sum|a||b| on all entries or on the sampled entries
    (mi, ni).  Announces and records the figures."""
    s32 = d32 if mi is None else d32[mi, ni]
    fro, worst = check_f32_gemm(name + " f32", s32, ref, mag)
    err = np.abs(s32.astype(np.float64) - ref)
    rel_max = float(err.max() / max(np.abs(ref).max(), 1e-300)) if ref.size else 0.0
    fields = dict(entries=int(np.size(ref)), sampled=mi is not None, rel_fro=fro,
                  max_err_over_sum_ab=worst, max_err_over_max_ref=rel_max)
    msg = f"{name}: f32 rel-fro {fro:.2e} max-err/sum|ab| {worst:.2e} max-err/max|ref| {rel_max:.2e}"
    if d16 is not None:
        check_bf16_is_rounded_f32(name + " bf16", d16, d32)
        s16 = d16 if mi is None else d16[mi, ni]
        flips, share, multi = check_bf16_vs_oracle(name + " bf16", s16, s32, ref, mag, max_flip_share)
        fields.update(bf16_flips=flips, bf16_flip_share=share, bf16_flip_bound=max_flip_share,
                      bf16_multi_step=multi)
        msg += (f"; bf16 == RNE(f32) on all {d16.size}, vs rounded oracle {flips} flips ({share:.2%}, "
                f"bound {max_flip_share:.0%}; {multi} of them more than one step, in cancellation entries)")
    record("gemm", name, **fields)
    announce(msg)
    return fro, worst


def sampled_check(name, qa, sa, qb, sb, d32_dev, d16_dev=None, bmode=oracle.BSCALE_BLOCK,
                  max_flip_share=DEFAULT_FLIP_SHARE):
    """FP32 result on sampled entries vs the oracle; the BF16 result (if
    given) on every entry vs the rounded FP32 result and on the sampled
    entries vs the rounded oracle."""
    M, N = qa.shape[0], qb.shape[0]
    mi, ni = sample_idx(M, N)
    ref = oracle.gemm_entries(qa, sa, qb, sb, mi, ni, bmode)
    mag = gemm_mag(qa, sa, qb, sb, bmode, mi, ni)
    d32 = host(d32_dev)
    d16 = host(d16_dev) if d16_dev is not None else None
    return check_gemm_outputs(name, d32, d16, ref, mag, mi, ni, max_flip_share)
