"""Shared helpers of the GPU parity tests: device transfer, the GEMM
comparison rules, and cached synthetic inputs with their oracle results.

Comparison rules (from the acceptance bar of the method):
* quantized codes and scales: bit-exact;
* FP32 GEMM outputs: relative Frobenius error <= 1e-4 and, per entry,
  |err| <= 1e-3 * sum_k |a_k||b_k|, against the binary64 oracle;
* BF16 GEMM outputs: bitwise equal to the same kernel's FP32 result rounded
  once to nearest-even, that FP32 result meeting the bounds above.  (The
  gfx950 FP8 matrix instruction truncates small products inside each
  8-product chunk, so the FP32 result differs from the binary64 value by up
  to ~1e-4 of sum|a||b| on outlier data and a bf16 rounding of it cannot be
  required to match the rounded oracle bit for bit; the number of such
  flips is reported.)
"""
from __future__ import annotations

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


def bf16_flips(d_bf16_u16, d_ref):
    """Entries whose bf16 output differs from the oracle rounded to bf16
    (reported, not bounded: the FP32 result may sit on either side of a
    bf16 rounding midpoint)."""
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


def sampled_check(name, qa, sa, qb, sb, d32_dev, d16_dev=None, bmode=oracle.BSCALE_BLOCK):
    """FP32 result on sampled entries vs the oracle; the BF16 result (if
    given) on every entry vs the rounded FP32 result."""
    M, N = qa.shape[0], qb.shape[0]
    mi, ni = sample_idx(M, N)
    ref = oracle.gemm_entries(qa, sa, qb, sb, mi, ni, bmode)
    mag = gemm_mag(qa, sa, qb, sb, bmode, mi, ni)
    d32 = host(d32_dev)
    fro, worst = check_f32_gemm(name, d32[mi, ni], ref, mag)
    msg = f"{name}: sampled f32 rel-fro {fro:.2e} max-err/sum|ab| {worst:.2e}"
    if d16_dev is not None:
        d16 = host(d16_dev)
        check_bf16_is_rounded_f32(name, d16, d32)
        msg += f"; bf16 == RNE(f32) on all {d16.size}; sampled flips vs rounded oracle {bf16_flips(d16[mi, ni], ref)}"
    announce(msg)
