"""Seeded synthetic inputs shared by the GPU path and the CPU oracle.

This module only draws random numbers and rounds them to bf16 bit patterns;
it holds none of the quantization or GEMM arithmetic.  Every array it returns
is a numpy ``uint16`` bf16 bit pattern (or an int32 offsets vector), so the
GPU library and the oracle consume exactly the same bits.

Recipe (one generator, ``numpy.random.default_rng(seed)``, seed 0 by
default; draws happen in the order written below):

* float32 draws are rounded to bf16 by round-to-nearest-even on the bit
  pattern (``bf16_bits``); wider draws are first rounded to float32.
* ``tiny``      A [M][K] N(0,1) with an iid 1 % mask of entries multiplied by
                50 (outliers; the factor is a parameter for the accuracy
                study); W [N][K] N(0, 0.02).  Default 128x512, 256x512.
* ``probe``     A, W [R][K] U(-1,1), each row multiplied by 10^u, u ~ U(-2,2).
                Default M=N=1024, K=4096.
* ``mlp_up``    X [T][K] N(0,1) except a seeded 1 % of the K channels drawn
                from Student-t(3); W [N][K] N(0, 0.006).  Default 4096 tokens,
                K=7168, N=18432.
* ``moe``       8 experts; token counts from Zipf(1.1) expected shares (largest
                remainder rounding to the total); A_up [T][7168] N(0,1),
                W_up [E][4096][7168] N(0,0.01), A_down [T][2048] N(0,1),
                W_down [E][7168][2048] N(0,0.01).  Default T=16384.
* ``wgrad``     X [T][7168] and dY [T][2048] N(0, 0.01), then (only when
                asked for) the layer weight W [2048][7168] N(0, 0.01) for the
                input gradient dX = dY W.  Default T=8192.

Sizes are parameters so tests can draw the same distributions at sizes the
oracle finishes in seconds.
"""
from __future__ import annotations

import numpy as np


def bf16_bits(a) -> np.ndarray:
    """float32 (or wider, rounded to float32 first) -> bf16 bit patterns by
    round-to-nearest-even on the float32 bits.  Inputs must be finite."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def tiny(M=128, N=256, K=512, seed=0, outlier=50.0):
    """A with 1 % outliers (x50 by default), W ~ N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    a = _normal(rng, (M, K))
    mask = rng.random((M, K)) < 0.01
    a[mask] *= np.float32(outlier)
    w = _normal(rng, (N, K), 0.02)
    return {"A": bf16_bits(a), "W": bf16_bits(w)}


def probe(M=1024, N=1024, K=4096, seed=0):
    """U(-1,1) rows scaled by 10^U(-2,2)."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(-1.0, 1.0, (M, K)) * (10.0 ** rng.uniform(-2.0, 2.0, (M, 1)))
    w = rng.uniform(-1.0, 1.0, (N, K)) * (10.0 ** rng.uniform(-2.0, 2.0, (N, 1)))
    return {"A": bf16_bits(a), "W": bf16_bits(w)}


def heavy_channels(K, seed=0, frac=0.01):
    """Indices of the Student-t channels of ``mlp_up`` (sorted)."""
    rng = np.random.default_rng(seed + 1000)
    n = max(1, int(round(frac * K)))
    return np.sort(rng.choice(K, size=n, replace=False))


def mlp_up(T=4096, K=7168, N=18432, seed=0, with_w=True):
    """Dense MLP up-projection: heavy-tailed activation channels."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, K))
    ch = heavy_channels(K, seed)
    x[:, ch] = rng.standard_t(3.0, (T, ch.size)).astype(np.float32)
    out = {"X": bf16_bits(x)}
    del x
    if with_w:
        out["W"] = bf16_bits(_normal(rng, (N, K), 0.006))
    return out


def zipf_counts(total=16384, experts=8, s=1.1) -> np.ndarray:
    """Deterministic Zipf(s) token counts over experts, summing to total."""
    p = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    raw = p * total
    c = np.floor(raw).astype(np.int64)
    rem = total - int(c.sum())
    order = np.argsort(-(raw - c), kind="stable")
    c[order[:rem]] += 1
    return c


def offsets_from_counts(counts) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def moe(T=16384, E=8, K_up=7168, N_up=4096, K_down=2048, N_down=7168, seed=0,
        parts=("A_up", "W_up", "A_down", "W_down")):
    """One GPU's share of MoE experts with ragged Zipf token counts."""
    rng = np.random.default_rng(seed)
    counts = zipf_counts(T, E)
    out = {"counts": counts, "offsets": offsets_from_counts(counts)}
    shapes = {"A_up": ((T, K_up), 1.0), "W_up": ((E, N_up, K_up), 0.01),
              "A_down": ((T, K_down), 1.0), "W_down": ((E, N_down, K_down), 0.01)}
    for name in ("A_up", "W_up", "A_down", "W_down"):
        shape, std = shapes[name]
        x = _normal(rng, shape, std)
        if name in parts:
            out[name] = bf16_bits(x)
        del x
    return out


def wgrad(T=8192, C_in=7168, C_out=2048, seed=0, with_w=False):
    """Backward inputs of one Linear layer: X [T][C_in], dY [T][C_out], and
    (with_w) the layer's weight W [C_out][C_in] for the input gradient."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (T, C_in), 0.01)
    dy = _normal(rng, (T, C_out), 0.01)
    out = {"X": bf16_bits(x), "dY": bf16_bits(dy)}
    if with_w:
        out["W"] = bf16_bits(_normal(rng, (C_out, C_in), 0.01))
    return out
