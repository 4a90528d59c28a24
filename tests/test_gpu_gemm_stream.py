"""GPU parity of the GEMM's tile stream, tile orders and tile shapes: a
persistent workgroup with more than one tile copies its next tile's first
scale block and K groups during the current tile's last K groups (when the
K-group count G is a multiple of 4 and at least 8), so the stages, scale
slots and fragment sets of every later tile run at a phase of 0, 4 or 8
groups.  Small block-scale problems take 128x128 tiles instead of 128x256.

With at most 256 tiles every workgroup runs one tile and no stream is
involved; each output element goes through the same operations in the
same order either way.  So the output of a launch with several tiles per
workgroup must equal, bit for bit, the outputs of launches over row slices
of at most 256 tiles each: BF16 and FP32 outputs, both B-scale modes and
the grouped form, at G values that give every phase, and the quantized
output (which does not stream); the full outputs are also checked against
the oracle on sampled entries.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs
from tests.gpu_common import announce, dev, host, native_loaded, sampled_check

pytestmark = pytest.mark.gpu


def _codes(rng, shape):
    q = rng.integers(0, 256, shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38   # no NaN codes
    return q


def _operands(M, N, K, seed, row_scales=False):
    rng = np.random.default_rng(seed)
    G = K // 128
    qa = _codes(rng, (M, K))
    qb = _codes(rng, (N, K))
    sa = rng.uniform(0.5, 1.5, (M, G)).astype(np.float32)
    sb = rng.uniform(0.5, 1.5, (N if row_scales else -(-N // 128), G)).astype(np.float32)
    return qa, sa, qb, sb


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def _bits(t):
    h = host(t)
    return h.view(np.uint32) if h.dtype == np.float32 else h


def _run(a, sa, b, sb, bmode, form):
    if form == "fp8":
        q, s = fp8bs.gemm_quant_1x128(a, sa, b, sb, bmode)
        return [q, s]
    return [fp8bs.gemm(a, sa, b, sb, bmode, out_f32=(form == "f32"))]


def _slices_equal(name, qa, sa, qb, sb, bmode, form, bm):
    """Full launch against launches over row slices of <= 256 tiles."""
    M, N = qa.shape[0], qb.shape[0]
    bn = 256 if bmode == fp8bs.BSCALE_BLOCK_128x128 else 128
    tiles_n = -(-N // bn)
    rows = (256 // tiles_n) * bm
    assert -(-M // bm) * tiles_n > 256 and rows > 0, "the full launch must walk several tiles per workgroup"
    a, sa_d, b, sb_d = _dev(qa), _dev(sa), _dev(qb), _dev(sb)
    full = _run(a, sa_d, b, sb_d, bmode, form)
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        part = _run(a[r0:r1], sa_d[r0:r1], b, sb_d, bmode, form)
        for f, p in zip(full, part):
            fb, pb = _bits(f[r0:r1]), _bits(p)
            bad = np.flatnonzero(fb != pb)
            assert bad.size == 0, (f"{name}: rows {r0}..{r1}: {bad.size} entries differ from the "
                                   f"single-tile launch, first at {np.unravel_index(bad[0], pb.shape)}")
    return full


# K groups: streamed at phases 0/8/4 (8), 0/4/8 (16, 20, 28), always 0 (12,
# 24), the headline K (56); 9 and 10 take the head path on every tile.
@pytest.mark.parametrize("G", [8, 12, 16, 20, 24, 28, 56, 9, 10])
def test_stream_block_scales_bf16_and_f32(G):
    native_loaded()
    M, N, K = 128 * 40 - 37, 256 * 20 - 96, 128 * G    # 800 tiles, up to 4 per workgroup, ragged
    qa, sa, qb, sb = _operands(M, N, K, seed=G)
    announce(f"stream block scales G={G} {M}x{N}x{K}")
    d16 = _slices_equal(f"stream bf16 G={G}", qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, "bf16", 128)[0]
    d32 = _slices_equal(f"stream f32 G={G}", qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, "f32", 128)[0]
    sampled_check(f"stream G={G}", qa, sa, qb, sb, d32, d16)


@pytest.mark.parametrize("G", [8, 16, 20])
def test_stream_row_scales_f32(G):
    """The weight-gradient form: B scales per row, 128 x 128 tiles."""
    native_loaded()
    M, N, K = 128 * 30 - 5, 128 * 20 - 64, 128 * G     # 600 tiles
    qa, sa, qb, sb = _operands(M, N, K, seed=100 + G, row_scales=True)
    announce(f"stream row scales G={G} {M}x{N}x{K}")
    d32 = _slices_equal(f"stream row G={G}", qa, sa, qb, sb, fp8bs.BSCALE_ROW_1x128, "f32", 128)[0]
    sampled_check(f"stream row G={G}", qa, sa, qb, sb, d32, bmode=oracle.BSCALE_ROW)


@pytest.mark.parametrize("G", [8, 16])
def test_stream_quantized_output(G):
    """Output quantized 1x128 in the epilogue: codes and scales.  This form
    keeps the head copies on every tile (no stream); several tiles per
    workgroup must still match single-tile launches."""
    native_loaded()
    M, N, K = 128 * 40 - 3, 256 * 20, 128 * G
    qa, sa, qb, sb = _operands(M, N, K, seed=200 + G)
    announce(f"stream quantized output G={G} {M}x{N}x{K}")
    _slices_equal(f"stream fp8 G={G}", qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, "fp8", 128)


@pytest.mark.parametrize("G", [8, 16, 56])
def test_stream_grouped(G):
    """The grouped form with empty, single-row and ragged experts, more
    than 256 tiles: equal to one launch per expert (each under 256 tiles)."""
    native_loaded()
    counts = np.array([700, 0, 513, 1, 900, 380, 0, 611])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    E, N, K, T = len(counts), 4096, 128 * G, int(counts.sum())
    rng = np.random.default_rng(300 + G)
    qa = _codes(rng, (T, K))
    sa = rng.uniform(0.5, 1.5, (T, G)).astype(np.float32)
    qb = _codes(rng, (E, N, K))
    sb = rng.uniform(0.5, 1.5, (E, N // 128, G)).astype(np.float32)
    assert sum(-(-c // 128) for c in counts) * (N // 256) > 256
    announce(f"stream grouped G={G} T={T}")
    a, sa_d, b, sb_d = _dev(qa), _dev(sa), _dev(qb), _dev(sb)
    for out_f32 in (False, True):
        full = fp8bs.grouped_gemm(a, sa_d, b, sb_d, _dev(off), out_f32=out_f32)
        for e in range(E):
            r0, r1 = int(off[e]), int(off[e + 1])
            if r1 == r0:
                continue
            part = fp8bs.gemm(a[r0:r1], sa_d[r0:r1], b[e], sb_d[e], fp8bs.BSCALE_BLOCK_128x128, out_f32=out_f32)
            fb, pb = _bits(full[r0:r1]), _bits(part)
            assert (fb == pb).all(), f"grouped G={G} expert {e}: {(fb != pb).sum()} entries differ"
    mi = np.concatenate([rng.integers(0, T, 1500), off[1:][counts > 0] - 1, off[:-1][counts > 0]])
    ni = rng.integers(0, N, mi.size)
    ref = oracle.grouped_gemm_entries(qa, sa, qb, sb, off, mi, ni)
    got = host(full)[mi, ni].astype(np.float64)
    mag = oracle.grouped_gemm_entries(qa & 0x7F, np.abs(sa), qb & 0x7F, np.abs(sb), off, mi, ni)
    assert (np.abs(got - ref) <= 1e-3 * mag).all(), f"grouped G={G}: sampled entries off the oracle"


@pytest.mark.parametrize("M", [1, 3, 129])
def test_stream_thin_m(M):
    """A few rows and more than 256 column tiles: workgroups stream from
    one ragged single-M-tile tile to the next along N."""
    native_loaded()
    N, K = 256 * 300 - 40, 128 * 12
    qa, sa, qb, sb = _operands(M, N, K, seed=400 + M)
    announce(f"stream thin M={M} N={N} K={K}")
    a, sa_d, b, sb_d = _dev(qa), _dev(sa), _dev(qb), _dev(sb)
    full = fp8bs.gemm(a, sa_d, b, sb_d, fp8bs.BSCALE_BLOCK_128x128, out_f32=True)
    # column slices of at most 256 tiles (128 column tiles x at most 2 row
    # tiles): the same operations on every element
    for n0 in range(0, N, 256 * 128):
        n1 = min(N, n0 + 256 * 128)
        part = fp8bs.gemm(a, sa_d, b[n0:n1], sb_d[n0 // 128:-(-n1 // 128)], fp8bs.BSCALE_BLOCK_128x128, out_f32=True)
        fb, pb = _bits(full[:, n0:n1]), _bits(part)
        assert (fb == pb).all(), f"thin M={M}: columns {n0}..{n1}: {(fb != pb).sum()} entries differ"
    sampled_check(f"stream thin M={M}", qa, sa, qb, sb, full)


@pytest.mark.parametrize("offsets", [[0, 300, 100, 5000, -7, 1000], [0, 1000, 0, 1000, 0, 1000], [0, 0, 0, 0, 0, 0]])
def test_grouped_inconsistent_offsets_stay_in_bounds(offsets):
    """Offsets that decrease, overlap, or leave [0, M]: the kernel clamps
    every expert's rows into [0, M] (and its own tile count to the launch's
    bound), so the rows it writes are wrong at worst; a guard region past
    the output keeps its values, and consistent rows of the same launch
    shape still compute."""
    native_loaded()
    M, N, K = 1000, 512, 256
    E = len(offsets) - 1
    rng = np.random.default_rng(500)
    qa = _codes(rng, (M, K))
    sa = rng.uniform(0.5, 1.5, (M, K // 128)).astype(np.float32)
    qb = _codes(rng, (E, N, K))
    sb = rng.uniform(0.5, 1.5, (E, N // 128, K // 128)).astype(np.float32)
    announce(f"grouped inconsistent offsets {offsets}")
    guard = torch.full((M + 64, N), 7.0, dtype=torch.float32, device=dev())
    off = torch.tensor(offsets, dtype=torch.int32, device=dev())
    fp8bs.fp8bs_grouped_gemm(_dev(qa), _dev(sa), _dev(qb), _dev(sb), off, guard[:M], fp8bs.OUT_F32)
    g = host(guard)
    assert (g[M:] == 7.0).all(), "wrote past the output rows"


@pytest.mark.parametrize("N,K,out", [(576, 128 * 56, "bf16"), (2048, 128 * 16, "f32"), (200, 128 * 9, "bf16")])
def test_small_tiles_equal_large_tiles(N, K, out):
    """Block-scale problems whose 128x128 tiles all fit in one round of the
    256 persistent workgroups run on 128x128 tiles, larger ones on 128x256
    tiles.  Both compute every element with the same MFMAs and promotions:
    the rows of a small launch equal, bit for bit, the same rows inside a
    launch tall enough to take the large tiles."""
    native_loaded()
    M = 2048 if N <= 576 else 1024
    G = K // 128
    tiles_n = -(-N // 128)
    assert (M // 128) * tiles_n <= 256, "the small launch must take 128x128 tiles"
    big_m = 128 * (256 // tiles_n + 1)
    assert big_m >= M and (big_m // 128) * tiles_n > 256, "the tall launch must take 128x256 tiles"
    qa, sa, qb, sb = _operands(big_m, N, K, seed=600 + N)
    announce(f"small vs large tiles {M}x{N}x{K} ({big_m} rows) {out}")
    a, sa_d, b, sb_d = _dev(qa), _dev(sa), _dev(qb), _dev(sb)
    small = fp8bs.gemm(a[:M], sa_d[:M], b, sb_d, fp8bs.BSCALE_BLOCK_128x128, out_f32=(out == "f32"))
    tall = fp8bs.gemm(a, sa_d, b, sb_d, fp8bs.BSCALE_BLOCK_128x128, out_f32=(out == "f32"))
    fb, pb = _bits(tall[:M]), _bits(small)
    assert (fb == pb).all(), f"{(fb != pb).sum()} entries differ between the tile shapes"
    if out == "f32":
        sampled_check(f"small tiles {M}x{N}x{K}", qa[:M], sa[:M], qb, sb, small)
    else:
        d32 = fp8bs.gemm(a[:M], sa_d[:M], b, sb_d, fp8bs.BSCALE_BLOCK_128x128, out_f32=True)
        sampled_check(f"small tiles {M}x{N}x{K}", qa[:M], sa[:M], qb, sb, d32, small)
