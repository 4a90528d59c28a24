"""CPU model of the block-scaled GEMM's global -> LDS copy plan
(fp8_fine_grained_fp8bs_amd/csrc/gemm.hip): for the two workgroup
configurations (128 x 256 with 128x128 B scales, 128 x 128 with per-row B
scales) and ragged shapes, every byte a copy can read lies inside its
buffer descriptor's range, every descriptor range lies inside its operand
(M rows of the row stride), and every code and scale the tile needs is
fetched by some lane.  Rows and groups past the end are read as zeros by
the descriptor range check, which covers the VGPR offset; the SGPR offset
carries only the K group's column offset of a tile copy.

The offsets below restate the kernel's copy plan (a model, not shared code).
"""
import numpy as np
import pytest

SBLK = 4


def cfg(brow):
    return dict(BM=128, BN=128 if brow else 256, NW=8)


def tile_copies(c, ld_a, ld_b, wave):
    """(is_a, voff per lane) of each tile copy of one wave."""
    BM, BN, NW = c["BM"], c["BN"], c["NW"]
    dpw, qa = (BM + BN) // 8 // NW, BM // 8 // NW
    lane = np.arange(64)
    r = 8 * wave + (lane >> 3)
    ch = (lane & 7) ^ ((r >> 1) & 7)
    out = []
    for k in range(dpw):
        rows = r + (k if k < qa else k - qa) * 8 * NW
        ld = ld_a if k < qa else ld_b
        out.append((k < qa, rows, rows * ld + ch * 16))
    return out


def scale_copies(c, brow, ldsa4, ldsb4, wave):
    """(kind, voff, qstep, hstep) of each scale copy of one wave; kind is
    'a', 'b' or 'dummy'."""
    BM, BN, NW = c["BM"], c["BN"], c["NW"]
    saw, sbw = BM // 64, (BN // 64 if brow else 1)
    spw = (saw + sbw + NW - 1) // NW
    lane = np.arange(64)
    grp = (lane >> 4) * 4
    out = []
    for u in range(spw):
        cc = wave + u * NW
        if cc < saw:
            out.append(("a", (16 * cc + (lane & 15)) * ldsa4 + grp, 16 * saw * ldsa4, SBLK * 4))
        elif cc < saw + sbw:
            w = cc - saw
            if brow:
                out.append(("b", (16 * w + (lane & 15)) * ldsb4 + grp, 16 * sbw * ldsb4, SBLK * 4))
            else:
                out.append(("b", (lane & 15) * ldsb4 + grp, 0, SBLK * 4))
        else:
            out.append(("dummy", np.zeros(64, np.int64), 0, 0))
    return out


CASES = [  # (brow, M, N, K, lda, ldb, ldsa, ldsb)
    (False, 4096, 18432, 7168, 7168, 7168, 56, 56),
    (False, 300, 200, 640, 640, 656, 5, 8),      # ragged M and N, G = 5 (partial scale block)
    (False, 1, 1, 128, 128, 128, 1, 1),
    (False, 129, 257, 1664, 1680, 1664, 13, 13),
    (True, 7168, 2048, 8192, 8192, 8192, 64, 64),
    (True, 200, 130, 384, 400, 384, 3, 4),
    (True, 1, 1, 128, 128, 128, 1, 1),
]


@pytest.mark.parametrize("brow,M,N,K,lda,ldb,ldsa,ldsb", CASES)
def test_copies_stay_inside_descriptors_and_cover_the_tile(brow, M, N, K, lda, ldb, ldsa, ldsb):
    c = cfg(brow)
    BM, BN, NW = c["BM"], c["BN"], c["NW"]
    G = K // 128
    ldsa4, ldsb4 = 4 * ldsa, 4 * ldsb
    tiles = [(m0, n0) for m0 in range(0, M, BM) for n0 in range(0, N, BN)]
    # the first, the last and a ragged tile are enough: offsets do not
    # depend on the tile position beyond rows_a / rows_b
    for m0, n0 in {tiles[0], tiles[-1], (tiles[-1][0], 0), (0, tiles[-1][1])}:
        rows_a, rows_b = min(BM, M - m0), min(BN, N - n0)
        num = {"a": rows_a * lda, "b": rows_b * ldb}
        # descriptor ranges inside the operands (M rows of lda bytes, ...)
        assert m0 * lda + num["a"] <= M * lda and n0 * ldb + num["b"] <= N * ldb
        got_a = np.zeros((rows_a, K), bool)
        got_b = np.zeros((rows_b, K), bool)
        for wave in range(NW):
            for is_a, rows, voff in tile_copies(c, lda, ldb, wave):
                key = "a" if is_a else "b"
                for t in range(G + 3):            # the clamped copies past the last group included
                    gk = min(t, G - 1) * 128
                    live = voff < num[key]         # lanes the range check lets through
                    assert (rows[live] < (rows_a if is_a else rows_b)).all()
                    assert (voff[live] + gk + 16 <= num[key]).all()
                    # a live lane reads 16 bytes of its row's first K bytes
                    col = (voff[live] - rows[live] * (lda if is_a else ldb)) + gk
                    assert (col + 16 <= K).all()
                    got = got_a if is_a else got_b
                    for rr, cc in zip(rows[live], col):
                        got[rr, cc:cc + 16] = True
        assert got_a.all() and got_b.all(), "some code of the tile is never copied"

        # scale copies: offset = voff + qstep q + hstep h, all in the VGPR offset
        nb = -(-rows_b // 128)
        snum = {"a": rows_a * ldsa4, "b": (rows_b if brow else nb) * ldsb4, "dummy": rows_a * ldsa4}
        assert m0 * ldsa4 + snum["a"] <= M * ldsa4
        if brow:
            assert n0 * ldsb4 + snum["b"] <= N * ldsb4
        else:
            assert (n0 // 128) * ldsb4 + snum["b"] <= -(-N // 128) * ldsb4
        need_a = np.zeros((rows_a, G), bool)
        need_b = np.zeros((rows_b if brow else nb, G), bool)
        blocks = -(-G // SBLK) + 2                 # every block a tile issues, clamped ones included
        for wave in range(NW):
            for kind, voff, qstep, hstep in scale_copies(c, brow, ldsa4, ldsb4, wave):
                for q in range(4):
                    for h in range(blocks):
                        off = voff + qstep * q + hstep * h
                        live = off < snum[kind]
                        assert (off[live] + 4 <= snum[kind]).all()
                        if kind == "dummy":
                            continue
                        ld4 = ldsa4 if kind == "a" else ldsb4
                        row, col = off[live] // ld4, (off[live] % ld4) // 4
                        ok = col < G
                        target = need_a if kind == "a" else need_b
                        target[row[ok], col[ok]] = True
        assert need_a.all() and need_b.all(), "some scale of the tile is never copied"
