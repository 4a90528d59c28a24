"""GPU parity past 32-bit sizes: inputs of more than 2^31 elements and
operands or outputs larger than 4 GiB, where any 32-bit element or byte
offset would wrap.  Sampled rows and tiles are checked against the CPU
oracle (bit-exact for codes and scales, the GEMM tolerance for outputs),
and properties that hold at any size are checked on the whole output on
the device:

* every 1x128 or 128x1 tile with a non-zero scale holds a code of
  magnitude 448 (0x7E), since amax / (amax / 448) rounds to 448;
* a BF16 GEMM output equals the FP32 output of the same launch rounded to
  nearest-even;
* padding columns past the last output column are never written.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs
from tests.gpu_common import (announce, check_f32_gemm, check_gemm_outputs, check_quant_equal, dev,
                              gemm_mag, host, native_loaded, sample_idx)
from tests.test_gpu_swiglu import _check as swiglu_check

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _random_codes(rows, cols, seed):
    """Random finite E4M3 codes (every byte but 0x7F and 0xFF) on the device."""
    g = torch.Generator(device=dev()).manual_seed(seed)
    q = torch.randint(0, 254, (rows, cols), dtype=torch.uint8, device=dev(), generator=g)
    q += (q >= 127).to(torch.uint8)
    return q


def _positive_scales(rows, cols, seed):
    g = torch.Generator(device=dev()).manual_seed(seed)
    return torch.rand((rows, cols), dtype=torch.float32, device=dev(), generator=g) * 0.01 + 0.001


def _max_code_per_tile(q_tiles, s_tiles):
    """All tiles with a positive scale have a code of magnitude 448."""
    amax = (q_tiles & 0x7F).amax(dim=-1)
    bad = ((amax != 0x7E) & (s_tiles > 0)).sum().item()
    zero = (s_tiles <= 0).sum().item()
    return bad, zero


def test_quant_act_past_2_31_elements():
    """x [2^19 + 3][4096] bf16 (2^31 + 12288 elements, 4 GiB)."""
    native_loaded()
    M, K = (1 << 19) + 3, 4096
    G = K // 128
    announce(f"large: quant_act {M}x{K}")
    g = torch.Generator(device=dev()).manual_seed(11)
    x = torch.randn((M, K), dtype=torch.float32, device=dev(), generator=g).to(torch.bfloat16)
    _free()
    q = torch.empty((M, K), dtype=torch.uint8, device=dev())
    s = torch.empty((M, G), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_act_1x128(x, q, s)
    torch.cuda.synchronize()
    bad, zero = _max_code_per_tile(q.view(M, G, 128), s)
    assert zero == 0 and bad == 0, f"{bad} tiles without a 448 code, {zero} zero scales"
    rows = np.array([0, 1, 2, 3, M // 2, M // 2 + 1, (1 << 18) - 1, 1 << 18,
                     (1 << 19) - 2, (1 << 19) - 1, 1 << 19, M - 2, M - 1])
    ri = torch.from_numpy(rows).to(dev())
    xs = host(x[ri].contiguous())
    q_ref, s_ref = oracle.quant_act_1x128(xs)
    check_quant_equal("quant_act past 2^31", host(q[ri].contiguous()), host(s[ri].contiguous()), q_ref, s_ref)
    del x, q, s
    _free()


def test_gemm_output_past_4_gib():
    """D [65541][32776] (ldd 32784): 4.3 GB of BF16 and 8.6 GB of FP32
    output, so the epilogue's row offsets pass 2^32 bytes; K = 256."""
    native_loaded()
    M, N, K = 65541, 32776, 256
    LD = N + 8
    announce(f"large: gemm output {M}x{N} (ld {LD}), K {K}")
    g = torch.Generator(device=dev()).manual_seed(12)
    xa = torch.randn((M, K), dtype=torch.float32, device=dev(), generator=g).to(torch.bfloat16)
    xb = (torch.randn((N, K), dtype=torch.float32, device=dev(), generator=g) * 0.02).to(torch.bfloat16)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev())
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev())
    qb = torch.empty((N, K), dtype=torch.uint8, device=dev())
    sb = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_act_1x128(xa, qa, sa)
    fp8bs.fp8bs_quant_w_128x128(xb, qb, sb)
    del xa, xb
    _free()
    d16 = torch.full((M, LD), -7.0, dtype=torch.bfloat16, device=dev())
    d32 = torch.full((M, LD), -7.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_gemm(qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, d16[:, :N], fp8bs.OUT_BF16)
    fp8bs.fp8bs_gemm(qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, d32[:, :N], fp8bs.OUT_F32)
    torch.cuda.synchronize()
    assert bool((d16[:, N:] == -7.0).all()) and bool((d32[:, N:] == -7.0).all()), "wrote into the padding"
    # BF16 == RNE(FP32) on every entry, in row slices to bound the temporaries
    for r0 in range(0, M, 8192):
        sl = slice(r0, min(M, r0 + 8192))
        same = torch.equal(d32[sl, :N].to(torch.bfloat16).view(torch.int16), d16[sl, :N].view(torch.int16))
        assert same, f"bf16 output differs from the rounded fp32 output in rows {sl}"
    mi, ni = sample_idx(M, N)
    mi = np.concatenate([mi, np.full(8, M - 1), np.arange(M - 8, M)])
    ni = np.concatenate([ni, np.arange(N - 8, N), np.full(8, N - 1)])
    qa_h, sa_h, qb_h, sb_h = host(qa), host(sa), host(qb), host(sb)
    ref = oracle.gemm_entries(qa_h, sa_h, qb_h, sb_h, mi, ni)
    mag = gemm_mag(qa_h, sa_h, qb_h, sb_h, oracle.BSCALE_BLOCK, mi, ni)
    mt, nt = torch.from_numpy(mi).to(dev()), torch.from_numpy(ni).to(dev())
    s32 = host(d32[mt, nt].contiguous())
    s16 = host(d16[mt, nt].contiguous())
    check_gemm_outputs("gemm output past 4 GiB", s32, s16, ref, mag)
    del qa, sa, qb, sb, d16, d32
    _free()


def test_gemm_a_operand_past_4_gib():
    """A [2^20 + 7][4224] codes (4.4 GB): the per-tile copy bases pass
    2^32 bytes; N = 136 (a ragged second column tile), FP32 output."""
    native_loaded()
    M, N, K = (1 << 20) + 7, 136, 4224
    G = K // 128
    announce(f"large: gemm A operand {M}x{K}, N {N}")
    qa = _random_codes(M, K, 13)
    _free()
    sa = _positive_scales(M, G, 14)
    qb = _random_codes(N, K, 15)
    sb = _positive_scales((N + 127) // 128, G, 16)
    d = torch.full((M, N), -7.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_gemm(qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, d, fp8bs.OUT_F32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, M // 2, (1 << 20) - 129, (1 << 20) - 1] + list(range(M - 9, M)))
    ri = torch.from_numpy(rows).to(dev())
    qa_h, sa_h = host(qa[ri].contiguous()), host(sa[ri].contiguous())
    qb_h, sb_h = host(qb), host(sb)
    ref = oracle.gemm(qa_h, sa_h, qb_h, sb_h)
    mag = gemm_mag(qa_h, sa_h, qb_h, sb_h)
    fro, worst = check_f32_gemm("gemm A past 4 GiB", host(d[ri].contiguous()), ref, mag)
    announce(f"gemm A past 4 GiB: rel-fro {fro:.2e} max-err/sum|ab| {worst:.2e} on {rows.size} rows")
    del qa, sa, qb, sb, d
    _free()


def test_requant_fp8_past_2_31_elements():
    """q [2^19 + 133][4096] FP8 codes (2^31 + 544768 elements) re-quantized
    to [4096][2^19 + 133]: the output row offsets pass 2^31 bytes and the
    last token tile is ragged."""
    native_loaded()
    T, C = (1 << 19) + 133, 4096
    TB = (T + 127) // 128
    Tp = (T + 15) // 16 * 16
    announce(f"large: requant fp8 {T}x{C}")
    x = _random_codes(T, C, 17)
    s_in = _positive_scales(T, C // 128, 18)
    q = torch.full((C, Tp), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((C, TB), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_FP8_1x128, x, s_in, q[:, :T], s)
    torch.cuda.synchronize()
    assert bool((q[:, T:] == 0x55).all()), "wrote past the output rows"
    full = (T // 128) * 128
    bad, zero = _max_code_per_tile(q[:, :full].reshape(C, T // 128, 128), s[:, :T // 128])
    assert zero == 0 and bad == 0, f"{bad} tiles without a 448 code, {zero} zero scales"
    for t0, c0 in [(0, 0), (1 << 18, 2048), (full - 128, C - 128), (full, C - 128), (full, 0)]:
        tt = min(128, T - t0)
        xs = host(x[t0:t0 + tt, c0:c0 + 128].contiguous())
        ss = host(s_in[t0:t0 + tt, c0 // 128:c0 // 128 + 1].contiguous())
        q_ref, s_ref = oracle.requant_T_128x1_fp8(xs, ss)
        check_quant_equal(f"requant past 2^31, tile ({t0}, {c0})",
                          host(q[c0:c0 + 128, t0:t0 + tt].contiguous()),
                          host(s[c0:c0 + 128, t0 // 128:t0 // 128 + 1].contiguous()), q_ref, s_ref)
    del x, s_in, q, s
    _free()


def test_quant_w_past_2_31_elements():
    """w [2^18 + 129][8192] bf16 (2^31 + 1M elements): 2050 block rows, the
    last one a single row."""
    native_loaded()
    N, K = (1 << 18) + 129, 8192
    G, NB = K // 128, (N + 127) // 128
    announce(f"large: quant_w {N}x{K}")
    g = torch.Generator(device=dev()).manual_seed(19)
    w = (torch.randn((N, K), dtype=torch.float32, device=dev(), generator=g) * 0.01).to(torch.bfloat16)
    _free()
    q = torch.empty((N, K), dtype=torch.uint8, device=dev())
    s = torch.empty((NB, G), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_w_128x128(w, q, s)
    torch.cuda.synchronize()
    full = (N // 128) * 128
    blocks = (q[:full].view(N // 128, 128, G, 128) & 0x7F).amax(dim=3).amax(dim=1)
    bad = ((blocks != 0x7E) & (s[:N // 128] > 0)).sum().item()
    assert bad == 0 and (s > 0).all().item(), f"{bad} blocks without a 448 code"
    for nb in [0, NB // 2, NB - 2, NB - 1]:
        r0, r1 = nb * 128, min(N, nb * 128 + 128)
        q_ref, s_ref = oracle.quant_w_128x128(host(w[r0:r1].contiguous()))
        check_quant_equal(f"quant_w past 2^31, block row {nb}", host(q[r0:r1].contiguous()),
                          host(s[nb:nb + 1].contiguous()), q_ref, s_ref)
    del w, q, s
    _free()


def test_requant_bf16_past_2_31_elements():
    """bf16 dY [2^18 + 65][8192] (4.3 GB) re-quantized to [8192][2^18 + 65]."""
    native_loaded()
    T, C = (1 << 18) + 65, 8192
    TB = (T + 127) // 128
    Tp = (T + 15) // 16 * 16
    announce(f"large: requant bf16 {T}x{C}")
    g = torch.Generator(device=dev()).manual_seed(20)
    x = (torch.randn((T, C), dtype=torch.float32, device=dev(), generator=g) * 0.01).to(torch.bfloat16)
    _free()
    q = torch.full((C, Tp), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((C, TB), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_BF16, x, None, q[:, :T], s)
    torch.cuda.synchronize()
    assert bool((q[:, T:] == 0x55).all()), "wrote past the output rows"
    full = (T // 128) * 128
    bad, zero = _max_code_per_tile(q[:, :full].reshape(C, T // 128, 128), s[:, :T // 128])
    assert zero == 0 and bad == 0, f"{bad} tiles without a 448 code, {zero} zero scales"
    for t0, c0 in [(0, 0), (full - 128, C - 128), (full, C - 128), (full, 4096)]:
        tt = min(128, T - t0)
        q_ref, s_ref = oracle.requant_T_128x1_bf16(host(x[t0:t0 + tt, c0:c0 + 128].contiguous()))
        check_quant_equal(f"requant bf16 past 2^31, tile ({t0}, {c0})",
                          host(q[c0:c0 + 128, t0:t0 + tt].contiguous()),
                          host(s[c0:c0 + 128, t0 // 128:t0 // 128 + 1].contiguous()), q_ref, s_ref)
    del x, q, s
    _free()


def test_e5m6_past_2_31_elements():
    """x [2^18 + 1][8192] bf16 encoded to 3.2 GB of packed E5M6 and decoded;
    on every element, encoding the decoded values gives the same codes."""
    native_loaded()
    T, C = (1 << 18) + 1, 8192
    P = (3 * C + 1) // 2
    announce(f"large: e5m6 {T}x{C}")
    g = torch.Generator(device=dev()).manual_seed(21)
    x = torch.randn((T, C), dtype=torch.float32, device=dev(), generator=g).to(torch.bfloat16)
    _free()
    y = torch.empty((T, P), dtype=torch.uint8, device=dev())
    fp8bs.fp8bs_encode_e5m6(x, y)
    x2 = torch.empty_like(x)
    fp8bs.fp8bs_decode_e5m6(y, x2)
    y2 = torch.empty_like(y)
    fp8bs.fp8bs_encode_e5m6(x2, y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "encode(decode(y)) != y"
    rows = np.array([0, 1, T // 2, T - 2, T - 1])
    ri = torch.from_numpy(rows).to(dev())
    y_ref = oracle.encode_e5m6(host(x[ri].contiguous()))
    y_h = host(y[ri].contiguous())
    assert np.array_equal(y_h, y_ref), "packed E5M6 rows differ from the oracle"
    x_ref = oracle.decode_e5m6(y_ref, C)
    assert np.array_equal(host(x2[ri].contiguous()), x_ref), "decoded rows differ from the oracle"
    del x, y, x2, y2
    _free()


def test_swiglu_quant_past_2_31_elements():
    """g, u [2^18 + 3][8192] bf16 (4.3 GB each) -> 1x128 codes and scales."""
    native_loaded()
    T, I = (1 << 18) + 3, 8192
    G = I // 128
    announce(f"large: swiglu quant {T}x{I}")
    gen = torch.Generator(device=dev()).manual_seed(22)
    g = torch.randn((T, I), dtype=torch.float32, device=dev(), generator=gen).to(torch.bfloat16)
    u = torch.randn((T, I), dtype=torch.float32, device=dev(), generator=gen).to(torch.bfloat16)
    _free()
    q = torch.empty((T, I), dtype=torch.uint8, device=dev())
    s = torch.empty((T, G), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_swiglu_quant_1x128(g, u, q, s, None)
    torch.cuda.synchronize()
    bad, zero = _max_code_per_tile(q.view(T, G, 128), s)
    assert zero == 0 and bad == 0, f"{bad} tiles without a 448 code, {zero} zero scales"
    # h is computed in FP32 (exp, a reciprocal, two products), so the
    # sampled rows follow the SwiGLU comparison rule (scales within 2^-19,
    # codes the oracle's or a midpoint neighbour, at most 0.5% differing)
    rows = np.array([0, 1, 2, 3, T // 2 - 1, T // 2, (1 << 18) - 1, 1 << 18] + list(range(T - 8, T)))
    ri = torch.from_numpy(rows).to(dev())
    ref = oracle.swiglu_quant_1x128(host(g[ri].contiguous()), host(u[ri].contiguous()))
    swiglu_check("swiglu quant past 2^31", {"q": host(q[ri].contiguous()), "s": host(s[ri].contiguous())}, ref)
    del g, u, q, s
    _free()


def test_grouped_gemm_weights_past_4_gib():
    """66 experts of B [8192][8192] codes (4.4 GB): the last experts' B
    starts past 2^32 bytes.  Their rows are checked against the dense
    oracle GEMM of the expert (the grouped GEMM is the per-expert GEMM over
    the expert's rows), B scales as 128-row blocks."""
    native_loaded()
    E, N, K = 66, 8192, 8192
    G = K // 128
    announce(f"large: grouped gemm {E} experts of {N}x{K}")
    counts = np.array([(37 * e) % 150 for e in range(E)], np.int64)
    counts[-1], counts[-2] = 300, 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    a = _random_codes(M, K, 23)
    sa = _positive_scales(M, G, 24)
    b = _random_codes(E * N, K, 25).view(E, N, K)
    _free()
    sb = _positive_scales(E * (N // 128), G, 26).view(E, N // 128, G)
    d = torch.empty((M, N), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_grouped_gemm(a, sa, b, sb, torch.from_numpy(off).to(dev()), d, fp8bs.OUT_F32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(27)
    for e in [0, E // 2, E - 3, E - 1]:
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        rows = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, 6)]))
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
        ri, ci = torch.from_numpy(rows).to(dev()), torch.from_numpy(cols).to(dev())
        a_h, sa_h = host(a[ri].contiguous()), host(sa[ri].contiguous())
        b_h = host(b[e][ci].contiguous())
        sb_rows = host(sb[e][ci // 128].contiguous())  # each B row's 128-row block scales
        ref = oracle.gemm(a_h, sa_h, b_h, sb_rows, oracle.BSCALE_ROW)
        mag = gemm_mag(a_h, sa_h, b_h, sb_rows, oracle.BSCALE_ROW)
        got = host(d[ri][:, ci].contiguous())
        fro, worst = check_f32_gemm(f"grouped past 4 GiB, expert {e}", got, ref, mag)
        announce(f"grouped past 4 GiB expert {e}: rel-fro {fro:.2e} max-err/sum|ab| {worst:.2e}")
    del a, sa, b, sb, d
    _free()


def test_transpose_w_past_2_31_elements():
    """q [2^18][8320] codes (2^31 + 33.5M elements) with their 128x128 block
    scales: the transpose equals q^T and s^T on every element, and sampled
    blocks equal the oracle's."""
    native_loaded()
    N, K = 1 << 18, 8320
    G = K // 128
    announce(f"large: transpose_w {N}x{K}")
    q = _random_codes(N, K, 28)
    s = _positive_scales(N // 128, G, 29)
    qt = torch.empty((K, N), dtype=torch.uint8, device=dev())
    st = torch.empty((G, N // 128), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_transpose_w_128x128(q, s, qt, st)
    torch.cuda.synchronize()
    for k0 in range(0, K, 1024):   # q^T in slices of 1024 rows of qt
        assert torch.equal(qt[k0:k0 + 1024], q[:, k0:k0 + 1024].t().contiguous()), f"qt rows {k0}.."
    assert torch.equal(st, s.t().contiguous())
    for nb, kb in [(0, 0), (N // 256, G // 2), (N // 128 - 1, G - 1)]:
        qb = host(q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].contiguous())
        sbk = host(s[nb:nb + 1, kb:kb + 1].contiguous())
        q_ref, s_ref = oracle.transpose_w_128x128(qb, sbk)
        check_quant_equal(f"transpose_w past 2^31, block ({nb}, {kb})",
                          host(qt[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128].contiguous()),
                          host(st[kb:kb + 1, nb:nb + 1].contiguous()), q_ref, s_ref)
    del q, s, qt, st
    _free()


def test_gemm_quant_output_past_4_gib():
    """GEMM with its output quantized 1x128: codes [65541][65792] (ld 65808),
    4.3 GB; K = 128.  Sampled rows follow the fused-output rule against the
    binary64 oracle GEMM (scales within the GEMM allowance of the tile's
    max-abs, codes within half an E4M3 step plus the allowance)."""
    from tests.test_gpu_gemm_quant import _check_against_f64
    native_loaded()
    M, N, K = 65541, 65792, 128
    LD = N + 16
    announce(f"large: gemm_quant output {M}x{N} (ld {LD}), K {K}")
    g = torch.Generator(device=dev()).manual_seed(30)
    xa = torch.randn((M, K), dtype=torch.float32, device=dev(), generator=g).to(torch.bfloat16)
    xb = (torch.randn((N, K), dtype=torch.float32, device=dev(), generator=g) * 0.05).to(torch.bfloat16)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev())
    sa = torch.empty((M, 1), dtype=torch.float32, device=dev())
    qb = torch.empty((N, K), dtype=torch.uint8, device=dev())
    sb = torch.empty(((N + 127) // 128, 1), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_act_1x128(xa, qa, sa)
    fp8bs.fp8bs_quant_w_128x128(xb, qb, sb)
    del xa, xb
    q = torch.full((M, LD), 0x55, dtype=torch.uint8, device=dev())
    s = torch.empty((M, N // 128), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_gemm_quant_1x128(qa, sa, qb, sb, fp8bs.BSCALE_BLOCK_128x128, q[:, :N], s)
    torch.cuda.synchronize()
    assert bool((q[:, N:] == 0x55).all()), "wrote into the padding"
    for r0 in range(0, M, 8192):
        sl = slice(r0, min(M, r0 + 8192))
        bad, zero = _max_code_per_tile(q[sl, :N].reshape(-1, N // 128, 128), s[sl])
        assert zero == 0 and bad == 0, f"rows {sl}: {bad} tiles without a 448 code, {zero} zero scales"
    rows = np.array([0, 1, M // 2, 65535, 65536, M - 2, M - 1])
    ri = torch.from_numpy(rows).to(dev())
    a_h, sa_h = host(qa[ri].contiguous()), host(sa[ri].contiguous())
    b_h, sb_h = host(qb), host(sb)
    d_ref = oracle.gemm(a_h, sa_h, b_h, sb_h)
    mag = gemm_mag(a_h, sa_h, b_h, sb_h)
    _check_against_f64("gemm_quant past 4 GiB", host(q[ri, :N].contiguous()), host(s[ri].contiguous()), d_ref, mag)
    del qa, sa, qb, sb, q, s
    _free()


def test_quant_per_tensor_past_2_31_elements():
    """2^31 + 384 bf16 values with one scale.  Element 0 holds the tensor's
    largest magnitude (the rest are clamped below it), so the oracle on the
    sampled elements together with element 0 has the same scale."""
    native_loaded()
    n = (1 << 31) + 384
    announce(f"large: quant_per_tensor n = {n}")
    g = torch.Generator(device=dev()).manual_seed(31)
    x = torch.randn((n,), dtype=torch.float32, device=dev(), generator=g).clamp_(-100.0, 100.0).to(torch.bfloat16)
    x[0] = 300.0
    _free()
    q = torch.empty((n,), dtype=torch.uint8, device=dev())
    s = torch.empty((1,), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_per_tensor(x, q, s)
    torch.cuda.synchronize()
    idx = np.concatenate([np.arange(0, 128), np.arange(1 << 30, (1 << 30) + 128),
                          np.arange(n - 256, n)])
    it = torch.from_numpy(idx).to(dev())
    q_ref, s_ref = oracle.quant_per_tensor(host(x[it].contiguous()))
    s_gpu = host(s)
    assert s_gpu.view(np.uint32)[0] == np.float32(s_ref).view(np.uint32), f"scale {s_gpu[0]!r} vs {s_ref!r}"
    q_gpu = host(q[it].contiguous())
    bad = np.flatnonzero(q_gpu != q_ref)
    assert bad.size == 0, f"{bad.size} codes differ, first at element {idx[bad[0]]}"
    del x, q, s
    _free()


def test_cast_e4m3_past_2_31_elements():
    """2^31 + 24 FP32 values (8.6 GB) encoded at unit scale; sampled
    elements against the oracle's encoder."""
    native_loaded()
    n = (1 << 31) + 24
    announce(f"large: cast_e4m3 n = {n}")
    g = torch.Generator(device=dev()).manual_seed(32)
    x = torch.randn((n,), dtype=torch.float32, device=dev(), generator=g) * 100.0
    q = torch.empty((n,), dtype=torch.uint8, device=dev())
    fp8bs.fp8bs_cast_e4m3(x, q)
    torch.cuda.synchronize()
    assert not bool(((q & 0x7F) == 0x7F).any()), "a NaN code for a finite input"
    rng = np.random.default_rng(33)
    idx = np.unique(np.concatenate([rng.integers(0, n, 2000), np.arange(n - 40, n), np.arange(0, 8)]))
    it = torch.from_numpy(idx).to(dev())
    xs, qs = host(x[it].contiguous()), host(q[it].contiguous())
    want = np.array([oracle.e4m3_encode(float(v)) for v in xs], np.uint8)
    bad = np.flatnonzero(qs != want)
    assert bad.size == 0, f"{bad.size} codes differ, first at element {idx[bad[0]]}: {xs[bad[0]]!r}"
    del x, q
    _free()


def test_gemm_bf16a_a_past_4_gib():
    """BF16 A [2^19 + 5][4224] (4.4 GB) quantized inside the GEMM, N = 136,
    codes stored: stored rows bit-exact against the oracle's 1x128
    quantizer, D rows within the GEMM tolerance of the oracle GEMM on those
    codes."""
    native_loaded()
    M, N, K = (1 << 19) + 5, 136, 4224
    G = K // 128
    announce(f"large: gemm_bf16a {M}x{K}, N {N}")
    gen = torch.Generator(device=dev()).manual_seed(34)
    x = torch.randn((M, K), dtype=torch.float32, device=dev(), generator=gen).to(torch.bfloat16)
    _free()
    qb = _random_codes(N, K, 35)
    sb = _positive_scales((N + 127) // 128, G, 36)
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev())
    sx = torch.empty((M, G), dtype=torch.float32, device=dev())
    d = torch.empty((M, N), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_gemm_bf16a(x, qx, sx, qb, sb, d, fp8bs.OUT_F32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, M // 2, (1 << 19) - 1, 1 << 19, M - 2, M - 1])
    ri = torch.from_numpy(rows).to(dev())
    q_ref, s_ref = oracle.quant_act_1x128(host(x[ri].contiguous()))
    check_quant_equal("gemm_bf16a codes past 4 GiB", host(qx[ri].contiguous()), host(sx[ri].contiguous()),
                      q_ref, s_ref)
    b_h, sb_h = host(qb), host(sb)
    ref = oracle.gemm(q_ref, s_ref, b_h, sb_h)
    mag = gemm_mag(q_ref, s_ref, b_h, sb_h)
    fro, worst = check_f32_gemm("gemm_bf16a past 4 GiB", host(d[ri].contiguous()), ref, mag)
    announce(f"gemm_bf16a past 4 GiB: rel-fro {fro:.2e} max-err/sum|ab| {worst:.2e}")
    del x, qb, sb, qx, sx, d
    _free()


def test_quant_act_w_past_2_31_elements():
    """One launch for X [2^19 + 3][4096] (2^31 + 12288 elements) and
    W [16385][4096]: sampled X rows and the first and last W block rows
    against the oracle's two quantizers."""
    native_loaded()
    M, N, K = (1 << 19) + 3, 16385, 4096
    G = K // 128
    announce(f"large: quant_act_w X {M}x{K}, W {N}x{K}")
    gen = torch.Generator(device=dev()).manual_seed(37)
    x = torch.randn((M, K), dtype=torch.float32, device=dev(), generator=gen).to(torch.bfloat16)
    _free()
    w = (torch.randn((N, K), dtype=torch.float32, device=dev(), generator=gen) * 0.02).to(torch.bfloat16)
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev())
    sx = torch.empty((M, G), dtype=torch.float32, device=dev())
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev())
    sw = torch.empty(((N + 127) // 128, G), dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_act_w(x, qx, sx, w, qw, sw)
    torch.cuda.synchronize()
    bad, zero = _max_code_per_tile(qx.view(M, G, 128), sx)
    assert zero == 0 and bad == 0, f"{bad} X tiles without a 448 code, {zero} zero scales"
    rows = np.array([0, 1, M // 2, (1 << 19) - 1, 1 << 19, M - 2, M - 1])
    ri = torch.from_numpy(rows).to(dev())
    q_ref, s_ref = oracle.quant_act_1x128(host(x[ri].contiguous()))
    check_quant_equal("quant_act_w X past 2^31", host(qx[ri].contiguous()), host(sx[ri].contiguous()), q_ref, s_ref)
    for nb in [0, (N + 127) // 128 - 1]:
        r0, r1 = nb * 128, min(N, nb * 128 + 128)
        q_ref, s_ref = oracle.quant_w_128x128(host(w[r0:r1].contiguous()))
        check_quant_equal(f"quant_act_w W block row {nb}", host(qw[r0:r1].contiguous()),
                          host(sw[nb:nb + 1].contiguous()), q_ref, s_ref)
    del x, w, qx, sx, qw, sw
    _free()
