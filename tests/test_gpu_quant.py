"""GPU parity of the quantizers: bit-exact codes and scales against the CPU
oracle on every configuration's full-size tensors, ragged and strided
shapes, and edge-case tiles."""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_fp8bs_amd import fp8bs, synth
from tests.gpu_common import (announce, bf16_dev, check_quant_equal, dev, host,
                              native_loaded)

pytestmark = pytest.mark.gpu


def _edge_rows(K, rng):
    """Rows of edge-case 1x128 tiles: zeros, signed zeros, bf16 subnormals,
    scales below 2^-100 and below the FP32 normal range, huge values,
    exact midpoints of the tile scale, one non-zero element."""
    G = K // 128
    rows = []
    def tiles(fn):
        r = np.zeros(K, np.float32)
        for g in range(G):
            r[g * 128:(g + 1) * 128] = fn(g)
        rows.append(r)
    tiles(lambda g: np.zeros(128, np.float32))
    tiles(lambda g: -np.zeros(128, np.float32) * (g % 2))
    for e in (-133, -128, -124, -118, -110, -95, -60, 0, 60, 120, 126):
        tiles(lambda g, e=e: np.clip(rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** (e - g % 3)),
                                     -3.38e38, 3.38e38))
    tab = oracle.e4m3_table()[:127]
    def mids(g):
        # amax 448 * 2^e makes the scale exactly 2^e; the other values are
        # exact E4M3 rounding midpoints times 2^e (ties to even)
        e = g % 7 - 3
        k = rng.integers(0, 126, 128)
        v = (0.5 * (tab[k] + tab[k + 1]) * 2.0 ** e).astype(np.float32)
        v[0] = np.float32(448.0 * 2.0 ** e)
        return v * rng.choice([-1, 1], 128).astype(np.float32)
    tiles(mids)
    def one(g):
        v = np.zeros(128, np.float32)
        v[g % 128] = -3.0
        return v
    tiles(one)
    tiles(lambda g: np.full(128, 3.3895e38, np.float32) * rng.choice([-1, 1], 128).astype(np.float32))
    return synth.bf16_bits(np.stack(rows))


def _run_act(x_u16, ldx_pad=0, ldq_pad=0, lds_pad=0):
    M, K = x_u16.shape
    G = K // 128
    xb = torch.zeros((M, K + ldx_pad), dtype=torch.bfloat16, device=dev())
    xb[:, :K] = bf16_dev(x_u16)
    q = torch.full((M, K + ldq_pad), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((M, G + lds_pad), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_act_1x128(xb[:, :K], q[:, :K], s[:, :G])
    qh, sh = host(q), host(s)
    if ldq_pad:
        assert (qh[:, K:] == 0x55).all(), "wrote past the row"
    if lds_pad:
        assert (sh[:, G:] == -1.0).all(), "wrote past the scale row"
    return qh[:, :K], sh[:, :G]


CONFIG_ACT = {
    "tiny_A_128x512": lambda: synth.tiny()["A"],
    "probe_A_1024x4096": lambda: synth.probe()["A"],
    "mlp_up_X_4096x7168": lambda: synth.mlp_up(with_w=False)["X"],
    "moe_A_up_16384x7168": lambda: synth.moe(parts=("A_up",))["A_up"],
    "moe_A_down_16384x2048": lambda: synth.moe(parts=("A_down",))["A_down"],
    "wgrad_X_8192x7168": lambda: synth.wgrad()["X"],
}


@pytest.mark.parametrize("name", list(CONFIG_ACT))
def test_quant_act_configs_bit_exact(name):
    native_loaded()
    announce(f"quant_act {name}")
    x = CONFIG_ACT[name]()
    q, s = _run_act(x)
    qr, sr = oracle.quant_act_1x128(x)
    check_quant_equal(name, q, s, qr, sr)


def test_quant_act_edge_tiles_ragged_strided():
    native_loaded()
    rng = np.random.default_rng(21)
    for K in (128, 384, 1024):
        edge = _edge_rows(K, rng)
        body = synth.tiny(M=1000 - edge.shape[0], N=1, K=K, seed=K)["A"]
        x = np.concatenate([edge, body])
        announce(f"quant_act edge/ragged M={x.shape[0]} K={K}")
        q, s = _run_act(x, ldx_pad=64, ldq_pad=32, lds_pad=3)
        qr, sr = oracle.quant_act_1x128(x)
        check_quant_equal(f"edge K={K}", q, s, qr, sr)


def test_quant_act_converter_all_bf16_values():
    """Tiles holding a 448 (so the scale is exactly 1) and every bf16 value
    of magnitude <= 448: the codes are the nearest-even E4M3 of each
    value, for all of them."""
    native_loaded()
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    v = vals[keep]
    per = 127
    n_tiles = (v.size + per - 1) // per
    pad = np.zeros(n_tiles * per, np.float32)
    pad[:v.size] = v
    tiles = np.concatenate([np.full((n_tiles, 1), 448.0, np.float32), pad.reshape(n_tiles, per)], axis=1)
    x = synth.bf16_bits(tiles.reshape(-1, 512)) if n_tiles % 4 == 0 else synth.bf16_bits(
        np.concatenate([tiles, np.zeros((4 - n_tiles % 4, 128), np.float32)]).reshape(-1, 512))
    announce(f"quant_act converter sweep {v.size} bf16 values")
    q, s = _run_act(x)
    qr, sr = oracle.quant_act_1x128(x)
    check_quant_equal("converter sweep", q, s, qr, sr)


def test_quant_act_deterministic():
    native_loaded()
    x = synth.mlp_up(T=512, K=7168, with_w=False)["X"]
    q1, s1 = _run_act(x)
    q2, s2 = _run_act(x)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def _run_w(w_u16, ldw_pad=0, ldq_pad=0, lds_pad=0):
    N, K = w_u16.shape
    G = K // 128
    NB = (N + 127) // 128
    wb = torch.zeros((N, K + ldw_pad), dtype=torch.bfloat16, device=dev())
    wb[:, :K] = bf16_dev(w_u16)
    q = torch.full((N, K + ldq_pad), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((NB, G + lds_pad), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_w_128x128(wb[:, :K], q[:, :K], s[:, :G])
    qh, sh = host(q), host(s)
    if ldq_pad:
        assert (qh[:, K:] == 0x55).all()
    if lds_pad:
        assert (sh[:, G:] == -1.0).all()
    return qh[:, :K], sh[:, :G]


CONFIG_W = {
    "tiny_W_256x512": lambda: synth.tiny()["W"],
    "probe_W_1024x4096": lambda: synth.probe()["W"],
    "mlp_up_W_18432x7168": lambda: synth.mlp_up(T=8, K=7168, N=18432)["W"],
    "moe_W_up_8x4096x7168": lambda: synth.moe(parts=("W_up",))["W_up"].reshape(-1, 7168),
    "moe_W_down_8x7168x2048": lambda: synth.moe(parts=("W_down",))["W_down"].reshape(-1, 2048),
}


@pytest.mark.parametrize("name", list(CONFIG_W))
def test_quant_w_configs_bit_exact(name):
    native_loaded()
    announce(f"quant_w {name}")
    w = CONFIG_W[name]()
    q, s = _run_w(w)
    qr, sr = oracle.quant_w_128x128(w)
    check_quant_equal(name, q, s, qr, sr)


def test_quant_w_ragged_strided_edge_blocks():
    native_loaded()
    rng = np.random.default_rng(5)
    for N in (1, 127, 200, 300):
        w = synth.tiny(M=1, N=N, K=512, seed=N)["W"].copy()
        wf = synth.bf16_to_f32(w).copy()
        if N >= 200:
            wf[128:, 128:256] = 0.0                                    # zero block (partial)
            wf[:128, 256:384] *= np.float32(2.0 ** -120)               # subnormal scale
            wf[:, 384:] *= np.float32(2.0 ** 100)                      # large
        w = synth.bf16_bits(wf)
        announce(f"quant_w ragged N={N}")
        q, s = _run_w(w, ldw_pad=8, ldq_pad=16, lds_pad=1)
        qr, sr = oracle.quant_w_128x128(w)
        check_quant_equal(f"quant_w N={N}", q, s, qr, sr)


def _run_act_w(x_u16, w_u16, pad=0):
    """fp8bs_quant_act_w on host bf16 arrays (rows optionally padded)."""
    M, K = x_u16.shape
    N = w_u16.shape[0]
    G, NB = K // 128, (N + 127) // 128
    xb = torch.zeros((M, K + pad), dtype=torch.bfloat16, device=dev())
    wb = torch.zeros((N, K + pad), dtype=torch.bfloat16, device=dev())
    if M:
        xb[:, :K] = bf16_dev(x_u16)
    if N:
        wb[:, :K] = bf16_dev(w_u16)
    qx = torch.full((M, K + pad), 0x55, dtype=torch.uint8, device=dev())
    sx = torch.full((M, G + pad // 16), -1.0, dtype=torch.float32, device=dev())
    qw = torch.full((N, K + pad), 0x55, dtype=torch.uint8, device=dev())
    sw = torch.full((NB, G + pad // 16), -1.0, dtype=torch.float32, device=dev())
    fp8bs.fp8bs_quant_act_w(xb[:, :K], qx[:, :K], sx[:, :G], wb[:, :K], qw[:, :K], sw[:, :G])
    qxh, sxh, qwh, swh = host(qx), host(sx), host(qw), host(sw)
    if pad:
        assert (qxh[:, K:] == 0x55).all() and (qwh[:, K:] == 0x55).all(), "wrote past a code row"
        assert (sxh[:, G:] == -1.0).all() and (swh[:, G:] == -1.0).all(), "wrote past a scale row"
    return qxh[:, :K], sxh[:, :G], qwh[:, :K], swh[:, :G]


@pytest.mark.parametrize("name", ["tiny", "mlp_up", "moe_down"])
def test_quant_act_w_one_launch_bit_exact(name):
    """The layer's activation and weight quantized in one launch: the same
    codes and scales as the two quantizers (oracle), at full size."""
    native_loaded()
    announce(f"quant_act_w {name}")
    if name == "tiny":
        d = synth.tiny()
        x, w = d["A"], d["W"]
    elif name == "mlp_up":
        d = synth.mlp_up()
        x, w = d["X"], d["W"]
    else:
        d = synth.moe(parts=("A_down", "W_down"))
        x, w = d["A_down"], d["W_down"].reshape(-1, 2048)
    qx, sx, qw, sw = _run_act_w(x, w)
    check_quant_equal(f"{name} activation", qx, sx, *oracle.quant_act_1x128(x))
    check_quant_equal(f"{name} weight", qw, sw, *oracle.quant_w_128x128(w))


def test_quant_act_w_ragged_strided_and_one_side_empty():
    native_loaded()
    rng = np.random.default_rng(77)
    for M, N, K in ((3, 300, 384), (1000, 1, 128), (0, 200, 512), (130, 0, 1664), (77, 129, 7168)):
        x = synth.tiny(M=max(M, 1), N=1, K=K, seed=M + K)["A"][:M]
        w = synth.tiny(M=1, N=max(N, 1), K=K, seed=N + K)["W"][:N]
        if M >= 3:
            x = np.concatenate([_edge_rows(K, rng)[:M], x])[:M]
        announce(f"quant_act_w ragged M={M} N={N} K={K}")
        qx, sx, qw, sw = _run_act_w(x, w, pad=32)
        if M:
            check_quant_equal(f"act M={M} K={K}", qx, sx, *oracle.quant_act_1x128(x))
        if N:
            check_quant_equal(f"w N={N} K={K}", qw, sw, *oracle.quant_w_128x128(w))
