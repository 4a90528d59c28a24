#!/usr/bin/env python3
"""Benchmark of the fine-grained FP8 hot path on one MI355X (gfx950).

One step = one forward pass of the K = 7168 dense MLP up-projection:
  quantize X [4096][7168] in 1x128 tiles and W [18432][7168] in 128x128
  blocks (one launch, fp8bs_quant_act_w), and the block-scaled FP8 GEMM
  Y = X W^T with BF16 output.
The inputs (seeded synthetic bf16, the heavy-tailed recipe of
``fp8_fine_grained_fp8bs_amd.synth.mlp_up``) are resident in HBM before the
timed region starts.  ``value`` is the step's throughput in GEMM TFLOP/s
(2*M*N*K flop per step divided by the wall time of the step, quantization
included).  Each kernel is also timed with HIP events on the stream it runs
on, one event before each kernel (the span to the next event is that
kernel's; an event costs about 2.5 us of GPU time, so the step records one
per kernel rather than a pair); the GEMM is the dominant kernel and its
roofline fraction is reported against the MI355X dense FP8 peak.

The other hot-path rows (the up-projection GEMM with its output quantized
for the next layer, fused and unfused; backward 1x128 -> 128x1
re-quantization, the weight-gradient GEMM with row scales, the weight
transpose and input-gradient GEMM; the grouped MoE GEMMs with their
quantization) are timed the same way after the step and reported under
"rows"; they are not part of ``value``.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: the path is
single-GPU (no collectives).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
QUEUE_FILL_CYCLES = 4_000_000  # spin before a batch of timed calls (about 2 ms)
FLUSH_BYTES = 1 << 30          # cache flush written between timed row calls
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mlp_up_4096x18432x7168_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "fp8_fine_grained_fp8bs_amd", "csrc", "gemm.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rows", choices=["all", "none"], default="all",
                    help="also time the re-quantization, wgrad and grouped rows")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--profile-kernel", choices=["quant_act", "quant_w", "quant_act_w", "gemm"],
                    help="only run this kernel of the step --steps times on the step's inputs "
                         "(for counter runs); prints no JSON line")
    return ap.parse_args()


def bf16_dev(a, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


class KernelTimer:
    """Per-kernel HIP-event timing on the current stream (the stream every
    library call here is launched on)."""

    def __init__(self):
        self.events = {}

    def run(self, name, fn):
        import torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.events.setdefault(name, []).append((s, e))

    def times_ms(self, name):
        return [s.elapsed_time(e) for s, e in self.events[name]]

    def mean_ms(self, name):
        t = self.times_ms(name)
        return sum(t) / len(t)

    def stats_us(self, name):
        """mean, median and min of the recorded calls, in microseconds."""
        t = sorted(self.times_ms(name))
        n = len(t)
        med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
        return {"us": sum(t) / n * 1e3, "us_median": med * 1e3, "us_min": t[0] * 1e3, "calls": n}

    def reset(self):
        self.events = {}


class ChainTimer(KernelTimer):
    """HIP events for a sequence of kernels run back to back on the current
    stream: one event before each kernel, and one after the last kernel of
    the sequence; a kernel's time is the span from its event to the next.
    Each event costs about 2.5 us of GPU time between kernels, so the
    step records one per kernel instead of a start and an end each."""

    def __init__(self):
        super().__init__()
        self.marks = []

    def run(self, name, fn):
        import torch
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append((name, e))
        fn()

    def close(self):
        """Record the closing event and turn the marks into (start, end)
        pairs per kernel name."""
        import torch
        end = torch.cuda.Event(enable_timing=True)
        end.record()
        for (name, s), (_, e) in zip(self.marks, self.marks[1:] + [(None, end)]):
            self.events.setdefault(name, []).append((s, e))
        self.marks = []

    def reset(self):
        super().reset()
        self.marks = []


class CacheFlush:
    """Writes FLUSH_BYTES (more than the 256 MB MALL and all L2s together,
    four times over) on the current stream, so that a following kernel
    finds none of its inputs in any cache.  Run between timed calls,
    outside their events."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)


def gemm_source_hash():
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic():
    """HBM bytes per GEMM launch from committed counter summaries, only if
    they were taken on the current GEMM source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != gemm_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibrate():
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def cpu_baseline(x_u16, w_u16, M, N, K):
    """The oracle as it stands, timed on host cores on a bounded sample of
    the step, extrapolated linearly to the whole step."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    qa_rows = 1024
    qa, sa = oracle.quant_act_1x128(x_u16[:qa_rows])
    t_qa = time.perf_counter() - t0
    t0 = time.perf_counter()
    qb, sb = oracle.quant_w_128x128(w_u16)
    t_qw = time.perf_counter() - t0
    g_rows = min(128, max(16, 6 * threads))
    t0 = time.perf_counter()
    oracle.gemm(qa[:g_rows], sa[:g_rows], qb, sb)
    t_g = time.perf_counter() - t0
    est = t_qa * (M / qa_rows) + t_qw + t_g * (M / g_rows)
    value = 2.0 * M * N * K / est / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"quant_act of {qa_rows}/{M} rows ({t_qa:.2f} s), quant_w of all {N} rows "
                       f"({t_qw:.2f} s), GEMM of {g_rows}/{M} rows x {N} x {K} ({t_g:.2f} s); "
                       f"extrapolated to the full step = {est:.1f} s"),
            "seconds_measured": t_qa + t_qw + t_g}


def time_quant_split(dev, X, W, qx, sx, qw, sw, reps=50, warm=3):
    """The step's quantization as two launches (quant_act, then quant_w)
    and as one (quant_act_w), each call after a cache flush."""
    import torch
    from fp8_fine_grained_fp8bs_amd import fp8bs
    M, K = X.shape
    N = W.shape[0]
    b_qa = M * K * 3 + M * (K // 128) * 4
    b_qw = N * K * 3 + (N // 128) * (K // 128) * 4
    flush = CacheFlush(dev)
    log("rows: step quantization, one and two launches")
    fns = {"qa": lambda: fp8bs.fp8bs_quant_act_1x128(X, qx, sx),
           "qw": lambda: fp8bs.fp8bs_quant_w_128x128(W, qw, sw),
           "qaw": lambda: fp8bs.fp8bs_quant_act_w(X, qx, sx, W, qw, sw)}
    for fn in fns.values():
        for _ in range(warm):
            fn()
    torch.cuda._sleep(QUEUE_FILL_CYCLES)
    kt = KernelTimer()
    for _ in range(reps):
        for name, fn in fns.items():
            flush()
            kt.run(name, fn)
    torch.cuda.synchronize()
    out = {}
    for key, name, b, shape in (("quant_act_1x128", "qa", b_qa, f"[{M}][{K}]"),
                                ("quant_w_128x128", "qw", b_qw, f"[{N}][{K}]"),
                                ("quant_act_w", "qaw", b_qa + b_qw, f"X [{M}][{K}] + W [{N}][{K}]")):
        st = kt.stats_us(name)
        us = st["us_median"]
        out[key] = {"shape": shape, "us": us, "GB/s": b / us / 1e3, "frac_hbm": b / us / 1e3 / HBM_PEAK_GBS,
                    "bytes": b, "us_mean": st["us"], "us_median": us, "us_min": st["us_min"], "calls": st["calls"],
                    "timing": f"after a {FLUSH_BYTES >> 30} GiB cache flush per call"}
    return out


def time_fused(dev, qx, sx, qw, sw, Y, reps=50, warm=3):
    """The up-projection GEMM with its output quantized for the next layer:
    fused into the epilogue, and unfused (BF16 GEMM, then quant_act of Y)."""
    import torch
    from fp8_fine_grained_fp8bs_amd import fp8bs
    M, K = qx.shape
    N = qw.shape[0]
    qy = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sy = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    kt = KernelTimer()
    log("rows: fused output quantization")

    def fused():
        kt.run("fused", lambda: fp8bs.fp8bs_gemm_quant_1x128(qx, sx, qw, sw, fp8bs.BSCALE_BLOCK_128x128, qy, sy))

    def unfused():
        kt.run("u_gemm", lambda: fp8bs.fp8bs_gemm(qx, sx, qw, sw, fp8bs.BSCALE_BLOCK_128x128, Y, fp8bs.OUT_BF16))
        kt.run("u_quant", lambda: fp8bs.fp8bs_quant_act_1x128(Y, qy, sy))

    for fn in (fused, unfused):
        for _ in range(warm):
            fn()
    kt.reset()
    for _ in range(reps):
        fused()
        unfused()
    torch.cuda.synchronize()
    fl = 2.0 * M * N * K
    ms_f = kt.mean_ms("fused")
    ms_u = kt.mean_ms("u_gemm") + kt.mean_ms("u_quant")
    sf, sg, sq = kt.stats_us("fused"), kt.stats_us("u_gemm"), kt.stats_us("u_quant")
    return {
        "gemm_quant_1x128": {"shape": f"M{M} N{N} K{K}, E4M3 out + 1x128 scales", "us": ms_f * 1e3,
                             "us_median": sf["us_median"], "us_min": sf["us_min"],
                             "TFLOP/s": fl / ms_f / 1e9, "frac_fp8_peak": fl / ms_f / 1e9 / FP8_PEAK_TFLOPS,
                             "timing": "alternating with the unfused pair, no flush (each launch streams > 1 GB)"},
        "gemm_bf16_then_quant_act": {"shape": f"M{M} N{N} K{K}, BF16 out, then quant_act of [{M}][{N}]",
                                     "us": ms_u * 1e3, "us_median": sg["us_median"] + sq["us_median"],
                                     "TFLOP/s": fl / ms_u / 1e9,
                                     "frac_fp8_peak": fl / ms_u / 1e9 / FP8_PEAK_TFLOPS,
                                     "quant_act_us": kt.mean_ms("u_quant") * 1e3},
    }


def time_rows(dev, reps=50, warm=3):
    """Re-quantization, wgrad GEMM, weight transpose and input-gradient GEMM, and
    grouped GEMM rows, at their full sizes."""
    import numpy as np
    import torch
    from fp8_fine_grained_fp8bs_amd import fp8bs, synth
    rows = {}
    flush = CacheFlush(dev)
    stats = {}

    def timed(name, fn):
        """Median event time (ms) of `reps` calls, each after a 1 GiB cache
        flush written outside its events; mean, median and min kept."""
        for _ in range(warm):
            fn()
        # keep the GPU busy while the timed calls are queued, so that the
        # host's launch latency (longer than the smallest kernels) never
        # leaves the stream idle between a start event and its kernel
        torch.cuda._sleep(QUEUE_FILL_CYCLES)
        kt = KernelTimer()
        for _ in range(reps):
            flush()
            kt.run(name, fn)
        torch.cuda.synchronize()
        stats[name] = kt.stats_us(name)
        return stats[name]["us_median"] * 1e-3

    # backward wgrad: X 8192x7168, dY 8192x2048
    log("rows: wgrad inputs")
    w = synth.wgrad(with_w=True)
    T, C_in = w["X"].shape
    C_out = w["dY"].shape[1]
    X = bf16_dev(w["X"], dev)
    dY = bf16_dev(w["dY"], dev)
    qx, sx = fp8bs.quant_act_1x128(X)
    qxt = torch.empty((C_in, T), dtype=torch.uint8, device=dev)
    sxt = torch.empty((C_in, T // 128), dtype=torch.float32, device=dev)
    qdt = torch.empty((C_out, T), dtype=torch.uint8, device=dev)
    sdt = torch.empty((C_out, T // 128), dtype=torch.float32, device=dev)
    dW = torch.empty((C_in, C_out), dtype=torch.float32, device=dev)
    ms = timed("requant_fp8", lambda: fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_FP8_1x128, qx, sx, qxt, sxt))
    b = T * C_in * (1 + 1) + T * (C_in // 128) * 4 + C_in * (T // 128) * 4
    rows["requant_T_128x1_fp8"] = {"shape": f"[{T}][{C_in}] -> [{C_in}][{T}]", "us": ms * 1e3,
                                   "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS,
                                   "bytes": b}
    ms = timed("requant_bf16", lambda: fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_BF16, dY, None, qdt, sdt))
    b = T * C_out * (2 + 1) + C_out * (T // 128) * 4
    rows["requant_T_128x1_bf16"] = {"shape": f"[{T}][{C_out}] -> [{C_out}][{T}]", "us": ms * 1e3,
                                    "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS,
                                    "bytes": b}
    # the activations cached in E5M6 instead: encode, then decode for the backward pass
    ye = torch.empty((T, C_in // 2 * 3), dtype=torch.uint8, device=dev)
    xe = torch.empty((T, C_in), dtype=torch.bfloat16, device=dev)
    b = T * C_in * (2 + 1.5)
    ms = timed("e5m6_enc", lambda: fp8bs.fp8bs_encode_e5m6(X, ye))
    rows["encode_e5m6"] = {"shape": f"[{T}][{C_in}]", "us": ms * 1e3, "GB/s": b / ms / 1e6,
                           "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS, "bytes": b}
    ms = timed("e5m6_dec", lambda: fp8bs.fp8bs_decode_e5m6(ye, xe))
    rows["decode_e5m6"] = {"shape": f"[{T}][{C_in}]", "us": ms * 1e3, "GB/s": b / ms / 1e6,
                           "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS, "bytes": b}
    # the weight gradient's 128x1 operand straight from the E5M6 cache (the
    # decode fused into the re-quantization) against decode + BF16 requant
    qet, set_ = torch.empty_like(qxt), torch.empty_like(sxt)
    ms = timed("requant_e5m6", lambda: fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_E5M6, ye, None, qet, set_))
    b = T * C_in * (1.5 + 1) + C_in * (T // 128) * 4
    t_pair = rows["decode_e5m6"]["us"] + rows["requant_T_128x1_bf16"]["us"] * C_in / C_out
    rows["requant_T_128x1_e5m6"] = {"shape": f"[{T}][{C_in}] E5M6 -> [{C_in}][{T}]", "us": ms * 1e3,
                                    "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS,
                                    "bytes": b,
                                    "speedup_vs_decode_then_requant_bf16": t_pair / (ms * 1e3),
                                    "pair_note": "decode row plus the BF16 requant row scaled to these columns"}
    del ye, xe, qet, set_
    ms = timed("wgrad", lambda: fp8bs.fp8bs_gemm(qxt, sxt, qdt, sdt, fp8bs.BSCALE_ROW_1x128, dW, fp8bs.OUT_F32))
    fl = 2.0 * C_in * C_out * T
    rows["gemm_wgrad_row_f32"] = {"shape": f"M{C_in} N{C_out} K{T}", "us": ms * 1e3,
                                  "TFLOP/s": fl / ms / 1e9, "frac_fp8_peak": fl / ms / 1e9 / FP8_PEAK_TFLOPS}

    # backward for the input: dX [T][C_in] = dY W, W [C_out][C_in] quantized in
    # 128x128 blocks and transposed for the K-contiguous GEMM
    log("rows: input-gradient inputs")
    Wd = bf16_dev(w["W"], dev)
    qdy, sdy = fp8bs.quant_act_1x128(dY)
    qw, sw = fp8bs.quant_w_128x128(Wd)
    qwt = torch.empty((C_in, C_out), dtype=torch.uint8, device=dev)
    swt = torch.empty((C_in // 128, C_out // 128), dtype=torch.float32, device=dev)
    dX = torch.empty((T, C_in), dtype=torch.bfloat16, device=dev)
    ms = timed("transpose_w", lambda: fp8bs.fp8bs_transpose_w_128x128(qw, sw, qwt, swt))
    b = C_out * C_in * 2 + 2 * (C_out // 128) * (C_in // 128) * 4
    rows["transpose_w_128x128"] = {"shape": f"[{C_out}][{C_in}] -> [{C_in}][{C_out}]", "us": ms * 1e3,
                                   "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS,
                                   "bytes": b}
    ms = timed("dgrad", lambda: fp8bs.fp8bs_gemm(qdy, sdy, qwt, swt, fp8bs.BSCALE_BLOCK_128x128, dX, fp8bs.OUT_BF16))
    fl = 2.0 * T * C_in * C_out
    rows["gemm_dgrad_bf16"] = {"shape": f"M{T} N{C_in} K{C_out}", "us": ms * 1e3,
                               "TFLOP/s": fl / ms / 1e9, "frac_fp8_peak": fl / ms / 1e9 / FP8_PEAK_TFLOPS}
    del X, dY, qx, sx, qxt, sxt, qdt, sdt, dW, w, Wd, qdy, sdy, qw, sw, qwt, swt, dX

    # grouped MoE (8 experts, 16384 tokens, Zipf counts)
    log("rows: moe inputs")
    m = synth.moe()
    off = torch.from_numpy(m["offsets"]).to(dev)
    Ttok = int(m["offsets"][-1])
    for tag, an, wn in (("up", "A_up", "W_up"), ("down", "A_down", "W_down")):
        A = bf16_dev(m[an], dev)
        E, N, K = m[wn].shape
        Wt = bf16_dev(m[wn].reshape(E * N, K), dev)
        qa = torch.empty((Ttok, K), dtype=torch.uint8, device=dev)
        sa = torch.empty((Ttok, K // 128), dtype=torch.float32, device=dev)
        qw = torch.empty((E * N, K), dtype=torch.uint8, device=dev)
        sw = torch.empty((E * N // 128, K // 128), dtype=torch.float32, device=dev)
        out = torch.empty((Ttok, N), dtype=torch.bfloat16, device=dev)
        ms = timed(f"qa_{tag}", lambda: fp8bs.fp8bs_quant_act_1x128(A, qa, sa))
        b = Ttok * K * 3 + Ttok * (K // 128) * 4
        rows[f"quant_act_moe_{tag}"] = {"shape": f"[{Ttok}][{K}]", "us": ms * 1e3, "GB/s": b / ms / 1e6,
                                        "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS, "bytes": b}
        ms = timed(f"qw_{tag}", lambda: fp8bs.fp8bs_quant_w_128x128(Wt, qw, sw))
        b = E * N * K * 3 + (E * N // 128) * (K // 128) * 4
        rows[f"quant_w_moe_{tag}"] = {"shape": f"{E}x[{N}][{K}]", "us": ms * 1e3, "GB/s": b / ms / 1e6,
                                      "frac_hbm": b / ms / 1e6 / HBM_PEAK_GBS, "bytes": b}
        qw3, sw3 = qw.view(E, N, K), sw.view(E, N // 128, K // 128)
        ms = timed(f"grouped_{tag}", lambda: fp8bs.fp8bs_grouped_gemm(qa, sa, qw3, sw3, off, out, fp8bs.OUT_BF16))
        fl = 2.0 * Ttok * N * K
        rows[f"grouped_gemm_{tag}"] = {"shape": f"E{E} sumM{Ttok} N{N} K{K}", "us": ms * 1e3,
                                       "TFLOP/s": fl / ms / 1e9, "frac_fp8_peak": fl / ms / 1e9 / FP8_PEAK_TFLOPS}
        del A, Wt, qa, sa, qw, sw, out
    # SwiGLU of the MoE up-projection's halves, quantized 1x128 for the down
    # projection (16384 tokens x 2048), fused against SwiGLU to BF16 then
    # quant_act
    log("rows: swiglu quantization")
    gen = torch.Generator(device=dev).manual_seed(7)
    Ttok, I = 16384, 2048
    gu = (torch.randn((Ttok, 2 * I), generator=gen, device=dev) * 1.5).to(torch.bfloat16)
    gs, us = gu[:, :I], gu[:, I:]
    qs = torch.empty((Ttok, I), dtype=torch.uint8, device=dev)
    ss = torch.empty((Ttok, I // 128), dtype=torch.float32, device=dev)
    hs = torch.empty((Ttok, I), dtype=torch.bfloat16, device=dev)
    t_f = timed("swiglu_fused", lambda: fp8bs.fp8bs_swiglu_quant_1x128(gs, us, qs, ss, None))

    def swiglu_unfused():
        fp8bs.fp8bs_swiglu_quant_1x128(gs, us, None, None, hs)
        fp8bs.fp8bs_quant_act_1x128(hs, qs, ss)
    t_u = timed("swiglu_unfused", swiglu_unfused)
    n_el = Ttok * I
    b_f = n_el * (2 + 2 + 1) + Ttok * (I // 128) * 4
    rows["swiglu_quant_1x128"] = {"shape": f"g, u [{Ttok}][{I}] (halves of [{Ttok}][{2 * I}])",
                                  "us": t_f * 1e3, "GB/s": b_f / t_f / 1e6,
                                  "frac_hbm": b_f / t_f / 1e6 / HBM_PEAK_GBS, "bytes": b_f,
                                  "us_unfused_bf16_h_then_quant_act": t_u * 1e3,
                                  "speedup_vs_unfused": t_u / t_f}
    del gu, gs, us, qs, ss, hs

    # BF16 A quantized inside the GEMM (the FP8 activation never crosses HBM)
    # against quant_act + gemm, on the low-rank projections 7168 -> 576 and
    # 7168 -> 1536 of 4096 tokens (small N: A is re-quantized per 256-column
    # tile of B, 3 and 6 times)
    log("rows: bf16-A projections")
    M, K = 4096, 7168
    rng = np.random.default_rng(5)
    Xp = bf16_dev(synth.mlp_up(T=M, K=K, N=1536, seed=1, with_w=False)["X"], dev)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    for N in (576, 1536):
        Wp = bf16_dev(synth.bf16_bits((rng.standard_normal((N, K)) * 0.006).astype(np.float32)), dev)
        qw, sw = fp8bs.quant_w_128x128(Wp)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fl = 2.0 * M * N * K
        t_q = timed(f"proj{N}_qa", lambda: fp8bs.fp8bs_quant_act_1x128(Xp, qa, sa))
        t_g = timed(f"proj{N}_gemm", lambda: fp8bs.fp8bs_gemm(qa, sa, qw, sw, fp8bs.BSCALE_BLOCK_128x128, out,
                                                               fp8bs.OUT_BF16))

        def pair():
            fp8bs.fp8bs_quant_act_1x128(Xp, qa, sa)
            fp8bs.fp8bs_gemm(qa, sa, qw, sw, fp8bs.BSCALE_BLOCK_128x128, out, fp8bs.OUT_BF16)
        t_p = timed(f"proj{N}_pair", pair)
        t_a = timed(f"proj{N}_bf16a", lambda: fp8bs.fp8bs_gemm_bf16a(Xp, None, None, qw, sw, out, fp8bs.OUT_BF16))
        t_c = timed(f"proj{N}_bf16a_codes", lambda: fp8bs.fp8bs_gemm_bf16a(Xp, qa, sa, qw, sw, out,
                                                                            fp8bs.OUT_BF16))
        rows[f"bf16a_projection_{N}"] = {
            "shape": f"M{M} N{N} K{K}",
            "us_quant_act": t_q * 1e3, "us_gemm": t_g * 1e3, "us_quant_act_then_gemm": t_p * 1e3,
            "us_gemm_bf16a": t_a * 1e3, "us_gemm_bf16a_with_codes": t_c * 1e3,
            "speedup_vs_pair": t_p / t_a, "speedup_with_codes_vs_pair": t_p / t_c,
            "TFLOP/s_gemm_bf16a": fl / t_a / 1e9, "TFLOP/s_pair": fl / t_p / 1e9,
            "timing": f"medians, each call after a {FLUSH_BYTES >> 30} GiB cache flush"}
        del Wp, qw, sw, out
    del Xp, qa, sa
    # every row: median as "us" (the rates above), plus mean and min, all
    # measured after a cache flush
    timer_of = {"requant_T_128x1_fp8": "requant_fp8", "requant_T_128x1_bf16": "requant_bf16",
                "encode_e5m6": "e5m6_enc", "decode_e5m6": "e5m6_dec", "requant_T_128x1_e5m6": "requant_e5m6",
                "gemm_wgrad_row_f32": "wgrad",
                "transpose_w_128x128": "transpose_w", "gemm_dgrad_bf16": "dgrad",
                "swiglu_quant_1x128": "swiglu_fused"}
    for tag in ("up", "down"):
        timer_of.update({f"quant_act_moe_{tag}": f"qa_{tag}", f"quant_w_moe_{tag}": f"qw_{tag}",
                         f"grouped_gemm_{tag}": f"grouped_{tag}"})
    for key, tname in timer_of.items():
        st = stats[tname]
        rows[key].update({"us_mean": st["us"], "us_median": st["us_median"], "us_min": st["us_min"],
                          "calls": st["calls"], "timing": f"after a {FLUSH_BYTES >> 30} GiB cache flush per call"})
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from fp8_fine_grained_fp8bs_amd import fp8bs, synth

    if args.copy_calibrate:
        copy_calibrate()
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    fp8bs.load()

    M, N, K = 4096, 18432, 7168
    log("inputs: mlp_up X 4096x7168, W 18432x7168")
    d = synth.mlp_up(T=M, K=K, N=N)
    X = bf16_dev(d["X"], dev)
    W = bf16_dev(d["W"], dev)
    qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sx = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    if args.profile_kernel:
        calls = {
            "quant_act": lambda: fp8bs.fp8bs_quant_act_1x128(X, qx, sx),
            "quant_w": lambda: fp8bs.fp8bs_quant_w_128x128(W, qw, sw),
            "quant_act_w": lambda: fp8bs.fp8bs_quant_act_w(X, qx, sx, W, qw, sw),
            "gemm": lambda: fp8bs.fp8bs_gemm(qx, sx, qw, sw, fp8bs.BSCALE_BLOCK_128x128, Y, fp8bs.OUT_BF16),
        }
        if args.profile_kernel == "gemm":
            fp8bs.fp8bs_quant_act_w(X, qx, sx, W, qw, sw)
        for _ in range(args.steps):
            calls[args.profile_kernel]()
        torch.cuda.synchronize()
        log(f"ran {args.profile_kernel} {args.steps} times")
        return

    kt = ChainTimer()

    def step():
        kt.run("quant_act_w", lambda: fp8bs.fp8bs_quant_act_w(X, qx, sx, W, qw, sw))
        kt.run("gemm", lambda: fp8bs.fp8bs_gemm(qx, sx, qw, sw, fp8bs.BSCALE_BLOCK_128x128, Y, fp8bs.OUT_BF16))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kt.reset()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    kt.close()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    assert torch.isfinite(Y.float()).all(), "non-finite GEMM output"

    ms_q, ms_g = kt.mean_ms("quant_act_w"), kt.mean_ms("gemm")
    flop = 2.0 * M * N * K
    b_qa = M * K * 3 + M * (K // 128) * 4
    b_qw = N * K * 3 + (N // 128) * (K // 128) * 4
    b_q = b_qa + b_qw
    gemm_tflops = flop / ms_g / 1e9
    traffic = read_traffic()
    kernels = {
        "quant_act_w": {"shape": f"X [{M}][{K}] 1x128 + W [{N}][{K}] 128x128, one launch", "us": ms_q * 1e3,
                        "GB/s": b_q / ms_q / 1e6, "frac_hbm": b_q / ms_q / 1e6 / HBM_PEAK_GBS, "bytes": b_q},
        "gemm_bf16_block": {"shape": f"M{M} N{N} K{K}", "us": ms_g * 1e3, "TFLOP/s": gemm_tflops,
                            "frac_fp8_peak": gemm_tflops / FP8_PEAK_TFLOPS},
    }
    for key, tname in (("quant_act_w", "quant_act_w"), ("gemm_bf16_block", "gemm")):
        st = kt.stats_us(tname)
        kernels[key].update({"us_median": st["us_median"], "us_min": st["us_min"],
                             "timing": "inside the step (the other kernels of the step stream "
                                       "> 500 MB between two calls of one kernel)"})
    result = {
        "metric": "block-scaled FP8 GEMM TFLOP/s (%FP8 peak) at K=7168; quantize GB/s (%HBM)",
        "value": flop / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": "dense MLP up-projection forward: 1x128 quantization of X[4096][7168] and "
                               "128x128 quantization of W[18432][7168] (one launch) + block-scaled FP8 GEMM "
                               "Y=X*W^T (BF16 out)",
                   "M": M, "N": N, "K": K, "inputs": "bf16 X ~N(0,1) with 1% Student-t(3) channels, "
                                                    "W ~N(0,0.006), seed 0"},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_tflops / FP8_PEAK_TFLOPS, "traffic": traffic,
                     "kernel": "gemm_kernel<bf16 out, block scales>", "flop_per_launch": flop},
        "kernels": kernels,
    }
    if args.rows == "all":
        rows = time_quant_split(dev, X, W, qx, sx, qw, sw)
        rows.update(time_fused(dev, qx, sx, qw, sw, Y))
        rows.update(time_rows(dev))
        result["rows"] = rows
    if args.cpu_baseline == "on":
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(d["X"], d["W"], M, N, K)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
