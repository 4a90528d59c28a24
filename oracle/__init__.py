"""CPU oracle for fine-grained FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
CPU-baseline leg of the benchmark are the only callers.  The GPU library
(``fp8_fine_grained_fp8bs_amd``) never imports this package, and this package
never imports the GPU library: the two share no code.

The arithmetic lives in ``fp8bs_oracle.c`` (plain C, binary64 sums, binary32
scales); this module only builds it, loads it with ctypes and marshals numpy
arrays.  Each wrapper names the passage of the DeepSeek-V3 report excerpts
(five web pages, cited as [p1] = xn--9g3bo1gtkw0l8ubf92bgle.kr post
wr_id=32373, [p2] = why-be.why-be.co.kr post wr_id=73620, [p3] =
xn--9g3bo1gtkw0l8ubf92bgle.kr post wr_id=113503, [p4] = bestpmk.kr post
wr_id=299512, with a paragraph number) that it follows.

Parity status: every function below is pinned by ``tests/test_oracle_*.py``.
The limited-precision accumulation model (:func:`gemm_unpromoted`, context
only) is pinned by hand-worked cases (``tests/golden/unpromoted_hand.json``)
that fix its window, truncation direction, chunk boundary, carried sum and
scale placement, and by the exact sum it reduces to with a wide window.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8bs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_fp8bs.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle_fp8bs.so`` (gcc, -O2,
    no fast-math, no FMA contraction, OpenMP for independent rows only)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    F32 = ctypes.c_float
    sigs = {
        "orc_num_threads": (ctypes.c_int, []),
        "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_double]),
        "orc_bf16_value": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_bf16_round": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_quant_act_1x128": (None, [P, I64, I64, P, P]),
        "orc_quant_act_1x128_f32": (None, [P, I64, I64, P, P]),
        "orc_quant_w_128x128": (None, [P, I64, I64, P, P]),
        "orc_swiglu_quant_1x128": (None, [P, P, I64, I64, P, P, P, P]),
        "orc_requant_T_128x1": (None, [ctypes.c_int, P, P, I64, I64, P, P]),
        "orc_gemm": (None, [P, P, P, P, ctypes.c_int, I64, I64, I64, P]),
        "orc_gemm_entries": (None, [P, P, P, P, ctypes.c_int, I64, P, P, I64, P]),
        "orc_grouped_gemm": (None, [P, P, P, P, P, I32, I64, I64, P]),
        "orc_grouped_gemm_entries": (None, [P, P, P, P, P, I32, I64, I64, P, P, I64, P]),
        "orc_round_to_bf16": (None, [P, I64, P]),
        "orc_gemm_bf16_f64": (None, [P, P, I64, I64, I64, P]),
        "orc_gemm_bf16_f32acc": (None, [P, P, I64, I64, I64, P]),
        "orc_gemm_unpromoted": (None, [P, F32, P, F32, I64, I64, I64, ctypes.c_int, ctypes.c_int, P]),
        "orc_quant_per_tensor": (None, [P, I64, P, P]),
        "orc_e5m6_value": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_e5m6_encode": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_encode_e5m6": (None, [P, I64, I64, P]),
        "orc_decode_e5m6": (None, [P, I64, I64, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle expects C-contiguous arrays"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 inputs are passed as uint16 bit patterns"
    return a


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8
    return a


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


# --------------------------------------------------------------------------
# scalar codecs
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN code (NaN for 0x7F / 0xFF)."""
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(y: float) -> int:
    """Nearest E4M3 code of a finite value, ties to even mantissa, |y| > 448
    saturates to 448; -0 keeps its sign."""
    return int(_load().orc_e4m3_encode(float(y)))


def e4m3_table() -> np.ndarray:
    """float64 values of all 256 codes (index = code)."""
    lib = _load()
    return np.array([lib.orc_e4m3_value(c) for c in range(256)], dtype=np.float64)


def bf16_value(b: int) -> float:
    return _load().orc_bf16_value(int(b))


def bf16_round(v: float) -> int:
    """binary64 -> bf16 bits, nearest-even, one rounding."""
    return int(_load().orc_bf16_round(float(v)))


def round_to_bf16(d: np.ndarray) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.float64)
    out = np.empty(d.shape, dtype=np.uint16)
    _load().orc_round_to_bf16(_p(d), d.size, _p(out))
    return out


# --------------------------------------------------------------------------
# quantization ([p1] para 3)
# --------------------------------------------------------------------------

def quant_act_1x128(x_bf16: np.ndarray):
    """1x128 activation tiles along K: returns (codes [M][K] u8, scales
    [M][K/128] f32).  [p1] para 3 (online amax per 1x128 tile), [p1] para 2
    (scales per group along K)."""
    x = _u16(x_bf16)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.float32)
    _load().orc_quant_act_1x128(_p(x), M, K, _p(q), _p(s))
    return q, s


def quant_act_1x128_f32(x_f32: np.ndarray):
    """Same tiles for an FP32 input (used to state the backward
    re-quantization as a composition)."""
    x = _f32(x_f32)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.float32)
    _load().orc_quant_act_1x128_f32(_p(x), M, K, _p(q), _p(s))
    return q, s


def swiglu_quant_1x128(g_bf16: np.ndarray, u_bf16: np.ndarray):
    """SwiGLU of the cached gate and up halves ([p1] para 4, [p4] para 3:
    the SwiGLU inputs are cached and its output recomputed), h = silu(g) u
    in binary64 rounded once to binary32, then 1x128 tiles along I as in
    quant_act_1x128_f32 ([p1] para 3).  g, u bf16 [T][I] -> (codes [T][I],
    scales [T][I/128], h binary32 [T][I], h bf16 bits [T][I] rounded once
    from binary64)."""
    g = _u16(g_bf16)
    u = _u16(u_bf16)
    assert g.shape == u.shape
    T, I = g.shape
    assert I % 128 == 0
    q = np.empty((T, I), np.uint8)
    s = np.empty((T, I // 128), np.float32)
    h32 = np.empty((T, I), np.float32)
    h16 = np.empty((T, I), np.uint16)
    _load().orc_swiglu_quant_1x128(_p(g), _p(u), T, I, _p(q), _p(s), _p(h32), _p(h16))
    return q, s, h32, h16


def quant_w_128x128(w_bf16: np.ndarray):
    """128x128 weight blocks: returns (codes [N][K], scales [ceil(N/128)][K/128]).
    [p1] para 3 (online amax per 128x128 weight block)."""
    w = _u16(w_bf16)
    N, K = w.shape
    assert K % 128 == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty(((N + 127) // 128, K // 128), np.float32)
    _load().orc_quant_w_128x128(_p(w), N, K, _p(q), _p(s))
    return q, s


def requant_T_128x1_fp8(q_in: np.ndarray, s_in: np.ndarray):
    """Backward 1x128 -> 128x1 re-quantization of cached FP8 activations
    ([p1] para 3, [p1] para 4: activations cached in FP8 for the Linear
    backward).  q_in [T][C], s_in [T][C/128] -> (q_out [C][T],
    s_out [C][ceil(T/128)])."""
    q = _u8(q_in)
    s = _f32(s_in)
    T, C = q.shape
    assert C % 128 == 0 and s.shape == (T, C // 128)
    qo = np.empty((C, T), np.uint8)
    so = np.empty((C, (T + 127) // 128), np.float32)
    _load().orc_requant_T_128x1(0, _p(q), _p(s), T, C, _p(qo), _p(so))
    return qo, so


def requant_T_128x1_bf16(x_bf16: np.ndarray):
    """128x1 quantization of a bf16 [T][C] tensor along T, written
    transposed: (q_out [C][T], s_out [C][ceil(T/128)])."""
    x = _u16(x_bf16)
    T, C = x.shape
    assert C % 128 == 0
    qo = np.empty((C, T), np.uint8)
    so = np.empty((C, (T + 127) // 128), np.float32)
    dummy = np.zeros(1, np.float32)
    _load().orc_requant_T_128x1(1, _p(x), _p(dummy), T, C, _p(qo), _p(so))
    return qo, so


def requant_T_128x1_e5m6(y_packed: np.ndarray, C: int):
    """128x1 re-quantization of E5M6-cached activations ([p1] para 3: E5M6
    for some activations cached for the backward pass): the exact E5M6
    decode followed by the bf16-source re-quantization, composed as
    written (decode_e5m6, then requant_T_128x1_bf16)."""
    return requant_T_128x1_bf16(decode_e5m6(y_packed, C))


def transpose_w_128x128(q_in: np.ndarray, s_in: np.ndarray):
    """Quantized W^T for the backward pass for the input ([p3] para 4 splits
    the backward pass into the input and the weight parts; blocks of [p1]
    para 3): q [N][K], s [N/128][K/128] -> (q^T [K][N], s^T [K/128][N/128]).
    A 128x128 block's max-abs does not depend on its orientation, so these
    are the codes and scales quant_w_128x128 gives for W^T (pinned in the
    tests).  A pure data movement: no arithmetic."""
    q = _u8(q_in)
    s = _f32(s_in)
    N, K = q.shape
    assert N % 128 == 0 and K % 128 == 0 and s.shape == (N // 128, K // 128)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


# --------------------------------------------------------------------------
# E5M6 cached-activation format ([p1] para 3)
# --------------------------------------------------------------------------

def e5m6_value(code: int) -> float:
    return float(_load().orc_e5m6_value(int(code)))


def e5m6_encode(y: float) -> int:
    return int(_load().orc_e5m6_encode(float(y)))


def encode_e5m6(x_bf16: np.ndarray) -> np.ndarray:
    """bf16 [T][C] -> packed E5M6 [T][1.5 C] bytes (value i of a row in bits
    12 i .. 12 i + 11, little-endian); nearest-even, IEEE overflow."""
    x = _u16(x_bf16)
    T, C = x.shape
    assert C % 2 == 0
    y = np.empty((T, C // 2 * 3), np.uint8)
    _load().orc_encode_e5m6(_p(x), T, C, _p(y))
    return y


def decode_e5m6(y_packed: np.ndarray, C: int) -> np.ndarray:
    """packed E5M6 [T][1.5 C] -> bf16 [T][C] bit patterns (exact)."""
    y = _u8(y_packed)
    T = y.shape[0]
    assert y.shape[1] == C // 2 * 3
    x = np.empty((T, C), np.uint16)
    _load().orc_decode_e5m6(_p(y), T, C, _p(x))
    return x


def quant_per_tensor(x_bf16: np.ndarray):
    """Per-tensor scaling, the practice [p1] para 4 contrasts with."""
    x = _u16(x_bf16)
    q = np.empty(x.shape, np.uint8)
    s = np.zeros(1, np.float32)
    _load().orc_quant_per_tensor(_p(x), x.size, _p(q), _p(s))
    return q, float(s[0])


# --------------------------------------------------------------------------
# GEMM ([p1] para 2, [p4] para 4)
# --------------------------------------------------------------------------

BSCALE_BLOCK = 0
BSCALE_ROW = 1


def gemm(a, sa, b, sb, bmode: int = BSCALE_BLOCK) -> np.ndarray:
    """D = A * B^T in binary64 from the dequantized operands; [M][N]."""
    a = _u8(a); b = _u8(b); sa = _f32(sa); sb = _f32(sb)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K and K % 128 == 0
    d = np.empty((M, N), np.float64)
    _load().orc_gemm(_p(a), _p(sa), _p(b), _p(sb), int(bmode), M, N, K, _p(d))
    return d


def gemm_quant_1x128(a, sa, b, sb, bmode: int = BSCALE_BLOCK):
    """The GEMM with the next layer's activation quantization fused into its
    output ([p2] para 1: quantizing separately costs a BF16 write and read
    back): D = A * B^T rounded once to FP32, then 1x128 tiles along N
    quantized as quant_act_1x128 does ([p1] para 3).  Returns (codes [M][N],
    scales [M][N/128])."""
    d = gemm(a, sa, b, sb, bmode)
    assert d.shape[1] % 128 == 0
    return quant_act_1x128_f32(d.astype(np.float32))


def gemm_entries(a, sa, b, sb, mi, ni, bmode: int = BSCALE_BLOCK) -> np.ndarray:
    a = _u8(a); b = _u8(b); sa = _f32(sa); sb = _f32(sb)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    K = a.shape[1]
    d = np.empty(mi.shape, np.float64)
    _load().orc_gemm_entries(_p(a), _p(sa), _p(b), _p(sb), int(bmode), K,
                             _p(mi), _p(ni), mi.size, _p(d))
    return d


def grouped_gemm(a, sa, b, sb, offsets) -> np.ndarray:
    """Per-expert block-scaled GEMM over ragged row ranges; [offsets[E]][N]."""
    a = _u8(a); b = _u8(b); sa = _f32(sa); sb = _f32(sb)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    E = off.size - 1
    N, K = b.shape[1], b.shape[2]
    d = np.empty((int(off[-1]), N), np.float64)
    _load().orc_grouped_gemm(_p(a), _p(sa), _p(b), _p(sb), _p(off), E, N, K, _p(d))
    return d


def grouped_gemm_entries(a, sa, b, sb, offsets, mi, ni) -> np.ndarray:
    a = _u8(a); b = _u8(b); sa = _f32(sa); sb = _f32(sb)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    E = off.size - 1
    N, K = b.shape[1], b.shape[2]
    d = np.empty(mi.shape, np.float64)
    _load().orc_grouped_gemm_entries(_p(a), _p(sa), _p(b), _p(sb), _p(off), E,
                                     N, K, _p(mi), _p(ni), mi.size, _p(d))
    return d


# --------------------------------------------------------------------------
# accuracy-probe references
# --------------------------------------------------------------------------

def gemm_bf16_f64(x, w) -> np.ndarray:
    """Unquantized X * W^T of the bf16 inputs in binary64."""
    x = _u16(x); w = _u16(w)
    M, K = x.shape
    N = w.shape[0]
    d = np.empty((M, N), np.float64)
    _load().orc_gemm_bf16_f64(_p(x), _p(w), M, N, K, _p(d))
    return d


def gemm_bf16_f32acc(x, w) -> np.ndarray:
    """BF16 GEMM with a binary32 accumulator (k ascending), binary32 result."""
    x = _u16(x); w = _u16(w)
    M, K = x.shape
    N = w.shape[0]
    d = np.empty((M, N), np.float32)
    _load().orc_gemm_bf16_f32acc(_p(x), _p(w), M, N, K, _p(d))
    return d


def gemm_unpromoted(a, sa_t: float, b, sb_t: float, chunk: int = 32,
                    bits: int = 14) -> np.ndarray:
    """Limited-precision accumulation model without promotion ([p1] para 3,
    [p2] para 3).  Context only (not the GPU path's reference); pinned by
    hand-worked cases."""
    a = _u8(a); b = _u8(b)
    M, K = a.shape
    N = b.shape[0]
    d = np.empty((M, N), np.float64)
    _load().orc_gemm_unpromoted(_p(a), float(sa_t), _p(b), float(sb_t), M, N, K,
                                int(chunk), int(bits), _p(d))
    return d
