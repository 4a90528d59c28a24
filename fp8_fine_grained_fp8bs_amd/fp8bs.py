"""Thin ctypes binding of libfp8bs (C ABI declared in ``include/fp8bs.h``).

Each ``fp8bs_*`` function has the name and argument order of the C entry
point; tensors (PyTorch, on the GPU) stand for the device pointers and their
row strides are taken from the tensor.  Nothing here computes: every step
runs in the library's HIP kernels.  The ``quant_*`` / ``gemm`` helpers at the
bottom only allocate output tensors and call the entry points.

The library must have been built (``python -m fp8_fine_grained_fp8bs_amd.build``);
loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8bs.so")

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED_SHAPE = 2
ERR_MISALIGNED = 3
ERR_NO_DEVICE = 4
ERR_LAUNCH = 5

OUT_BF16 = 0
OUT_F32 = 1
BSCALE_BLOCK_128x128 = 0
BSCALE_ROW_1x128 = 1
SRC_FP8_1x128 = 0
SRC_BF16 = 1
SRC_E5M6 = 2

ENTRY_POINTS = ("fp8bs_quant_act_1x128", "fp8bs_quant_w_128x128", "fp8bs_quant_act_w",
                "fp8bs_swiglu_quant_1x128",
                "fp8bs_quant_per_tensor",
                "fp8bs_cast_e4m3",
                "fp8bs_encode_e5m6", "fp8bs_decode_e5m6", "fp8bs_requant_T_128x1",
                "fp8bs_transpose_w_128x128", "fp8bs_gemm", "fp8bs_gemm_quant_1x128", "fp8bs_gemm_bf16a",
                "fp8bs_grouped_gemm",
                "fp8bs_status_string", "fp8bs_version")

_lib = None
_lib_path = LIB_PATH


def use_library(path: str) -> str:
    """Route every later call through another build of the library (the
    tests use the LDS-poisoning debug build, ``libfp8bs_poison.so``);
    returns the path in use before."""
    global _lib, _lib_path
    prev = _lib_path
    _lib_path, _lib = path, None
    return prev


class Fp8bsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libfp8bs.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_lib_path):
        raise RuntimeError(f"{_lib_path} is missing: build it with "
                           "`python -m fp8_fine_grained_fp8bs_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_lib_path)
    P, I64, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    sigs = {
        "fp8bs_quant_act_1x128": [P, I64, I64, I64, P, I64, P, I64, P],
        "fp8bs_swiglu_quant_1x128": [P, I64, P, I64, I64, I64, P, I64, P, I64, P, I64, P],
        "fp8bs_quant_w_128x128": [P, I64, I64, I64, P, I64, P, I64, P],
        "fp8bs_quant_act_w": [P, I64, I64, P, I64, P, I64, P, I64, I64, P, I64, P, I64, I64, P],
        "fp8bs_quant_per_tensor": [P, I64, P, P, P],
        "fp8bs_cast_e4m3": [P, I64, P, P],
        "fp8bs_encode_e5m6": [P, I64, I64, I64, P, I64, P],
        "fp8bs_decode_e5m6": [P, I64, I64, I64, P, I64, P],
        "fp8bs_requant_T_128x1": [I, P, P, I64, I64, I64, I64, P, I64, P, I64, P],
        "fp8bs_transpose_w_128x128": [P, I64, I64, I64, P, I64, P, I64, P, I64, P],
        "fp8bs_gemm": [P, P, I64, I64, P, P, I64, I64, I, P, I64, I, I64, I64, I64, P],
        "fp8bs_gemm_quant_1x128": [P, P, I64, I64, P, P, I64, I64, I, P, I64, P, I64, I64, I64, I64, P],
        "fp8bs_grouped_gemm": [P, P, I64, P, P, P, I32, I64, P, I, I64, I64, P],
        "fp8bs_gemm_bf16a": [P, I64, P, I64, P, I64, P, P, I64, I64, P, I64, I, I64, I64, I64, P],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fp8bs_status_string.argtypes = [ctypes.c_int]
    lib.fp8bs_status_string.restype = ctypes.c_char_p
    lib.fp8bs_version.argtypes = []
    lib.fp8bs_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(st: int) -> str:
    return load().fp8bs_status_string(int(st)).decode()


def _ptr(t):
    """Device pointer of a GPU tensor (or an int address, or None for NULL).
    A host tensor is refused here: its address would reach the kernels as a
    device pointer."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libfp8bs takes device tensors; got a tensor on " + str(t.device))
    return t.data_ptr()


def _ld(t):
    """Row stride (elements) of a row-major 2-D tensor view."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"expected a 2-D tensor with contiguous rows, got shape {tuple(t.shape)} "
                         f"strides {tuple(t.stride())}")
    return t.stride(0)


_CODES = ("uint8", "float8_e4m3fn")


def _check(t, what, shape, dtypes, contiguous=False):
    """Refuse a tensor whose shape or dtype does not fit what the kernels
    will read or write (a short output would be written past its end).
    shape entries: an int (exact), (">=", n) (at least n) or None (any)."""
    if t is None:
        raise ValueError(f"{what}: missing tensor")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != len(shape):
        raise ValueError(f"{what}: {t.dim()}-D tensor, expected {len(shape)}-D")
    for i, want in enumerate(shape):
        got = t.shape[i]
        if want is None:
            continue
        if isinstance(want, tuple):
            if got < want[1]:
                raise ValueError(f"{what}: dimension {i} is {got}, needs at least {want[1]}")
        elif got != want:
            raise ValueError(f"{what}: dimension {i} is {got}, expected {want}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if t.dim() == 2:
        _ld(t)


def _groups(K):
    return K // 128


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st != OK:
        raise Fp8bsError(st, name)


# ---------------------------------------------------------------------------
# entry points (same names and argument order as the C ABI)
# ---------------------------------------------------------------------------

def fp8bs_quant_act_1x128(x, q, s, stream=None):
    """x bf16 [M][K] -> q u8 [M][K], s f32 [M][K/128]."""
    M, K = x.shape
    _check(x, "x", (M, K), ("bfloat16",))
    _check(q, "q", (M, K), _CODES)
    _check(s, "s", (M, (">=", _groups(K))), ("float32",))
    _call("fp8bs_quant_act_1x128", _ptr(x), M, K, _ld(x), _ptr(q), _ld(q), _ptr(s), _ld(s),
          _stream(stream))


def fp8bs_quant_w_128x128(w, q, s, stream=None):
    """w bf16 [N][K] -> q u8 [N][K], s f32 [ceil(N/128)][K/128]."""
    N, K = w.shape
    _check(w, "w", (N, K), ("bfloat16",))
    _check(q, "q", (N, K), _CODES)
    _check(s, "s", ((N + 127) // 128, (">=", _groups(K))), ("float32",))
    _call("fp8bs_quant_w_128x128", _ptr(w), N, K, _ld(w), _ptr(q), _ld(q), _ptr(s), _ld(s),
          _stream(stream))


def fp8bs_quant_per_tensor(x, q, s, stream=None):
    """x bf16 (contiguous, n % 128 == 0) -> q u8 (same shape), s f32 [1]."""
    if not (x.is_contiguous() and q.is_contiguous()) or q.numel() != x.numel():
        raise ValueError("x and q must be contiguous with the same number of elements")
    if str(x.dtype) != "torch.bfloat16" or str(q.dtype).replace("torch.", "") not in _CODES:
        raise ValueError("x must be bfloat16 and q uint8 codes")
    if s is None or s.numel() < 1 or str(s.dtype) != "torch.float32":
        raise ValueError("s must hold one float32")
    _call("fp8bs_quant_per_tensor", _ptr(x), x.numel(), _ptr(q), _ptr(s), _stream(stream))


def fp8bs_cast_e4m3(x, q, stream=None):
    """x f32 (contiguous) -> q u8 (same number of elements): nearest-even
    E4M3 codes, saturated to +-448."""
    if not (x.is_contiguous() and q.is_contiguous()) or q.numel() != x.numel():
        raise ValueError("x and q must be contiguous with the same number of elements")
    if str(x.dtype) != "torch.float32" or str(q.dtype).replace("torch.", "") not in _CODES:
        raise ValueError("x must be float32 and q uint8 codes")
    _call("fp8bs_cast_e4m3", _ptr(x), x.numel(), _ptr(q), _stream(stream))


def fp8bs_encode_e5m6(x, y, stream=None):
    """bf16 x [T][C] -> packed E5M6 y u8 [T][>= 1.5 C]."""
    T, C = x.shape
    _check(x, "x", (T, C), ("bfloat16",))
    _check(y, "y", (T, (">=", (3 * C + 1) // 2)), ("uint8",))
    _call("fp8bs_encode_e5m6", _ptr(x), T, C, _ld(x), _ptr(y), _ld(y), _stream(stream))


def fp8bs_decode_e5m6(y, x, stream=None):
    """packed E5M6 y u8 [T][>= 1.5 C] -> bf16 x [T][C] (exact)."""
    T, C = x.shape
    _check(x, "x", (T, C), ("bfloat16",))
    _check(y, "y", (T, (">=", (3 * C + 1) // 2)), ("uint8",))
    _call("fp8bs_decode_e5m6", _ptr(y), T, C, _ld(y), _ptr(x), _ld(x), _stream(stream))


def fp8bs_requant_T_128x1(src, x, s_in, q_out, s_out, stream=None):
    """x [T][C] (codes with s_in [T][C/128], or bf16), or packed E5M6
    x u8 [T][1.5 C] -> q_out [C][T], s_out [C][ceil(T/128)]."""
    if int(src) == SRC_E5M6:
        T, C = x.shape[0], q_out.shape[0]
        _check(x, "x", (T, C // 2 * 3), _CODES)
    else:
        T, C = x.shape
    if int(src) == SRC_FP8_1x128:
        _check(x, "x", (T, C), _CODES)
        _check(s_in, "s_in", (T, (">=", _groups(C))), ("float32",))
    elif int(src) == SRC_BF16:
        _check(x, "x", (T, C), ("bfloat16",))
    _check(q_out, "q_out", (C, T), _CODES)
    _check(s_out, "s_out", (C, (">=", (T + 127) // 128)), ("float32",))
    lds_in = _ld(s_in) if s_in is not None else 0
    _call("fp8bs_requant_T_128x1", int(src), _ptr(x), _ptr(s_in), T, C, _ld(x), lds_in,
          _ptr(q_out), _ld(q_out), _ptr(s_out), _ld(s_out), _stream(stream))


def fp8bs_transpose_w_128x128(q, s, qt, st, stream=None):
    """Codes q [N][K] with 128x128 block scales s [N/128][K/128] -> their
    transpose qt [K][N], st [K/128][N/128]."""
    N, K = q.shape
    _check(q, "q", (N, K), _CODES)
    _check(s, "s", ((N + 127) // 128, (">=", _groups(K))), ("float32",))
    _check(qt, "qt", (K, N), _CODES)
    _check(st, "st", (_groups(K), (">=", (N + 127) // 128)), ("float32",))
    _call("fp8bs_transpose_w_128x128", _ptr(q), N, K, _ld(q), _ptr(s), _ld(s), _ptr(qt), _ld(qt),
          _ptr(st), _ld(st), _stream(stream))


def _check_gemm_operands(a, sa, b, sb, bmode):
    M, K = a.shape
    N = b.shape[0]
    _check(a, "a", (M, K), _CODES)
    _check(sa, "sa", (M, (">=", _groups(K))), ("float32",))
    _check(b, "b", (N, K), _CODES)
    rows_sb = N if int(bmode) == BSCALE_ROW_1x128 else (N + 127) // 128
    _check(sb, "sb", (rows_sb, (">=", _groups(K))), ("float32",))


def fp8bs_gemm(a, sa, b, sb, bmode, d, dt, stream=None):
    """D [M][N] = A [M][K] * B [N][K]^T with block scales."""
    M, K = a.shape
    N = b.shape[0]
    _check_gemm_operands(a, sa, b, sb, bmode)
    _check(d, "d", (M, N), ("float32",) if int(dt) == OUT_F32 else ("bfloat16",))
    _call("fp8bs_gemm", _ptr(a), _ptr(sa), _ld(a), _ld(sa), _ptr(b), _ptr(sb), _ld(b), _ld(sb),
          int(bmode), _ptr(d), _ld(d), int(dt), M, N, K, _stream(stream))


def fp8bs_gemm_quant_1x128(a, sa, b, sb, bmode, q, s, stream=None):
    """D = A [M][K] * B [N][K]^T, quantized in 1x128 tiles along N:
    q u8 [M][N], s f32 [M][N/128]."""
    M, K = a.shape
    N = b.shape[0]
    _check_gemm_operands(a, sa, b, sb, bmode)
    _check(q, "q", (M, N), _CODES)
    _check(s, "s", (M, (">=", N // 128)), ("float32",))
    _call("fp8bs_gemm_quant_1x128", _ptr(a), _ptr(sa), _ld(a), _ld(sa), _ptr(b), _ptr(sb), _ld(b),
          _ld(sb), int(bmode), _ptr(q), _ld(q), _ptr(s), _ld(s), M, N, K, _stream(stream))


def fp8bs_gemm_bf16a(x, qx, sx, b, sb, d, dt, stream=None):
    """D [M][N] = quant_1x128(x bf16 [M][K]) * B [N][K]^T with 128x128 B
    scales; qx u8 [M][K] and sx f32 [M][K/128] receive the codes of x when
    given (both or neither)."""
    M, K = x.shape
    N = b.shape[0]
    _check(x, "x", (M, K), ("bfloat16",))
    if (qx is None) != (sx is None):
        raise ValueError("qx and sx: both or neither")
    if qx is not None:
        _check(qx, "qx", (M, K), _CODES)
        _check(sx, "sx", (M, (">=", _groups(K))), ("float32",))
    _check(b, "b", (N, K), _CODES)
    _check(sb, "sb", ((N + 127) // 128, (">=", _groups(K))), ("float32",))
    _check(d, "d", (M, N), ("float32",) if int(dt) == OUT_F32 else ("bfloat16",))
    _call("fp8bs_gemm_bf16a", _ptr(x), _ld(x), _ptr(qx), _ld(qx) if qx is not None else 0, _ptr(sx),
          _ld(sx) if sx is not None else 0, _ptr(b), _ptr(sb), _ld(b), _ld(sb), _ptr(d), _ld(d), int(dt),
          M, N, K, _stream(stream))


def fp8bs_grouped_gemm(a, sa, b, sb, offsets, d, dt, stream=None):
    """Per-expert D rows = A rows * B[e]^T; offsets int32 [E+1] on the device."""
    M_total, K = a.shape
    E, N, _ = b.shape
    _check(a, "a", (M_total, K), _CODES, contiguous=True)
    _check(sa, "sa", (M_total, (">=", _groups(K))), ("float32",))
    _check(b, "b", (E, N, K), _CODES, contiguous=True)
    _check(sb, "sb", (E, (N + 127) // 128, _groups(K)), ("float32",), contiguous=True)
    _check(offsets, "offsets", (E + 1,), ("int32",), contiguous=True)
    _check(d, "d", (M_total, N), ("float32",) if int(dt) == OUT_F32 else ("bfloat16",), contiguous=True)
    _call("fp8bs_grouped_gemm", _ptr(a), _ptr(sa), _ld(sa), _ptr(b), _ptr(sb), _ptr(offsets),
          int(E), M_total, _ptr(d), int(dt), N, K, _stream(stream))


# ---------------------------------------------------------------------------
# allocating helpers (torch tensors on the current device)
# ---------------------------------------------------------------------------

def quant_act_1x128(x, stream=None):
    import torch
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    fp8bs_quant_act_1x128(x, q, s, stream)
    return q, s


def quant_w_128x128(w, stream=None):
    import torch
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    fp8bs_quant_w_128x128(w, q, s, stream)
    return q, s


def fp8bs_quant_act_w(x, qx, sx, w, qw, sw, stream=None):
    """x bf16 [M][K] -> qx, sx (1x128 tiles) and w bf16 [N][K] -> qw, sw
    (128x128 blocks), in one launch."""
    M, K = x.shape
    N = w.shape[0]
    _check(x, "x", (M, K), ("bfloat16",))
    _check(qx, "qx", (M, K), _CODES)
    _check(sx, "sx", (M, (">=", _groups(K))), ("float32",))
    _check(w, "w", (N, K), ("bfloat16",))
    _check(qw, "qw", (N, K), _CODES)
    _check(sw, "sw", ((N + 127) // 128, (">=", _groups(K))), ("float32",))
    _call("fp8bs_quant_act_w", _ptr(x), M, _ld(x), _ptr(qx), _ld(qx), _ptr(sx), _ld(sx),
          _ptr(w), N, _ld(w), _ptr(qw), _ld(qw), _ptr(sw), _ld(sw), K, _stream(stream))


def fp8bs_swiglu_quant_1x128(g, u, q, s, h, stream=None):
    """h = silu(g) u of bf16 [T][I] halves -> q u8 [T][I] + s f32 [T][I/128]
    (1x128 tiles; both or neither) and/or h bf16 [T][I]."""
    T, I = g.shape
    _check(g, "g", (T, I), ("bfloat16",))
    _check(u, "u", (T, I), ("bfloat16",))
    if (q is None) != (s is None):
        raise ValueError("q and s: both or neither")
    if q is None and h is None:
        raise ValueError("no output")
    if q is not None:
        _check(q, "q", (T, I), _CODES)
        _check(s, "s", (T, (">=", _groups(I))), ("float32",))
    if h is not None:
        _check(h, "h", (T, I), ("bfloat16",))
    _call("fp8bs_swiglu_quant_1x128", _ptr(g), _ld(g), _ptr(u), _ld(u), T, I, _ptr(q),
          _ld(q) if q is not None else 0, _ptr(s), _ld(s) if s is not None else 0, _ptr(h),
          _ld(h) if h is not None else 0, _stream(stream))


def swiglu_quant_1x128(g, u, with_h=False, stream=None):
    import torch
    T, I = g.shape
    q = torch.empty((T, I), dtype=torch.uint8, device=g.device)
    s = torch.empty((T, I // 128), dtype=torch.float32, device=g.device)
    h = torch.empty((T, I), dtype=torch.bfloat16, device=g.device) if with_h else None
    fp8bs_swiglu_quant_1x128(g, u, q, s, h, stream)
    return (q, s, h) if with_h else (q, s)


def quant_act_w(x, w, stream=None):
    import torch
    M, K = x.shape
    N = w.shape[0]
    qx = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    sx = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    qw = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    sw = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    fp8bs_quant_act_w(x, qx, sx, w, qw, sw, stream)
    return qx, sx, qw, sw


def quant_per_tensor(x, stream=None):
    import torch
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty((1,), dtype=torch.float32, device=x.device)
    fp8bs_quant_per_tensor(x, q, s, stream)
    return q, s


def encode_e5m6(x, stream=None):
    import torch
    T, C = x.shape
    y = torch.empty((T, C // 2 * 3), dtype=torch.uint8, device=x.device)
    fp8bs_encode_e5m6(x, y, stream)
    return y


def decode_e5m6(y, C, stream=None):
    import torch
    x = torch.empty((y.shape[0], C), dtype=torch.bfloat16, device=y.device)
    fp8bs_decode_e5m6(y, x, stream)
    return x


def requant_T_128x1(x, s_in=None, stream=None):
    """FP8 source when s_in is given (x u8 codes), bf16 source otherwise."""
    import torch
    T, C = x.shape
    Tp = (T + 15) // 16 * 16  # 16-byte aligned output rows
    q = torch.empty((C, Tp), dtype=torch.uint8, device=x.device)[:, :T]
    s = torch.empty((C, (T + 127) // 128), dtype=torch.float32, device=x.device)
    src = SRC_FP8_1x128 if s_in is not None else SRC_BF16
    fp8bs_requant_T_128x1(src, x, s_in, q, s, stream)
    return q, s


def requant_T_128x1_e5m6(y, C, stream=None):
    """Packed E5M6 rows y u8 [T][1.5 C] -> (q [C][T], s [C][ceil(T/128)])."""
    import torch
    T = y.shape[0]
    Tp = (T + 15) // 16 * 16  # 16-byte aligned output rows
    q = torch.empty((C, Tp), dtype=torch.uint8, device=y.device)[:, :T]
    s = torch.empty((C, (T + 127) // 128), dtype=torch.float32, device=y.device)
    fp8bs_requant_T_128x1(SRC_E5M6, y, None, q, s, stream)
    return q, s


def transpose_w_128x128(q, s, stream=None):
    import torch
    N, K = q.shape
    qt = torch.empty((K, N), dtype=torch.uint8, device=q.device)
    st = torch.empty((K // 128, N // 128), dtype=torch.float32, device=q.device)
    fp8bs_transpose_w_128x128(q, s, qt, st, stream)
    return qt, st


def gemm(a, sa, b, sb, bmode=BSCALE_BLOCK_128x128, out_f32=False, stream=None):
    import torch
    M, N = a.shape[0], b.shape[0]
    d = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=a.device)
    fp8bs_gemm(a, sa, b, sb, bmode, d, OUT_F32 if out_f32 else OUT_BF16, stream)
    return d


def gemm_quant_1x128(a, sa, b, sb, bmode=BSCALE_BLOCK_128x128, stream=None):
    import torch
    M, N = a.shape[0], b.shape[0]
    q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    s = torch.empty((M, N // 128), dtype=torch.float32, device=a.device)
    fp8bs_gemm_quant_1x128(a, sa, b, sb, bmode, q, s, stream)
    return q, s


def gemm_bf16a(x, b, sb, out_f32=False, with_codes=False, stream=None):
    import torch
    M, K = x.shape
    N = b.shape[0]
    d = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=x.device)
    qx = sx = None
    if with_codes:
        qx = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        sx = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    fp8bs_gemm_bf16a(x, qx, sx, b, sb, d, OUT_F32 if out_f32 else OUT_BF16, stream)
    return (d, qx, sx) if with_codes else d


def grouped_gemm(a, sa, b, sb, offsets, out_f32=False, stream=None):
    import torch
    M, N = a.shape[0], b.shape[1]
    d = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=a.device)
    fp8bs_grouped_gemm(a, sa, b, sb, offsets, d, OUT_F32 if out_f32 else OUT_BF16, stream)
    return d
