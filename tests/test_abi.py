"""CPU tests of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call
(fake, never dereferenced device addresses are used)."""
import os
import re

import pytest

from fp8_fine_grained_fp8bs_amd import fp8bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")
A = 0x100000          # a 16-byte aligned fake device address
NULL = None


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8bs_[A-Za-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = fp8bs.load()
    names = _declared()
    assert set(fp8bs.ENTRY_POINTS) <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fp8bs_version() >= 100


def test_status_strings():
    for code, name in [(0, "FP8BS_OK"), (1, "FP8BS_ERR_INVALID_ARG"), (2, "FP8BS_ERR_UNSUPPORTED_SHAPE"),
                       (3, "FP8BS_ERR_MISALIGNED"), (4, "FP8BS_ERR_NO_DEVICE"), (5, "FP8BS_ERR_LAUNCH")]:
        assert fp8bs.status_string(code) == name


def quant_act(x=A, M=4, K=256, ldx=256, q=A, ldq=256, s=A, lds=2):
    return fp8bs.load().fp8bs_quant_act_1x128(x, M, K, ldx, q, ldq, s, lds, NULL)


def quant_w(w=A, N=4, K=256, ldw=256, q=A, ldq=256, s=A, lds=2):
    return fp8bs.load().fp8bs_quant_w_128x128(w, N, K, ldw, q, ldq, s, lds, NULL)


def quant_aw(x=A, M=4, ldx=256, qx=A, ldqx=256, sx=A, ldsx=2, w=A, N=4, ldw=256, qw=A, ldqw=256, sw=A,
             ldsw=2, K=256):
    return fp8bs.load().fp8bs_quant_act_w(x, M, ldx, qx, ldqx, sx, ldsx, w, N, ldw, qw, ldqw, sw, ldsw, K, NULL)


def quant_pt(x=A, n=256, q=A, s=A):
    return fp8bs.load().fp8bs_quant_per_tensor(x, n, q, s, NULL)


def cast(x=A, n=100, q=A):
    return fp8bs.load().fp8bs_cast_e4m3(x, n, q, NULL)


def enc6(x=A, T=4, C=128, ldx=128, y=A, ldy=192):
    return fp8bs.load().fp8bs_encode_e5m6(x, T, C, ldx, y, ldy, NULL)


def dec6(y=A, T=4, C=128, ldy=192, x=A, ldx=128):
    return fp8bs.load().fp8bs_decode_e5m6(y, T, C, ldy, x, ldx, NULL)


def requant(src=0, x=A, s_in=A, T=256, C=128, ld_in=128, lds_in=1, q=A, ld_out=256, s_out=A, lds_out=2):
    return fp8bs.load().fp8bs_requant_T_128x1(src, x, s_in, T, C, ld_in, lds_in, q, ld_out, s_out, lds_out, NULL)


def transpose_w(q=A, N=256, K=384, ldq=384, s=A, lds=3, qt=A, ldqt=256, st=A, ldst=2):
    return fp8bs.load().fp8bs_transpose_w_128x128(q, N, K, ldq, s, lds, qt, ldqt, st, ldst, NULL)


def gemm(a=A, sa=A, lda=256, ldsa=2, b=A, sb=A, ldb=256, ldsb=2, bmode=0, d=A, ldd=64, dt=0,
         M=8, N=64, K=256):
    return fp8bs.load().fp8bs_gemm(a, sa, lda, ldsa, b, sb, ldb, ldsb, bmode, d, ldd, dt, M, N, K, NULL)


def gemm_quant(a=A, sa=A, lda=256, ldsa=2, b=A, sb=A, ldb=256, ldsb=2, bmode=0, q=A, ldq=128, s=A,
               lds=1, M=8, N=128, K=256):
    return fp8bs.load().fp8bs_gemm_quant_1x128(a, sa, lda, ldsa, b, sb, ldb, ldsb, bmode, q, ldq, s, lds,
                                               M, N, K, NULL)


def gemm_bf16a(x=A, ldx=256, qx=A, ldqx=256, sx=A, ldsx=2, b=A, sb=A, ldb=256, ldsb=2, d=A, ldd=64, dt=0,
               M=8, N=64, K=256):
    return fp8bs.load().fp8bs_gemm_bf16a(x, ldx, qx, ldqx, sx, ldsx, b, sb, ldb, ldsb, d, ldd, dt, M, N, K,
                                         NULL)


def swiglu(g=A, ldg=256, u=A, ldu=256, T=4, I=256, q=A, ldq=256, s=A, lds=2, h=A, ldh=256):
    return fp8bs.load().fp8bs_swiglu_quant_1x128(g, ldg, u, ldu, T, I, q, ldq, s, lds, h, ldh, NULL)


def grouped(a=A, sa=A, ldsa=2, b=A, sb=A, off=A, E=2, M=10, d=A, dt=0, N=128, K=256):
    return fp8bs.load().fp8bs_grouped_gemm(a, sa, ldsa, b, sb, off, E, M, d, dt, N, K, NULL)


@pytest.mark.parametrize("call,expect", [
    (lambda: quant_act(K=200, ldx=256, ldq=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: quant_act(M=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(K=0), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(x=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(q=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(s=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(ldx=128), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(lds=1), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_act(x=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: quant_act(q=A + 4), fp8bs.ERR_MISALIGNED),
    (lambda: quant_act(s=A + 2), fp8bs.ERR_MISALIGNED),
    (lambda: quant_act(ldx=260), fp8bs.ERR_MISALIGNED),
    (lambda: quant_act(ldq=264), fp8bs.ERR_MISALIGNED),
    (lambda: quant_act(M=0, x=NULL, q=NULL, s=NULL), fp8bs.OK),
    (lambda: quant_w(K=130, ldw=256, ldq=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: quant_w(N=-5), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_w(w=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_w(ldq=100), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_w(w=A + 2), fp8bs.ERR_MISALIGNED),
    (lambda: quant_w(N=0), fp8bs.OK),
    (lambda: quant_aw(K=200, ldx=256, ldqx=256, ldw=256, ldqw=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: quant_aw(M=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(N=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(K=0), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(x=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(sw=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(ldqw=128), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(ldsx=1), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_aw(w=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: quant_aw(ldqx=264), fp8bs.ERR_MISALIGNED),
    (lambda: quant_aw(M=0, N=0, x=NULL, qx=NULL, sx=NULL, w=NULL, qw=NULL, sw=NULL), fp8bs.OK),
    (lambda: quant_pt(n=-128), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_pt(n=200), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: quant_pt(x=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_pt(q=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_pt(s=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: quant_pt(x=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: quant_pt(q=A + 4), fp8bs.ERR_MISALIGNED),
    (lambda: quant_pt(s=A + 2), fp8bs.ERR_MISALIGNED),
    (lambda: quant_pt(n=0, x=NULL, q=NULL, s=NULL), fp8bs.OK),
    (lambda: cast(n=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: cast(x=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: cast(q=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: cast(x=A + 4), fp8bs.ERR_MISALIGNED),
    (lambda: cast(q=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: cast(n=0, x=NULL, q=NULL), fp8bs.OK),
    (lambda: enc6(T=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: enc6(C=0), fp8bs.ERR_INVALID_ARG),
    (lambda: enc6(C=64, ldx=64, ldy=96), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: enc6(x=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: enc6(y=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: enc6(ldy=176), fp8bs.ERR_INVALID_ARG),
    (lambda: enc6(ldy=200), fp8bs.ERR_MISALIGNED),
    (lambda: enc6(x=A + 2), fp8bs.ERR_MISALIGNED),
    (lambda: enc6(T=0, x=NULL, y=NULL), fp8bs.OK),
    (lambda: dec6(ldx=64), fp8bs.ERR_INVALID_ARG),
    (lambda: dec6(y=A + 4), fp8bs.ERR_MISALIGNED),
    (lambda: dec6(C=200, ldx=208, ldy=304), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: dec6(T=0), fp8bs.OK),
    (lambda: requant(src=7), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(C=100, ld_in=128), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: requant(T=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(s_in=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(ld_out=128), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(lds_out=1), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(q=A + 1), fp8bs.ERR_MISALIGNED),
    (lambda: requant(ld_out=264), fp8bs.ERR_MISALIGNED),
    (lambda: requant(ld_in=1 << 25), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: requant(T=0), fp8bs.OK),
    (lambda: requant(src=2, s_in=NULL, ld_in=192, T=0), fp8bs.OK),    # E5M6 source: a no-op too
    (lambda: requant(src=3), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(src=2, s_in=NULL, ld_in=176), fp8bs.ERR_INVALID_ARG),   # E5M6 rows: 1.5 C bytes
    (lambda: requant(src=2, s_in=NULL, ld_in=200), fp8bs.ERR_MISALIGNED),
    (lambda: requant(src=2, s_in=NULL, C=192, ld_in=288), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: requant(src=2, x=NULL, s_in=NULL, ld_in=192), fp8bs.ERR_INVALID_ARG),
    (lambda: requant(src=2, s_in=NULL, ld_in=1 << 25), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: transpose_w(N=-128), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(K=0), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(N=200, ldqt=208), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: transpose_w(K=320, ldq=320), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: transpose_w(q=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(s=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(qt=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(st=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(ldq=256), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(lds=2), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(ldqt=128), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(ldst=1), fp8bs.ERR_INVALID_ARG),
    (lambda: transpose_w(q=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: transpose_w(ldqt=264), fp8bs.ERR_MISALIGNED),
    (lambda: transpose_w(st=A + 1), fp8bs.ERR_MISALIGNED),
    (lambda: transpose_w(ldq=1 << 25), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: transpose_w(N=0), fp8bs.OK),
    (lambda: gemm(bmode=2), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm(dt=9), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm(K=192, lda=256, ldb=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm(M=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm(a=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm(sb=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm(ldd=32), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm(lda=264), fp8bs.ERR_MISALIGNED),
    (lambda: gemm(d=A + 4), fp8bs.ERR_MISALIGNED),
    (lambda: gemm(ldd=68), fp8bs.ERR_MISALIGNED),
    (lambda: gemm(lda=1 << 24), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm(ldsb=1 << 22), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm(M=0), fp8bs.OK),
    (lambda: gemm(N=0), fp8bs.OK),
    (lambda: swiglu(I=200, ldg=256, ldu=256, ldq=256, ldh=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: swiglu(T=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: swiglu(I=0), fp8bs.ERR_INVALID_ARG),
    (lambda: swiglu(g=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: swiglu(q=NULL), fp8bs.ERR_INVALID_ARG),                  # codes without scales
    (lambda: swiglu(q=NULL, s=NULL, h=NULL), fp8bs.ERR_INVALID_ARG),  # no output
    (lambda: swiglu(ldu=128), fp8bs.ERR_INVALID_ARG),
    (lambda: swiglu(lds=1), fp8bs.ERR_INVALID_ARG),
    (lambda: swiglu(u=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: swiglu(ldh=260), fp8bs.ERR_MISALIGNED),
    (lambda: swiglu(T=0), fp8bs.OK),
    (lambda: gemm_bf16a(dt=5), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(K=192, ldx=256, ldb=256, ldqx=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm_bf16a(M=-1), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(x=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(qx=NULL), fp8bs.ERR_INVALID_ARG),             # codes without scales
    (lambda: gemm_bf16a(sx=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(ldx=128), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(ldsx=1), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(ldsb=1), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_bf16a(x=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_bf16a(ldx=260), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_bf16a(ldqx=264), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_bf16a(ldd=68), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_bf16a(ldx=1 << 23), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm_bf16a(ldb=1 << 24), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm_bf16a(M=0), fp8bs.OK),
    (lambda: gemm_bf16a(N=0, qx=NULL, sx=NULL), fp8bs.OK),
    (lambda: gemm_quant(bmode=3), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_quant(N=192, ldq=192, lds=2), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm_quant(K=200, lda=256, ldb=256), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm_quant(M=-2), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_quant(q=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_quant(s=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_quant(ldq=64), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_quant(lds=0), fp8bs.ERR_INVALID_ARG),
    (lambda: gemm_quant(q=A + 8), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_quant(ldq=136), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_quant(s=A + 2), fp8bs.ERR_MISALIGNED),
    (lambda: gemm_quant(lda=1 << 24), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: gemm_quant(M=0), fp8bs.OK),
    (lambda: gemm_quant(N=0), fp8bs.OK),
    (lambda: grouped(E=0), fp8bs.ERR_INVALID_ARG),
    (lambda: grouped(off=NULL), fp8bs.ERR_INVALID_ARG),
    (lambda: grouped(off=A + 2), fp8bs.ERR_MISALIGNED),
    (lambda: grouped(K=100), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: grouped(N=0), fp8bs.ERR_INVALID_ARG),
    (lambda: grouped(N=68), fp8bs.ERR_MISALIGNED),
    (lambda: grouped(K=1 << 24, ldsa=1 << 17), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: grouped(ldsa=1 << 22), fp8bs.ERR_UNSUPPORTED_SHAPE),
    (lambda: grouped(M=0), fp8bs.OK),
])
def test_argument_checks_before_any_hip_call(call, expect):
    assert call() == expect


def test_valid_call_without_gpu_reports_no_device():
    """Host checks pass, then the device query fails cleanly: nothing runs."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert quant_act() == fp8bs.ERR_NO_DEVICE
    assert transpose_w() == fp8bs.ERR_NO_DEVICE
    assert quant_pt() == fp8bs.ERR_NO_DEVICE
    assert enc6() == fp8bs.ERR_NO_DEVICE and dec6() == fp8bs.ERR_NO_DEVICE
    assert requant(src=2, s_in=NULL, ld_in=192) == fp8bs.ERR_NO_DEVICE   # E5M6 source, no scales
    assert gemm_quant() == fp8bs.ERR_NO_DEVICE
    assert gemm() == fp8bs.ERR_NO_DEVICE


def test_python_binding_raises_on_error():
    import torch

    class Fake:
        shape = (4, 100)
        is_cuda = True
        def __init__(self, dtype):
            self.dtype = dtype
        def data_ptr(self):
            return A
        def stride(self, i):
            return (100, 1)[i]
        def dim(self):
            return 2
        def is_contiguous(self):
            return True
    with pytest.raises(fp8bs.Fp8bsError) as ei:
        fp8bs.fp8bs_quant_act_1x128(Fake(torch.bfloat16), Fake(torch.uint8), Fake(torch.float32), stream=0)
    assert ei.value.status == fp8bs.ERR_UNSUPPORTED_SHAPE


def test_binding_refuses_mismatched_outputs():
    """Shapes, dtypes and contiguity are checked before any pointer is
    passed: a short output would otherwise be written past its end."""
    import torch
    x = torch.zeros((256, 256), dtype=torch.bfloat16)
    q = torch.zeros((256, 256), dtype=torch.uint8)
    s = torch.zeros((256, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_quant_act_1x128(x, q[:200], s, stream=0)
    with pytest.raises(ValueError, match="dimension 1"):
        fp8bs.fp8bs_quant_act_1x128(x, q, s[:, :1], stream=0)
    with pytest.raises(ValueError, match="dtype"):
        fp8bs.fp8bs_quant_act_1x128(x.float(), q, s, stream=0)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_quant_w_128x128(x, q, s[:1], stream=0)
    a = torch.zeros((300, 256), dtype=torch.uint8)
    sa = torch.zeros((300, 2), dtype=torch.float32)
    b = torch.zeros((384, 256), dtype=torch.uint8)
    sb = torch.zeros((3, 2), dtype=torch.float32)
    d = torch.zeros((300, 384), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_gemm(a, sa, b, sb, fp8bs.BSCALE_BLOCK_128x128, d[:299], fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="dtype"):
        fp8bs.fp8bs_gemm(a, sa, b, sb, fp8bs.BSCALE_BLOCK_128x128, d, fp8bs.OUT_F32, stream=0)
    with pytest.raises(ValueError, match="dimension 0"):   # row mode needs a scale row per B row
        fp8bs.fp8bs_gemm(a, sa, b, sb, fp8bs.BSCALE_ROW_1x128, d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_gemm(a, sa[:100], b, sb, fp8bs.BSCALE_BLOCK_128x128, d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="rows"):
        fp8bs.fp8bs_gemm(a.t(), sa, b, sb, fp8bs.BSCALE_BLOCK_128x128, d, fp8bs.OUT_BF16, stream=0)
    qo = torch.zeros((300, 384), dtype=torch.uint8)
    with pytest.raises(ValueError, match="dimension 1"):
        fp8bs.fp8bs_gemm_quant_1x128(a, sa, b, sb, fp8bs.BSCALE_BLOCK_128x128, qo,
                                     torch.zeros((300, 2), dtype=torch.float32), stream=0)
    # grouped: contiguous operands, offsets of E + 1 int32
    bg = torch.zeros((2, 384, 256), dtype=torch.uint8)
    sbg = torch.zeros((2, 3, 2), dtype=torch.float32)
    off = torch.zeros((3,), dtype=torch.int32)
    with pytest.raises(ValueError, match="offsets"):
        fp8bs.fp8bs_grouped_gemm(a, sa, bg, sbg, off[:2], d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        fp8bs.fp8bs_grouped_gemm(a, sa, bg, sbg, off, torch.zeros((384, 300), dtype=torch.bfloat16).t(),
                                 fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        fp8bs.fp8bs_grouped_gemm(torch.zeros((300, 512), dtype=torch.uint8)[:, :256], sa, bg, sbg, off, d,
                                 fp8bs.OUT_BF16, stream=0)
    # requant: the transposed output must have C rows of T
    xq = torch.zeros((256, 384), dtype=torch.uint8)
    with pytest.raises(ValueError, match="q_out"):
        fp8bs.fp8bs_requant_T_128x1(fp8bs.SRC_FP8_1x128, xq, torch.zeros((256, 3), dtype=torch.float32),
                                    torch.zeros((256, 384), dtype=torch.uint8),
                                    torch.zeros((384, 2), dtype=torch.float32), stream=0)


def test_binding_refuses_mismatched_bf16a_operands():
    import torch
    x = torch.zeros((100, 256), dtype=torch.bfloat16)
    qx = torch.zeros((100, 256), dtype=torch.uint8)
    sx = torch.zeros((100, 2), dtype=torch.float32)
    b = torch.zeros((300, 256), dtype=torch.uint8)
    sb = torch.zeros((3, 2), dtype=torch.float32)
    d = torch.zeros((100, 300), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="both or neither"):
        fp8bs.fp8bs_gemm_bf16a(x, qx, None, b, sb, d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_gemm_bf16a(x, qx[:99], sx, b, sb, d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_gemm_bf16a(x, qx, sx, b, sb[:2], d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="dtype"):
        fp8bs.fp8bs_gemm_bf16a(x.float(), qx, sx, b, sb, d, fp8bs.OUT_BF16, stream=0)
    with pytest.raises(ValueError, match="dtype"):
        fp8bs.fp8bs_gemm_bf16a(x, qx, sx, b, sb, d, fp8bs.OUT_F32, stream=0)
    with pytest.raises(ValueError, match="dimension 1"):
        fp8bs.fp8bs_gemm_bf16a(x, qx, sx, b, sb, d[:, :299], fp8bs.OUT_BF16, stream=0)


def test_binding_refuses_mismatched_swiglu_operands():
    import torch
    g = torch.zeros((10, 256), dtype=torch.bfloat16)
    q = torch.zeros((10, 256), dtype=torch.uint8)
    s = torch.zeros((10, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="dimension 0"):
        fp8bs.fp8bs_swiglu_quant_1x128(g, g[:9], q, s, None, stream=0)
    with pytest.raises(ValueError, match="both or neither"):
        fp8bs.fp8bs_swiglu_quant_1x128(g, g, q, None, None, stream=0)
    with pytest.raises(ValueError, match="no output"):
        fp8bs.fp8bs_swiglu_quant_1x128(g, g, None, None, None, stream=0)
    with pytest.raises(ValueError, match="dimension 1"):
        fp8bs.fp8bs_swiglu_quant_1x128(g, g, q, s[:, :1], None, stream=0)
    with pytest.raises(ValueError, match="dtype"):
        fp8bs.fp8bs_swiglu_quant_1x128(g, g, q, s, g.float(), stream=0)


def test_binding_refuses_host_tensors():
    """A CPU tensor's address must never reach a kernel as a device pointer."""
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    q = torch.zeros((4, 128), dtype=torch.uint8)
    s = torch.zeros((4, 1), dtype=torch.float32)
    with pytest.raises(ValueError):
        fp8bs.fp8bs_quant_act_1x128(x, q, s, stream=0)
