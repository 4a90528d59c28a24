"""fp8_fine_grained_fp8bs_amd: fine-grained FP8 quantization and block-scaled
FP8 GEMM for AMD Instinct MI355X (gfx950).

The compute lives in ``libfp8bs.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/fp8bs.h``).  ``fp8_fine_grained_fp8bs_amd.fp8bs`` is the
thin ctypes binding; ``fp8_fine_grained_fp8bs_amd.synth`` draws the seeded
synthetic inputs.  Importing the package itself loads nothing.
"""
__all__ = ["fp8bs", "synth"]
