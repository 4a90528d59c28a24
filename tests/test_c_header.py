"""The C ABI from C (CPU only): `include/fp8bs.h` compiles as C99 with every
warning an error, a C program links against libfp8bs.so, and host-side
argument checks answer through the C entry points with no GPU present
(the fake device addresses are never dereferenced)."""
import os
import shutil
import subprocess

import pytest

from fp8_fine_grained_fp8bs_amd import fp8bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(fp8bs.LIB_PATH)

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fp8bs.h"

int main(void) {
    const void *x = (const void *)0x100000;     /* fake, 16-byte aligned */
    uint8_t *q = (uint8_t *)0x200000;
    float *s = (float *)0x300000;
    int bad = 0;
    /* K not a multiple of 128 */
    bad |= fp8bs_quant_act_1x128(x, 4, 200, 256, q, 256, s, 2, NULL) != FP8BS_ERR_UNSUPPORTED_SHAPE;
    /* misaligned input */
    bad |= fp8bs_quant_act_1x128((const char *)x + 8, 4, 256, 256, q, 256, s, 2, NULL) != FP8BS_ERR_MISALIGNED;
    /* bad enum */
    bad |= fp8bs_gemm(q, s, 256, 2, q, s, 256, 2, (fp8bs_bscale)7, (void *)q, 64, FP8BS_OUT_BF16,
                      8, 64, 256, NULL) != FP8BS_ERR_INVALID_ARG;
    /* empty work is a no-op */
    bad |= fp8bs_gemm(q, s, 256, 2, q, s, 256, 2, FP8BS_BSCALE_BLOCK_128x128, (void *)q, 64,
                      FP8BS_OUT_F32, 0, 64, 256, NULL) != FP8BS_OK;
    bad |= strcmp(fp8bs_status_string(FP8BS_ERR_MISALIGNED), "FP8BS_ERR_MISALIGNED") != 0;
    printf("version %d %s\n", fp8bs_version(), bad ? "FAIL" : "OK");
    return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_c99_and_a_c_program_links_and_runs(tmp_path):
    fp8bs.load()   # the library has been built
    src = tmp_path / "use_fp8bs.c"
    exe = tmp_path / "use_fp8bs"
    src.write_text(PROGRAM)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, str(src),
           "-L", LIBDIR, "-lfp8bs", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), (r.stdout, r.stderr)
