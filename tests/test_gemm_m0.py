"""Build invariant of the GEMM's global -> LDS copies (CPU only).

The GEMM loop sets M0 (the LDS destination of buffer_load ... lds) without
saving or restoring it, which is safe only while the compiler itself never
uses M0 in gemm.hip's kernels.  This test compiles gemm.hip for gfx950 and
checks that every instruction touching M0 is one of those copies: an
`s_mov_b32 m0, s<N>` directly followed by a `buffer_load_dword{,x4} ... lds`.
"""
import re
import shutil

import pytest

from fp8_fine_grained_fp8bs_amd import build


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_gemm_m0_only_set_by_the_copies():
    asm = build.asm("gemm.hip")
    lines = [l.strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    uses = [i for i, l in enumerate(code) if re.search(r"\bm0\b", l)]
    assert uses, "expected the copies to set M0"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", code[i]), f"unexpected use of M0: {code[i]!r}"
        assert re.match(r"buffer_load_dword(x4)? .* offen lds$", code[i + 1]), \
            f"M0 set without an LDS copy after it: {code[i]!r} then {code[i + 1]!r}"
