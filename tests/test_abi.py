"""The C ABI: library loads, exports what include/fa.h declares, and rejects bad
arguments before touching HIP (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _lib():
    from tiled_online_softmax_fa_amd import LIB_PATH, load_library, open_library

    # the sanitizer run (tests/test_abi_asan.py) points this module at its instrumented build
    other = os.environ.get("FA_ABI_TEST_LIB")
    if other:
        return open_library(other)
    if not os.path.exists(LIB_PATH):
        pytest.skip("libfa.so not built (run __graft_entry__.build())")
    return load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == ["fa_bwd", "fa_bwd_noalloc", "fa_bwd_timed", "fa_bwd_workspace_bytes", "fa_fwd",
                                    "fa_fwd_blocksparse", "fa_fwd_f32", "fa_fwd_fp8", "fa_fwd_splitkv",
                                    "fa_fwd_splitkv_workspace_bytes", "fa_quantize_fp8", "fa_status_string"]


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


BAD = ctypes.c_void_p(16)  # never dereferenced: validation fails before any use
NULL = ctypes.c_void_p(0)


def _fwd(lib, B=1, Hq=2, Hkv=2, N=8, d=64, causal=0, scale=0.125, ptrs=None, entry="fa_fwd"):
    p = ptrs or [BAD] * 5
    return getattr(lib, entry)(*p, B, Hq, Hkv, N, d, causal, scale, NULL)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f32"])
def test_forward_argument_errors(entry):
    from tiled_online_softmax_fa_amd import FA_ERR_INVALID_ARG as INV, FA_ERR_UNSUPPORTED as UNS, FA_OK

    lib = _lib()
    assert _fwd(lib, d=96, entry=entry) == UNS
    assert _fwd(lib, d=512, entry=entry) == UNS
    # head dim 256: bf16 forward only (there validation goes on to the pointer check)
    assert _fwd(lib, d=256, ptrs=[NULL] * 5, entry=entry) == (INV if entry == "fa_fwd" else UNS)
    assert _fwd(lib, Hq=3, Hkv=2, entry=entry) == INV
    assert _fwd(lib, Hkv=0, entry=entry) == INV
    assert _fwd(lib, B=-1, entry=entry) == INV
    assert _fwd(lib, N=-5, entry=entry) == INV
    assert _fwd(lib, causal=2, entry=entry) == INV
    assert _fwd(lib, scale=float("nan"), entry=entry) == INV
    assert _fwd(lib, scale=float("inf"), entry=entry) == INV
    assert _fwd(lib, scale=0.0, entry=entry) == INV
    assert _fwd(lib, scale=-0.5, entry=entry) == INV
    assert _fwd(lib, B=1 << 12, Hq=64, Hkv=8, N=1 << 12, d=128, entry=entry) == INV  # >= 2^31 elements
    assert _fwd(lib, ptrs=[BAD, BAD, NULL, BAD, BAD], entry=entry) == INV
    misaligned = ctypes.c_void_p(16 + 2)
    assert _fwd(lib, ptrs=[BAD, misaligned, BAD, BAD, BAD], entry=entry) == INV
    # empty problems succeed without touching the pointers
    assert _fwd(lib, B=0, ptrs=[NULL] * 5, entry=entry) == FA_OK
    assert _fwd(lib, N=0, ptrs=[NULL] * 5, entry=entry) == FA_OK


def test_backward_argument_errors():
    from tiled_online_softmax_fa_amd import FA_ERR_INVALID_ARG as INV, FA_ERR_UNSUPPORTED as UNS, FA_OK

    lib = _lib()
    ws = lib.fa_bwd_workspace_bytes(1, 2, 2, 8, 64)
    assert ws >= 2 * 8 * 4
    assert lib.fa_bwd_workspace_bytes(1, 2, 2, 8, 96) == 0
    assert lib.fa_bwd_workspace_bytes(1, 3, 2, 8, 64) == 0
    # empty problems: a size (nothing is launched), for grouped and ungrouped heads
    for shape in ((0, 2, 2, 8, 64), (1, 2, 2, 0, 64), (0, 8, 2, 16, 128), (1, 8, 2, 0, 256)):
        lib.fa_bwd_workspace_bytes(*shape)
    # small grids split the dK/dV work: the workspace also holds the fp32 partial sums
    assert lib.fa_bwd_workspace_bytes(1, 4, 4, 4096, 128) >= 2 * 2 * 4 * 4096 * 128 * 4
    assert lib.fa_bwd_workspace_bytes(2, 16, 16, 4096, 128) < 2 * 16 * 4096 * 128

    def call(ptrs=None, wsb=ws, **kw):
        a = dict(B=1, Hq=2, Hkv=2, N=8, d=64, causal=0, scale=0.125)
        a.update(kw)
        p = ptrs or [BAD] * 10
        return lib.fa_bwd(*p, wsb, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], NULL)

    assert call(d=80) == UNS
    assert call(d=256, ptrs=[NULL] * 10) == INV  # d = 256 is supported: validation reaches the pointers
    assert lib.fa_bwd_workspace_bytes(1, 2, 2, 8, 256) >= 2 * 8 * 4
    assert call(Hq=4, Hkv=3) == INV
    assert call(wsb=ws - 1) == INV
    assert call(ptrs=[BAD] * 9 + [NULL]) == INV
    assert call(scale=-1.0) == INV
    assert call(B=0, ptrs=[NULL] * 10, wsb=0) == FA_OK


def test_splitkv_argument_errors():
    from tiled_online_softmax_fa_amd import FA_ERR_INVALID_ARG as INV, FA_ERR_UNSUPPORTED as UNS, FA_OK

    lib = _lib()
    ws = lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 64, 3)
    assert ws >= 3 * (2 * 8 * 64 * 4 + 2 * 8 * 4)
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 64, -1) == 0
    # n_splits = 0: the library's choice. 128 workgroups (B1 H4 N8192) -> 2 parts, 512 or more -> 1
    one = lib.fa_fwd_splitkv_workspace_bytes(1, 4, 4, 8192, 128, 1)
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 4, 4, 8192, 128, 0) == lib.fa_fwd_splitkv_workspace_bytes(
        1, 4, 4, 8192, 128, 2) > one
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 8, 8, 16384, 128, 0) == lib.fa_fwd_splitkv_workspace_bytes(
        1, 8, 8, 16384, 128, 1)
    # few key tiles: no more than one part per 4 of them (N = 8 -> 1 tile -> 1 part)
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 64, 0) == lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 64, 1)
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 64, 65) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 96, 2) == 0

    def call(ptrs=None, wsb=ws, splits=3, **kw):
        a = dict(B=1, Hq=2, Hkv=2, N=8, d=64, causal=0, scale=0.125)
        a.update(kw)
        p = ptrs or [BAD] * 6
        return lib.fa_fwd_splitkv(*p, wsb, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"],
                                  splits, NULL)

    assert call(d=96) == UNS
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 8, 256, 2) >= 2 * (2 * 8 * 256 * 4 + 2 * 8 * 4)
    assert call(d=256, ptrs=[NULL] * 6) == INV
    assert call(splits=-1) == INV
    assert call(splits=65) == INV
    assert call(wsb=ws - 1) == INV
    assert call(ptrs=[BAD] * 5 + [NULL]) == INV
    assert call(Hq=3, Hkv=2) == INV
    assert call(B=0, ptrs=[NULL] * 6, wsb=0) == FA_OK
    # empty problems with the automatic part count (no division by an empty grid)
    assert call(B=0, ptrs=[NULL] * 6, wsb=0, splits=0) == FA_OK
    assert call(N=0, ptrs=[NULL] * 6, wsb=0, splits=0) == FA_OK
    assert lib.fa_fwd_splitkv_workspace_bytes(0, 2, 2, 8, 64, 0) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 2, 0, 64, 0) == 0


def test_blocksparse_argument_errors():
    from tiled_online_softmax_fa_amd import FA_ERR_INVALID_ARG as INV, FA_ERR_UNSUPPORTED as UNS, FA_OK

    lib = _lib()

    def call(ptrs=None, mask=BAD, sb=0, sh=0, **kw):
        a = dict(B=1, Hq=2, Hkv=2, N=8, d=64, causal=0, scale=0.125)
        a.update(kw)
        p = ptrs or [BAD] * 5
        return lib.fa_fwd_blocksparse(*p, mask, sb, sh, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                                      a["scale"], NULL)

    assert call(d=96) == UNS
    assert call(N=131073) == UNS
    assert call(sb=-1) == INV
    assert call(sh=-128) == INV
    assert call(Hq=3, Hkv=2) == INV
    assert call(mask=NULL) == INV
    assert call(ptrs=[BAD, BAD, BAD, NULL, BAD]) == INV
    assert call(d=256, ptrs=[NULL] * 5) == INV
    assert call(B=0, ptrs=[NULL] * 5, mask=NULL) == FA_OK


def test_fp8_argument_errors():
    from tiled_online_softmax_fa_amd import FA_ERR_INVALID_ARG as INV, FA_ERR_UNSUPPORTED as UNS, FA_OK

    lib = _lib()

    def fwd(ptrs=None, **kw):
        a = dict(B=1, Hq=2, Hkv=2, N=8, d=128, causal=0, scale=0.125)
        a.update(kw)
        p = ptrs or [BAD] * 7
        return lib.fa_fwd_fp8(*p, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], NULL)

    assert fwd(d=64) == UNS
    assert fwd(d=96) == UNS
    assert fwd(Hq=3, Hkv=2) == INV
    assert fwd(ptrs=[BAD, BAD, BAD, NULL, BAD, BAD, BAD]) == INV  # q_scale
    assert fwd(ptrs=[NULL] + [BAD] * 6) == INV
    assert fwd(scale=0.0) == INV
    assert fwd(B=0, ptrs=[NULL] * 7) == FA_OK

    def quant(ptrs=None, **kw):
        a = dict(B=1, H=2, N=8, d=128)
        a.update(kw)
        p = ptrs or [BAD] * 3
        return lib.fa_quantize_fp8(*p, a["B"], a["H"], a["N"], a["d"], NULL)

    assert quant(d=96) == UNS
    assert quant(N=-1) == INV
    assert quant(ptrs=[BAD, NULL, BAD]) == INV
    assert quant(N=0, ptrs=[NULL] * 3) == FA_OK


def test_status_strings():
    lib = _lib()
    for s in range(-7, 1):
        assert lib.fa_status_string(s)
    assert b"scratch" in lib.fa_status_string(-6)


def test_bwd_noalloc_argument_errors():
    # the allocation-free backward checks sizes and its scratch limit before any HIP call
    from tiled_online_softmax_fa_amd import (FA_ERR_INVALID_ARG as INV, FA_ERR_TOO_LARGE as BIG,
                                             FA_ERR_UNSUPPORTED as UNS, FA_OK, BWD_NOALLOC_SCRATCH_BYTES)

    lib = _lib()

    def call(B=1, Hq=2, Hkv=2, N=8, d=64, causal=0, scale=0.125, ptrs=None):
        return lib.fa_bwd_noalloc(*(ptrs or [BAD] * 9), B, Hq, Hkv, N, d, causal, scale, NULL)

    assert call(d=96) == UNS
    assert call(Hq=3, Hkv=2) == INV
    assert call(scale=float("nan")) == INV
    assert call(ptrs=[BAD] * 8 + [NULL]) == INV
    assert call(N=0, ptrs=[NULL] * 9) == FA_OK
    # B * Hq * N rows need 8 bytes of scratch each (D and lse * log2 e): 2^22 rows fit, 2^22 + 1024 do not
    assert lib.fa_bwd_workspace_bytes(1, 1024, 1024, 4096, 128) == BWD_NOALLOC_SCRATCH_BYTES
    assert call(B=1, Hq=1024, Hkv=1024, N=4097, d=128) == BIG
    # grouped heads on a small grid add split dK/dV partial sums: over the limit well before 2^22 rows
    assert lib.fa_bwd_workspace_bytes(1, 16, 1, 8192, 128) > BWD_NOALLOC_SCRATCH_BYTES
    assert call(B=1, Hq=16, Hkv=1, N=8192, d=128) == BIG
