"""C-ABI checks that need no GPU: the library loads, exports every function
include/qlin.h declares, and rejects bad arguments with the documented status
before any device work (every case below returns before a launch)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")
# QLIN_ABI_LIB: another build of the same library (the sanitized host build
# in test_abi_sanitized.py)
LIB = os.environ.get("QLIN_ABI_LIB") or os.path.join(ROOT, "decode_nvfp4_rtn_amd", "libqlin.so")

QL_OK, QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EDTYPE, QL_EWORKSPACE, QL_EHIP, QL_EFORMAT = range(8)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:size_t|int|char|void)\s*\*?\s*(\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (python -m decode_nvfp4_rtn_amd.build)")
    L = ctypes.CDLL(LIB)
    vp, i64, sz, i, u = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint
    sigs = {
        "ql_status_str": (ctypes.c_char_p, [i]),
        "ql_version": (i, []),
        "quantize_nvfp4_workspace": (sz, [i64, i64]),
        "quantize_nvfp4": (i, [vp, i, i64, i64, vp, vp, vp, u, vp, sz, vp]),
        "quantize_nvfp4_noalloc": (i, [vp, i, i64, i64, vp, vp, vp, u, vp]),
        "quantize_int4_g128": (i, [vp, i64, i64, vp, vp, vp]),
        "quantize_int4_g128_sp24": (i, [vp, i64, i64, vp, vp, vp]),
        "fit_lut2_workspace": (sz, [i64, i64]),
        "fit_lut2": (i, [vp, i64, i64, vp, vp, vp, sz, vp]),
        "repack_weights_bytes": (sz, [i, i64, i64]),
        "repack_weights": (i, [i, i64, i64, vp, vp, vp, vp, sz, vp]),
        "gemm_w4a4": (i, [vp, vp, vp, vp, i64, i64, i64, vp, i, vp]),
        "gemm_w4a4_workspace": (sz, [i64, i64, i64]),
        "gemm_w4a4_ws": (i, [vp, vp, vp, vp, i64, i64, i64, vp, i, vp, sz, vp]),
        "gemm_w4a16": (i, [vp, vp, i64, i64, i64, vp, i, vp]),
        "gemm_lut2": (i, [vp, vp, i64, i64, i64, vp, i, vp]),
        "gemm_w4a16_sp24": (i, [vp, vp, i64, i64, i64, vp, i, vp]),
        "gemm_w4a16_workspace": (sz, [i64, i64, i64]),
        "gemm_lut2_workspace": (sz, [i64, i64, i64]),
        "gemm_w4a16_ws": (i, [vp, vp, i64, i64, i64, vp, i, vp, sz, vp]),
        "gemm_lut2_ws": (i, [vp, vp, i64, i64, i64, vp, i, vp, sz, vp]),
        "gemm_w4a16_sp24_workspace": (sz, [i64, i64, i64]),
        "quantize_gemm_w4a4_workspace": (sz, [i64, i64]),
        "quantize_gemm_w4a4": (i, [vp, i64, i64, vp, u, vp, i64, vp, i, vp, sz, vp]),
        "gemm_w4a16_sp24_ws": (i, [vp, vp, i64, i64, i64, vp, i, vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


A = 0x10000  # fake, 16-byte aligned addresses: never dereferenced (calls return early)
B, C, D, E = 0x20000, 0x30000, 0x40000, 0x50000


def test_header_declares_the_boundary():
    names = set(_declared())
    for n in ("quantize_nvfp4", "repack_weights", "gemm_w4a4", "gemm_w4a16", "gemm_lut2",
              "quantize_int4_g128_sp24", "gemm_w4a16_sp24", "gemm_w4a4_workspace",
              "gemm_w4a4_ws", "quantize_gemm_w4a4", "quantize_gemm_w4a4_workspace"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(8):
        assert lib.ql_status_str(s)
    assert lib.ql_status_str(QL_OK) == b"ok"
    assert lib.ql_status_str(99) == b"unknown status"
    assert lib.ql_version() >= 1


def test_quantize_validation(lib):
    q = lib.quantize_nvfp4
    assert q(A, 1, 4, 15, B, C, D, 0, E, 4096, None) == QL_ESHAPE
    assert q(A, 7, 4, 16, B, C, D, 0, E, 4096, None) == QL_EDTYPE
    assert q(A, 1, 4, 16, B, C, D, 4, E, 4096, None) == QL_EINVAL
    assert q(None, 1, 4, 16, B, C, D, 0, E, 4096, None) == QL_EINVAL
    assert q(A + 4, 1, 4, 16, B, C, D, 0, E, 4096, None) == QL_EALIGN
    assert q(A, 1, 4, 16, B, C, D, 0, E, 0, None) == QL_EWORKSPACE
    assert q(A, 1, -1, 16, B, C, D, 0, E, 4096, None) == QL_EINVAL
    assert q(None, 1, 0, 16, None, None, None, 0, None, 0, None) == QL_OK   # empty: no-op
    assert lib.quantize_nvfp4_workspace(0, 16) == 0
    assert lib.quantize_nvfp4_workspace(8192, 4096) >= 4


def test_quantize_noalloc_validation(lib):
    q = lib.quantize_nvfp4_noalloc
    assert q(A, 1, 4, 15, B, C, D, 0, None) == QL_ESHAPE
    assert q(A, 7, 4, 16, B, C, D, 0, None) == QL_EDTYPE
    assert q(A, 1, 4, 16, B, C, D, 4, None) == QL_EINVAL
    assert q(None, 1, 4, 16, B, C, D, 0, None) == QL_EINVAL
    assert q(A, 1, 4, 16, B, C, None, 0, None) == QL_EINVAL
    assert q(A + 4, 1, 4, 16, B, C, D, 0, None) == QL_EALIGN
    assert q(A, 1, -1, 16, B, C, D, 0, None) == QL_EINVAL
    assert q(None, 1, 0, 16, None, None, None, 0, None) == QL_OK   # empty: no-op


def test_weight_prep_validation(lib):
    assert lib.quantize_int4_g128(A, 16, 100, B, C, None) == QL_ESHAPE
    assert lib.quantize_int4_g128(None, 16, 128, B, C, None) == QL_EINVAL
    assert lib.quantize_int4_g128(None, 0, 128, None, None, None) == QL_OK
    assert lib.quantize_int4_g128_sp24(A, 16, 100, B, C, None) == QL_ESHAPE
    assert lib.quantize_int4_g128_sp24(A, 16, 128, B + 4, C, None) == QL_EALIGN
    assert lib.quantize_int4_g128_sp24(None, 0, 128, None, None, None) == QL_OK
    assert lib.fit_lut2(A, 16, 33024, B, C, D, 1 << 20, None) == QL_ESHAPE
    assert lib.fit_lut2(A, 16, 128, B, C, D, 0, None) == QL_EWORKSPACE
    assert lib.fit_lut2(A, 16, 128, B + 2, C, D, 1 << 20, None) == QL_EALIGN


def test_repack_validation_and_sizes(lib):
    r = lib.repack_weights
    assert r(9, 16, 128, A, B, C, D, 1 << 20, None) == QL_EFORMAT
    assert r(0, 8, 128, A, B, C, D, 1 << 20, None) == QL_ESHAPE
    assert r(0, 16, 120, A, B, C, D, 1 << 20, None) == QL_ESHAPE
    assert r(0, 16, 128, A, B, None, D, 1 << 20, None) == QL_EINVAL   # NVFP4 needs s_t
    assert r(1, 16, 128, A, B, None, D, 10, None) == QL_EWORKSPACE
    for fmt, per in ((0, 0.5 + 1 / 16), (1, 0.5 + 2 / 128), (2, 0.25), (3, 0.25 + 0.125 + 2 / 128)):
        for n, k in ((16, 128), (4096, 4096), (30720, 3840)):
            nb = lib.repack_weights_bytes(fmt, n, k)
            assert nb % 256 == 0 and nb >= 256 + n * k * per
            assert nb <= 256 + n * k * per + 3 * 256 + (8 * n if fmt == 2 else 0)
    assert lib.repack_weights_bytes(5, 16, 128) == 0


@pytest.mark.parametrize("fn", ["gemm_w4a16", "gemm_lut2", "gemm_w4a16_sp24"])
def test_decode_gemm_validation(lib, fn):
    g = getattr(lib, fn)
    assert g(A, B, 1, 20, 128, C, 1, None) == QL_ESHAPE
    assert g(A, B, 1, 16, 100, C, 1, None) == QL_ESHAPE
    assert g(A, B, 1, 16, 128, C, 5, None) == QL_EDTYPE
    assert g(None, B, 1, 16, 128, C, 1, None) == QL_EINVAL
    assert g(A, None, 1, 16, 128, C, 1, None) == QL_EINVAL
    assert g(A, B, 1, 16, 128, C + 8, 1, None) == QL_EALIGN
    assert g(A, B, -2, 16, 128, C, 1, None) == QL_EINVAL
    assert g(A, B, 0, 16, 128, C, 1, None) == QL_OK


@pytest.mark.parametrize("fn", ["gemm_w4a16_ws", "gemm_lut2_ws", "gemm_w4a16_sp24_ws"])
def test_decode_ws_validation(lib, fn):
    g = getattr(lib, fn)
    assert g(A, B, 1, 20, 128, C, 1, None, 0, None) == QL_ESHAPE
    assert g(A, B, 1, 16, 128, C, 5, None, 0, None) == QL_EDTYPE
    assert g(None, B, 1, 16, 128, C, 1, None, 0, None) == QL_EINVAL
    assert g(A, B, 1, 16, 128, C, 1, D + 8, 64, None) == QL_EALIGN
    assert g(A, B, 0, 16, 128, C, 1, None, 0, None) == QL_OK
    assert lib.gemm_w4a16_workspace(0, 4096, 12288) == 0
    assert lib.gemm_lut2_workspace(16, 20, 15360) == 0
    assert lib.gemm_w4a16_sp24_workspace(16, 4096, 12000) == 0


def test_quantize_gemm_w4a4_validation(lib):
    g = lib.quantize_gemm_w4a4   # (x, m, k, ts, flags, w, n, y, y_dtype, ws, ws_bytes, stream)
    assert g(A, 4, 512, B, 0, C, 20, D, 0, E, 4096, None) == QL_ESHAPE      # n % 16
    assert g(A, 4, 500, B, 0, C, 256, D, 0, E, 4096, None) == QL_ESHAPE     # k % 128
    assert g(A, 4, 512, B, 0, C, 256, D, 3, E, 4096, None) == QL_EDTYPE
    assert g(A, 4, 512, B, 2, C, 256, D, 0, E, 4096, None) == QL_EINVAL     # unknown flag
    assert g(None, 4, 512, B, 0, C, 256, D, 0, E, 4096, None) == QL_EINVAL
    assert g(A, 4, 512, None, 0, C, 256, D, 0, E, 4096, None) == QL_EINVAL  # no tensor scale
    assert g(A, 4, 512, B, 0, None, 256, D, 0, E, 4096, None) == QL_EINVAL
    assert g(A + 8, 4, 512, B, 0, C, 256, D, 0, E, 4096, None) == QL_EALIGN
    assert g(A, 4, 512, B, 0, C, 256, D, 0, None, 0, None) == QL_EINVAL     # amax needs a workspace
    assert g(A, 4, 512, B, 0, C, 256, D, 0, E, 0, None) == QL_EWORKSPACE
    assert g(A, 4, 512, B, 0, C, 256, D, 0, E + 4, 4096, None) == QL_EALIGN
    assert g(A, -1, 512, B, 0, C, 256, D, 0, E, 4096, None) == QL_EINVAL
    assert g(None, 0, 512, None, 0, None, 256, None, 0, None, 0, None) == QL_OK   # empty: no-op
    assert lib.quantize_gemm_w4a4_workspace(0, 512) == 0
    assert lib.quantize_gemm_w4a4_workspace(8192, 4096) == lib.quantize_nvfp4_workspace(8192, 4096)


def test_w4a4_validation(lib):
    g = lib.gemm_w4a4
    assert g(A, B, C, D, 64, 20, 512, E, 0, None) == QL_ESHAPE
    assert g(A, B, C, D, 64, 256, 500, E, 0, None) == QL_ESHAPE
    assert g(A, B, C, D, 64, 256, 512, E, 3, None) == QL_EDTYPE
    assert g(A, B, None, D, 64, 256, 512, E, 0, None) == QL_EINVAL
    assert g(A + 1, B, C, D, 64, 256, 512, E, 0, None) == QL_EALIGN
    assert g(A, B + 8, C, D, 64, 256, 512, E, 0, None) == QL_EALIGN
    assert g(A, B, C, D, 0, 256, 512, E, 0, None) == QL_OK


def test_w4a4_ws_validation(lib):
    g = lib.gemm_w4a4_ws
    assert lib.gemm_w4a4_workspace(0, 256, 512) == 0
    assert lib.gemm_w4a4_workspace(64, 20, 512) == 0
    assert lib.gemm_w4a4_workspace(64, 256, 500) == 0
    assert g(A, B, C, D, 64, 20, 512, E, 0, None, 0, None) == QL_ESHAPE
    assert g(A, B, C, D, 64, 256, 512, E, 3, None, 0, None) == QL_EDTYPE
    assert g(A, B, None, D, 64, 256, 512, E, 0, None, 0, None) == QL_EINVAL
    assert g(A, B, C, D, 64, 256, 512, E, 0, B + 8, 64, None) == QL_EALIGN
    assert g(A, B, C, D, 0, 256, 512, E, 0, None, 0, None) == QL_OK
