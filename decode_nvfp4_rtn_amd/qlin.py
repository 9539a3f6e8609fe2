"""Thin Python binding over libqlin.so (include/qlin.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libqlin.so.  torch supplies device memory and the current stream.
Importing this module loads the library and raises ImportError when it has
not been built (``python -m decode_nvfp4_rtn_amd.build``); there is no
fallback implementation.

Function names match the C entry points.  Tensors must be contiguous and on
the GPU; outputs are allocated with torch unless passed in.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlin.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_nvfp4_rtn_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

QL_OK, QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EDTYPE, QL_EWORKSPACE, QL_EHIP, QL_EFORMAT = range(8)
QL_F32, QL_BF16 = 0, 1
QL_NVFP4, QL_INT4_G128, QL_LUT2, QL_INT4_SP24 = 0, 1, 2, 3
QL_STATIC_SCALE = 1

_vp, _i64, _sz, _int, _uint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint

_SIGS = {
    "ql_status_str": (ctypes.c_char_p, [_int]),
    "ql_version": (_int, []),
    "quantize_nvfp4_workspace": (_sz, [_i64, _i64]),
    "quantize_nvfp4": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _uint, _vp, _sz, _vp]),
    "quantize_nvfp4_noalloc": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _uint, _vp]),
    "quantize_int4_g128": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "quantize_int4_g128_sp24": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "fit_lut2_workspace": (_sz, [_i64, _i64]),
    "fit_lut2": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "repack_weights_bytes": (_sz, [_int, _i64, _i64]),
    "repack_weights": (_int, [_int, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gemm_w4a4": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp]),
    "gemm_w4a4_workspace": (_sz, [_i64, _i64, _i64]),
    "gemm_w4a4_ws": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _sz, _vp]),
    "gemm_w4a16": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp]),
    "gemm_lut2": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp]),
    "gemm_w4a16_workspace": (_sz, [_i64, _i64, _i64]),
    "gemm_lut2_workspace": (_sz, [_i64, _i64, _i64]),
    "gemm_w4a16_ws": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _sz, _vp]),
    "gemm_lut2_ws": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _sz, _vp]),
    "gemm_w4a16_sp24": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp]),
    "gemm_w4a16_sp24_workspace": (_sz, [_i64, _i64, _i64]),
    "quantize_gemm_w4a4_workspace": (_sz, [_i64, _i64]),
    "quantize_gemm_w4a4": (_int, [_vp, _i64, _i64, _vp, _uint, _vp, _i64, _vp, _int, _vp, _sz,
                                  _vp]),
    "gemm_w4a16_sp24_ws": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class QlinError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {_lib.ql_status_str(status).decode()} (status {status})")


def _check(fn, status):
    if status != QL_OK:
        raise QlinError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _bytes(t, name, nbytes, dtype=None):
    """t is a contiguous GPU tensor (of dtype, if given) of at least nbytes bytes."""
    _dev(t, name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes; the call needs {nbytes}")
    return t


def _matrix(t, name, dtype):
    _dev(t, name)
    if t.dtype != dtype or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D {dtype} tensor, got {t.dim()}-D {t.dtype}")
    return t.shape


def ql_status_str(status):
    return _lib.ql_status_str(status).decode()


def ql_version():
    return _lib.ql_version()


def quantize_nvfp4_workspace(rows, cols):
    return _lib.quantize_nvfp4_workspace(rows, cols)


def quantize_nvfp4(x, tensor_scale=None, codes=None, scales=None, workspace=None, stream=None,
                   ts_out=None):
    """NVFP4 round-to-nearest quantization of x [rows, cols] (fp32 or bf16).

    tensor_scale: None computes s_t from max|x| (written to ts_out, a 1-element
    fp32 GPU tensor, allocated when not given); a 1-element fp32 GPU tensor
    holding a calibrated s_t is used as is (QL_STATIC_SCALE).
    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], s_t fp32 [1]).
    """
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D, got {x.dim()}-D")
    rows, cols = x.shape
    dt = {torch.float32: QL_F32, torch.bfloat16: QL_BF16}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be float32 or bfloat16")
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    _bytes(codes, "codes", rows * (cols // 2), torch.uint8)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    _bytes(scales, "scales", rows * (cols // 16), torch.uint8)
    flags = 0
    if tensor_scale is None:
        ts = ts_out if ts_out is not None else torch.empty(1, dtype=torch.float32, device=dev)
        _bytes(ts, "ts_out", 4, torch.float32)
    else:
        ts = _bytes(tensor_scale, "tensor_scale", 4, torch.float32)
        flags = QL_STATIC_SCALE
    wsb = _lib.quantize_nvfp4_workspace(rows, cols)
    if workspace is None and not flags:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    if workspace is not None:
        _bytes(workspace, "workspace", 0, torch.uint8)
    _check("quantize_nvfp4", _lib.quantize_nvfp4(
        _ptr(x), dt, rows, cols, _ptr(codes), _ptr(scales), _ptr(ts), flags,
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return codes, scales, ts


def quantize_nvfp4_noalloc(x, codes, scales, tensor_scale, static_scale=False, stream=None):
    """quantize_nvfp4 without a workspace (the library keeps the partial maxima
    in a per-GPU array), for callers that cannot allocate: every output is the
    caller's.  tensor_scale (1-element fp32 GPU tensor) receives s_t, or holds
    a calibrated s_t when static_scale.  Calls that may overlap on one GPU
    (different streams without ordering) race on that array.
    Returns (codes, scales, tensor_scale)."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D, got {x.dim()}-D")
    rows, cols = x.shape
    dt = {torch.float32: QL_F32, torch.bfloat16: QL_BF16}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be float32 or bfloat16")
    _bytes(codes, "codes", rows * (cols // 2), torch.uint8)
    _bytes(scales, "scales", rows * (cols // 16), torch.uint8)
    _bytes(tensor_scale, "tensor_scale", 4, torch.float32)
    _check("quantize_nvfp4_noalloc", _lib.quantize_nvfp4_noalloc(
        _ptr(x), dt, rows, cols, _ptr(codes), _ptr(scales), _ptr(tensor_scale),
        QL_STATIC_SCALE if static_scale else 0, _stream(stream)))
    return codes, scales, tensor_scale


def quantize_int4_g128(w, codes=None, scales=None, stream=None, sparse24=False):
    """Symmetric INT4 group-128 quantization of fp32 weights [n, k]; with
    sparse24, 2:4 magnitude pruning along k first (quantize_int4_g128_sp24).
    Returns (codes uint8 [n, k/2], scales int16 (bf16 bits) [n, k/128])."""
    n, k = _matrix(w, "w", torch.float32)
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    _bytes(codes, "codes", n * (k // 2), torch.uint8)
    if scales is None:
        scales = torch.empty((n, k // 128), dtype=torch.int16, device=w.device)
    _bytes(scales, "scales", n * (k // 128) * 2)
    name = "quantize_int4_g128_sp24" if sparse24 else "quantize_int4_g128"
    _check(name, getattr(_lib, name)(_ptr(w), n, k, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def fit_lut2_workspace(n, k):
    return _lib.fit_lut2_workspace(n, k)


def fit_lut2(w, idx=None, centroids=None, workspace=None, stream=None):
    """2-bit codebook fit of fp32 weights [n, k] (10 Lloyd iterations per row).
    Returns (idx uint8 [n, k/4], centroids int16 (bf16 bits) [n, 4])."""
    n, k = _matrix(w, "w", torch.float32)
    if idx is None:
        idx = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    _bytes(idx, "idx", n * (k // 4), torch.uint8)
    if centroids is None:
        centroids = torch.empty((n, 4), dtype=torch.int16, device=w.device)
    _bytes(centroids, "centroids", n * 8)
    wsb = _lib.fit_lut2_workspace(n, k)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=w.device)
    _bytes(workspace, "workspace", 0, torch.uint8)
    _check("fit_lut2", _lib.fit_lut2(_ptr(w), n, k, _ptr(idx), _ptr(centroids), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))
    return idx, centroids


# Bytes of the canonical (codes, scales or codebook) inputs of repack_weights.
_CANONICAL_BYTES = {
    QL_NVFP4: lambda n, k: (n * (k // 2), n * (k // 16)),
    QL_INT4_G128: lambda n, k: (n * (k // 2), n * (k // 128) * 2),
    QL_INT4_SP24: lambda n, k: (n * (k // 2), n * (k // 128) * 2),
    QL_LUT2: lambda n, k: (n * (k // 4), n * 8),
}


def repack_weights_bytes(fmt, n, k):
    return _lib.repack_weights_bytes(fmt, n, k)


def repack_weights(fmt, n, k, codes, scales_or_lut, tensor_scale=None, packed=None, stream=None):
    """Repack canonical quantized weights into the kernel operand order.
    Returns the packed blob (uint8 GPU tensor)."""
    if fmt not in _CANONICAL_BYTES:
        raise ValueError(f"unknown weight format {fmt}")
    code_bytes, aux_bytes = _CANONICAL_BYTES[fmt](n, k)
    _bytes(codes, "codes", code_bytes, torch.uint8)
    _bytes(scales_or_lut, "scales_or_lut", aux_bytes)
    if fmt == QL_NVFP4:
        if tensor_scale is None:
            raise ValueError("an NVFP4 blob needs the weights' tensor_scale")
        _bytes(tensor_scale, "tensor_scale", 4, torch.float32)
    nbytes = _lib.repack_weights_bytes(fmt, n, k)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _bytes(packed, "packed", nbytes, torch.uint8)
    _check("repack_weights", _lib.repack_weights(
        fmt, n, k, _ptr(codes), _ptr(scales_or_lut), _ptr(tensor_scale), _ptr(packed),
        packed.numel(), _stream(stream)))
    return packed


def _out(y, m, n, dtype, dev):
    if y is None:
        y = torch.empty((m, n), dtype=dtype, device=dev)
    else:
        _dev(y, "y")
        if tuple(y.shape) != (m, n):
            raise ValueError(f"y must be [{m}, {n}], got {list(y.shape)}")
    dt = {torch.float32: QL_F32, torch.bfloat16: QL_BF16}.get(y.dtype)
    if dt is None:
        raise ValueError("y must be float32 or bfloat16")
    return y, dt


# Host-side shape and size checks (no device access, no synchronisation).
# Every buffer a kernel reads or writes must be at least as large as the call
# says; in particular a packed blob must hold repack_weights_bytes(fmt, n, k)
# bytes, so no kernel reads past it whatever its contents.

def _typed(t, name, dtype):
    _dev(t, name)
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _rows(t, name, dtype, m, cols):
    _typed(t, name, dtype)
    if t.dim() != 2 or t.shape[1] != cols or t.shape[0] < m:
        raise ValueError(f"{name} must be [>= {m}, {cols}], got {list(t.shape)}")


def _blob(w_packed, fmt, n, k):
    _typed(w_packed, "w_packed", torch.uint8)
    need = _lib.repack_weights_bytes(fmt, n, k)
    if w_packed.numel() < need:
        raise ValueError(f"w_packed holds {w_packed.numel()} bytes; a format-{fmt} blob "
                         f"of [{n}, {k}] takes {need}")


def gemm_w4a4_workspace(m, n, k):
    return _lib.gemm_w4a4_workspace(m, n, k)


def gemm_w4a4(a_codes, a_scales, a_tensor_scale, w_packed, m, n, k, y=None,
              out_dtype=torch.float32, stream=None, workspace=None):
    """NVFP4 W4A4 prefill GEMM: Y [m, n] = dequant(A) dequant(W)^T.

    workspace: None calls gemm_w4a4 (no k split of the last round of tiles);
    a uint8 GPU tensor of at least gemm_w4a4_workspace(m, n, k) bytes calls
    gemm_w4a4_ws with it."""
    _rows(a_codes, "a_codes", torch.uint8, m, k // 2)
    _rows(a_scales, "a_scales", torch.uint8, m, k // 16)
    _typed(a_tensor_scale, "a_tensor_scale", torch.float32)
    if a_tensor_scale.numel() < 1:
        raise ValueError("a_tensor_scale must hold one value")
    _blob(w_packed, QL_NVFP4, n, k)
    y, dt = _out(y, m, n, out_dtype, a_codes.device)
    if workspace is not None:
        _typed(workspace, "workspace", torch.uint8)
    if workspace is None:
        _check("gemm_w4a4", _lib.gemm_w4a4(
            _ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), _ptr(w_packed), m, n, k,
            _ptr(y), dt, _stream(stream)))
    else:
        _check("gemm_w4a4_ws", _lib.gemm_w4a4_ws(
            _ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), _ptr(w_packed), m, n, k,
            _ptr(y), dt, _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def quantize_gemm_w4a4_workspace(m, k):
    return _lib.quantize_gemm_w4a4_workspace(m, k)


def quantize_gemm_w4a4(x, w_packed, n, y=None, out_dtype=torch.float32, tensor_scale=None,
                       ts_out=None, workspace=None, stream=None):
    """quantize_nvfp4(x) then gemm_w4a4 in one call whose GEMM quantizes the
    activation tiles as it loads them (x: bf16 [m, k]).

    tensor_scale: None computes s_t (written to ts_out, allocated when not
    given); a 1-element fp32 GPU tensor holding a calibrated s_t is used as is
    (QL_STATIC_SCALE: one launch).  workspace: the amax pass's partial maxima
    (quantize_gemm_w4a4_workspace(m, k) bytes), allocated when not given.
    Returns (y, s_t)."""
    _typed(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D, got {x.dim()}-D")
    m, k = x.shape
    _blob(w_packed, QL_NVFP4, n, k)
    y, dt = _out(y, m, n, out_dtype, x.device)
    flags = 0
    if tensor_scale is None:
        ts = ts_out if ts_out is not None else torch.empty(1, dtype=torch.float32, device=x.device)
        _bytes(ts, "ts_out", 4, torch.float32)
        if workspace is None:
            workspace = torch.empty(max(16, _lib.quantize_gemm_w4a4_workspace(m, k)),
                                    dtype=torch.uint8, device=x.device)
    else:
        ts = _bytes(tensor_scale, "tensor_scale", 4, torch.float32)
        flags = QL_STATIC_SCALE
    if workspace is not None:
        _typed(workspace, "workspace", torch.uint8)
    _check("quantize_gemm_w4a4", _lib.quantize_gemm_w4a4(
        _ptr(x), m, k, _ptr(ts), flags, _ptr(w_packed), n, _ptr(y), dt, _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    return y, ts


def gemm_w4a16_workspace(m, n, k):
    return _lib.gemm_w4a16_workspace(m, n, k)


def gemm_lut2_workspace(m, n, k):
    return _lib.gemm_lut2_workspace(m, n, k)


def gemm_w4a16_sp24_workspace(m, n, k):
    return _lib.gemm_w4a16_sp24_workspace(m, n, k)


def _decode(name, fmt, x, w_packed, n, k, y, out_dtype, stream, workspace):
    m = x.shape[0] if x.dim() == 2 else -1
    _rows(x, "x", torch.bfloat16, m, k)
    _blob(w_packed, fmt, n, k)
    y, dt = _out(y, m, n, out_dtype, x.device)
    if workspace is None:
        _check(name, getattr(_lib, name)(_ptr(x), _ptr(w_packed), m, n, k, _ptr(y), dt,
                                         _stream(stream)))
    else:
        _typed(workspace, "workspace", torch.uint8)
        _check(name + "_ws", getattr(_lib, name + "_ws")(
            _ptr(x), _ptr(w_packed), m, n, k, _ptr(y), dt, _ptr(workspace), workspace.numel(),
            _stream(stream)))
    return y


def gemm_w4a16(x, w_packed, n, k, y=None, out_dtype=torch.bfloat16, stream=None, workspace=None):
    """W4A16 decode GEMM: Y [m, n] = X bf16 [m, k] times INT4-g128 weights^T.

    workspace: None calls gemm_w4a16; a uint8 GPU tensor of at least
    gemm_w4a16_workspace(m, n, k) bytes calls gemm_w4a16_ws with it (k split
    over blocks for shapes with long k or few row tiles)."""
    return _decode("gemm_w4a16", QL_INT4_G128, x, w_packed, n, k, y, out_dtype, stream, workspace)


def gemm_lut2(x, w_packed, n, k, y=None, out_dtype=torch.bfloat16, stream=None, workspace=None):
    """LUT2 decode GEMM: Y [m, n] = X bf16 [m, k] times codebook weights^T.

    workspace: as gemm_w4a16 (gemm_lut2_workspace / gemm_lut2_ws)."""
    return _decode("gemm_lut2", QL_LUT2, x, w_packed, n, k, y, out_dtype, stream, workspace)


def gemm_w4a16_sp24(x, w_packed, n, k, y=None, out_dtype=torch.bfloat16, stream=None,
                    workspace=None):
    """2:4 sparse W4A16 decode GEMM: Y [m, n] = X bf16 [m, k] times 2:4 INT4 weights^T.

    workspace: as gemm_w4a16 (gemm_w4a16_sp24_workspace / gemm_w4a16_sp24_ws)."""
    return _decode("gemm_w4a16_sp24", QL_INT4_SP24, x, w_packed, n, k, y, out_dtype, stream,
                   workspace)


def raw():
    """The ctypes handle of libqlin.so (for tests that call the C ABI directly)."""
    return _lib
