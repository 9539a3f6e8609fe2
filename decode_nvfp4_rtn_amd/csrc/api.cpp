// extern "C" entry points of libqlin.so: argument validation and dispatch.
// Every check here runs on the host before any device work, so argument
// errors never launch anything.  See include/qlin.h for the contract.
#include "../../include/qlin.h"
#include "qlin_internal.hpp"

using namespace qlin;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? QL_OK : QL_EHIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// shared checks of the three GEMMs
int check_gemm(const void* w_packed, const void* y, int64_t m, int64_t n, int64_t k,
               int y_dtype) {
  if (m < 0 || n < 0 || k < 0) return QL_EINVAL;
  if (y_dtype != QL_F32 && y_dtype != QL_BF16) return QL_EDTYPE;
  if (n % 16 != 0 || k % 128 != 0 || n == 0 || k == 0) return QL_ESHAPE;
  if (m > (int64_t(1) << 31) / 2 || n > (int64_t(1) << 24) || k > (int64_t(1) << 20))
    return QL_ESHAPE;
  if (m == 0) return QL_OK;
  if (!w_packed || !y) return QL_EINVAL;
  if (!aligned16(w_packed) || !aligned16(y)) return QL_EALIGN;
  return -1;  // continue
}

}  // namespace

extern "C" {

const char* ql_status_str(int status) {
  switch (status) {
    case QL_OK: return "ok";
    case QL_EINVAL: return "invalid argument";
    case QL_ESHAPE: return "unsupported shape";
    case QL_EALIGN: return "pointer not 16-byte aligned";
    case QL_EDTYPE: return "unsupported dtype";
    case QL_EWORKSPACE: return "workspace or output buffer too small";
    case QL_EHIP: return "HIP launch failed";
    case QL_EFORMAT: return "unknown weight format";
    default: return "unknown status";
  }
}

int ql_version(void) { return kBlobVersion; }

size_t quantize_nvfp4_workspace(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return size_t(quantize_blocks(rows, cols)) * sizeof(uint32_t);
}

int quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                   uint8_t* scales, float* tensor_scale, unsigned flags, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (rows < 0 || cols < 0) return QL_EINVAL;
  if (flags & ~QL_STATIC_SCALE) return QL_EINVAL;
  if (x_dtype != QL_F32 && x_dtype != QL_BF16) return QL_EDTYPE;
  if (cols % 16 != 0) return QL_ESHAPE;
  if (rows > 0 && cols > (int64_t(1) << 40) / rows) return QL_ESHAPE;
  if (rows == 0 || cols == 0) return QL_OK;
  if (!x || !codes || !scales || !tensor_scale) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(codes)) return QL_EALIGN;
  const bool stat = (flags & QL_STATIC_SCALE) != 0;
  if (!stat) {
    size_t need = quantize_nvfp4_workspace(rows, cols);
    if (!workspace) return need ? QL_EINVAL : QL_EWORKSPACE;
    if (workspace_bytes < need) return QL_EWORKSPACE;
    if (!aligned16(workspace)) return QL_EALIGN;
  }
  return launch_status(launch_quantize_nvfp4(x, x_dtype, rows, cols, codes, scales,
                                             tensor_scale, stat,
                                             static_cast<uint32_t*>(workspace),
                                             as_stream(stream)));
}

int quantize_nvfp4_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale, unsigned flags,
                           void* stream) {
  if (rows < 0 || cols < 0) return QL_EINVAL;
  if (flags & ~QL_STATIC_SCALE) return QL_EINVAL;
  if (x_dtype != QL_F32 && x_dtype != QL_BF16) return QL_EDTYPE;
  if (cols % 16 != 0) return QL_ESHAPE;
  if (rows > 0 && cols > (int64_t(1) << 40) / rows) return QL_ESHAPE;
  if (rows == 0 || cols == 0) return QL_OK;
  if (!x || !codes || !scales || !tensor_scale) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(codes)) return QL_EALIGN;
  const bool stat = (flags & QL_STATIC_SCALE) != 0;
  uint32_t* partial = nullptr;
  if (!stat) {
    if (quantize_blocks(rows, cols) > quantize_scratch_partials()) return QL_EWORKSPACE;
    partial = quantize_scratch();
    if (!partial) return QL_EHIP;
  }
  return launch_status(launch_quantize_nvfp4(x, x_dtype, rows, cols, codes, scales,
                                             tensor_scale, stat, partial, as_stream(stream)));
}

int quantize_int4_g128(const float* w, int64_t n, int64_t k, uint8_t* codes, uint16_t* scales,
                       void* stream) {
  if (n < 0 || k < 0) return QL_EINVAL;
  if (k % 128 != 0) return QL_ESHAPE;
  if (n == 0 || k == 0) return QL_OK;
  if (!w || !codes || !scales) return QL_EINVAL;
  if (!aligned16(w) || !aligned16(codes)) return QL_EALIGN;
  return launch_status(launch_quantize_int4(w, n, k, codes, scales, false, as_stream(stream)));
}

int quantize_int4_g128_sp24(const float* w, int64_t n, int64_t k, uint8_t* codes,
                            uint16_t* scales, void* stream) {
  if (n < 0 || k < 0) return QL_EINVAL;
  if (k % 128 != 0) return QL_ESHAPE;
  if (n == 0 || k == 0) return QL_OK;
  if (!w || !codes || !scales) return QL_EINVAL;
  if (!aligned16(w) || !aligned16(codes)) return QL_EALIGN;
  return launch_status(launch_quantize_int4(w, n, k, codes, scales, true, as_stream(stream)));
}

size_t fit_lut2_workspace(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return 0;
  return lut2_workspace(n, k);
}

int fit_lut2(const float* w, int64_t n, int64_t k, uint8_t* idx, uint16_t* centroids,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || k < 0) return QL_EINVAL;
  if (k % 128 != 0 || k > 32768) return QL_ESHAPE;
  if (n == 0 || k == 0) return QL_OK;
  if (!w || !idx || !centroids) return QL_EINVAL;
  if (!aligned16(w) || !aligned16(idx) || !aligned16(centroids)) return QL_EALIGN;
  size_t need = fit_lut2_workspace(n, k);
  if (need && !workspace) return QL_EINVAL;
  if (workspace_bytes < need) return QL_EWORKSPACE;
  if (need && !aligned16(workspace)) return QL_EALIGN;
  return launch_status(launch_fit_lut2(w, n, k, idx, centroids, workspace, as_stream(stream)));
}

size_t repack_weights_bytes(int fmt, int64_t n, int64_t k) {
  if (fmt < QL_NVFP4 || fmt > QL_INT4_SP24 || n <= 0 || k <= 0) return 0;
  return blob_layout(fmt, n, k).total;
}

int repack_weights(int fmt, int64_t n, int64_t k, const uint8_t* codes,
                   const void* scales_or_lut, const float* tensor_scale, void* packed,
                   size_t packed_bytes, void* stream) {
  if (fmt < QL_NVFP4 || fmt > QL_INT4_SP24) return QL_EFORMAT;
  if (n < 0 || k < 0) return QL_EINVAL;
  if (n % 16 != 0 || k % 128 != 0) return QL_ESHAPE;
  if (n > (int64_t(1) << 24) || k > (int64_t(1) << 20)) return QL_ESHAPE;
  if (n == 0 || k == 0) return QL_OK;
  if (!codes || !scales_or_lut || !packed) return QL_EINVAL;
  if (fmt == QL_NVFP4 && !tensor_scale) return QL_EINVAL;
  if (!aligned16(codes) || !aligned16(packed)) return QL_EALIGN;
  if (packed_bytes < repack_weights_bytes(fmt, n, k)) return QL_EWORKSPACE;
  return launch_status(launch_repack(fmt, n, k, codes, scales_or_lut, tensor_scale, packed,
                                     as_stream(stream)));
}

int gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
              const void* w_packed, int64_t m, int64_t n, int64_t k, void* y, int y_dtype,
              void* stream) {
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!a_codes || !a_scales || !a_tensor_scale) return QL_EINVAL;
  if (!aligned16(a_codes) || !aligned16(a_scales)) return QL_EALIGN;
  return launch_status(launch_gemm_w4a4(a_codes, a_scales, a_tensor_scale, w_packed, m, n, k,
                                        y, y_dtype, nullptr, 0, as_stream(stream)));
}

size_t gemm_w4a4_workspace(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || n % 16 != 0 || k % 128 != 0) return 0;
  if (m > (int64_t(1) << 31) / 2 || n > (int64_t(1) << 24) || k > (int64_t(1) << 20)) return 0;
  return gemm_w4a4_ws_bytes(m, n, k);
}

int gemm_w4a4_ws(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                 const void* w_packed, int64_t m, int64_t n, int64_t k, void* y, int y_dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!a_codes || !a_scales || !a_tensor_scale) return QL_EINVAL;
  if (!aligned16(a_codes) || !aligned16(a_scales)) return QL_EALIGN;
  if (workspace) {
    if (!aligned16(workspace)) return QL_EALIGN;
    if (workspace_bytes < gemm_w4a4_workspace(m, n, k)) return QL_EWORKSPACE;
  }
  return launch_status(launch_gemm_w4a4(a_codes, a_scales, a_tensor_scale, w_packed, m, n, k,
                                        y, y_dtype, workspace, workspace_bytes,
                                        as_stream(stream)));
}

size_t quantize_gemm_w4a4_workspace(int64_t m, int64_t k) {
  if (m <= 0 || k <= 0 || k % 128 != 0 || k > (int64_t(1) << 20)) return 0;
  if (m > (int64_t(1) << 31) / 2) return 0;
  return quantize_nvfp4_workspace(m, k);
}

int quantize_gemm_w4a4(const void* x_bf16, int64_t m, int64_t k, float* a_tensor_scale,
                       unsigned flags, const void* w_packed, int64_t n, void* y, int y_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (flags & ~QL_STATIC_SCALE) return QL_EINVAL;
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!x_bf16 || !a_tensor_scale) return QL_EINVAL;
  if (!aligned16(x_bf16)) return QL_EALIGN;
  const bool stat = (flags & QL_STATIC_SCALE) != 0;
  if (!stat) {
    if (!workspace) return QL_EINVAL;
    if (workspace_bytes < quantize_gemm_w4a4_workspace(m, k)) return QL_EWORKSPACE;
    if (!aligned16(workspace)) return QL_EALIGN;
  }
  return launch_status(launch_quantize_gemm_w4a4(x_bf16, m, k, a_tensor_scale, stat,
                                                 static_cast<uint32_t*>(workspace), w_packed, n,
                                                 y, y_dtype, as_stream(stream)));
}

int gemm_w4a16(const void* x_bf16, const void* w_packed, int64_t m, int64_t n, int64_t k,
               void* y, int y_dtype, void* stream) {
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!x_bf16) return QL_EINVAL;
  if (!aligned16(x_bf16)) return QL_EALIGN;
  return launch_status(launch_gemm_w4a16(x_bf16, w_packed, m, n, k, y, y_dtype, nullptr, 0,
                                         as_stream(stream)));
}

int gemm_lut2(const void* x_bf16, const void* w_packed, int64_t m, int64_t n, int64_t k,
              void* y, int y_dtype, void* stream) {
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!x_bf16) return QL_EINVAL;
  if (!aligned16(x_bf16)) return QL_EALIGN;
  return launch_status(launch_gemm_lut2(x_bf16, w_packed, m, n, k, y, y_dtype, nullptr, 0,
                                        as_stream(stream)));
}

// fmt: 1 INT4, 2 LUT2, 3 INT4 2:4 sparse
static size_t decode_ws(int fmt, int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || n % 16 != 0 || k % 128 != 0) return 0;
  if (m > (int64_t(1) << 31) / 2 || n > (int64_t(1) << 24) || k > (int64_t(1) << 20)) return 0;
  const DecodeSplit p = fmt == 3 ? sp24_split_plan(m, n, k) : decode_split_plan(fmt == 2, m, n, k);
  return decode_split_bytes(p, m, n);
}

size_t gemm_w4a16_workspace(int64_t m, int64_t n, int64_t k) { return decode_ws(1, m, n, k); }
size_t gemm_lut2_workspace(int64_t m, int64_t n, int64_t k) { return decode_ws(2, m, n, k); }
size_t gemm_w4a16_sp24_workspace(int64_t m, int64_t n, int64_t k) { return decode_ws(3, m, n, k); }

static int decode_ws_call(int fmt, const void* x_bf16, const void* w_packed, int64_t m, int64_t n,
                          int64_t k, void* y, int y_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!x_bf16) return QL_EINVAL;
  if (!aligned16(x_bf16)) return QL_EALIGN;
  if (workspace) {
    if (!aligned16(workspace)) return QL_EALIGN;
    if (workspace_bytes < decode_ws(fmt, m, n, k)) return QL_EWORKSPACE;
  }
  hipStream_t s = as_stream(stream);
  switch (fmt) {
    case 2:
      return launch_status(launch_gemm_lut2(x_bf16, w_packed, m, n, k, y, y_dtype, workspace,
                                            workspace_bytes, s));
    case 3:
      return launch_status(launch_gemm_w4a16_sp24(x_bf16, w_packed, m, n, k, y, y_dtype,
                                                  workspace, workspace_bytes, s));
    default:
      return launch_status(launch_gemm_w4a16(x_bf16, w_packed, m, n, k, y, y_dtype, workspace,
                                             workspace_bytes, s));
  }
}

int gemm_w4a16_ws(const void* x_bf16, const void* w_packed, int64_t m, int64_t n, int64_t k,
                  void* y, int y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_ws_call(1, x_bf16, w_packed, m, n, k, y, y_dtype, workspace, workspace_bytes,
                        stream);
}

int gemm_lut2_ws(const void* x_bf16, const void* w_packed, int64_t m, int64_t n, int64_t k,
                 void* y, int y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_ws_call(2, x_bf16, w_packed, m, n, k, y, y_dtype, workspace, workspace_bytes,
                        stream);
}

int gemm_w4a16_sp24(const void* x_bf16, const void* w_packed, int64_t m, int64_t n, int64_t k,
                    void* y, int y_dtype, void* stream) {
  int st = check_gemm(w_packed, y, m, n, k, y_dtype);
  if (st >= 0) return st;
  if (!x_bf16) return QL_EINVAL;
  if (!aligned16(x_bf16)) return QL_EALIGN;
  return launch_status(launch_gemm_w4a16_sp24(x_bf16, w_packed, m, n, k, y, y_dtype, nullptr, 0,
                                              as_stream(stream)));
}

int gemm_w4a16_sp24_ws(const void* x_bf16, const void* w_packed, int64_t m, int64_t n, int64_t k,
                       void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_ws_call(3, x_bf16, w_packed, m, n, k, y, y_dtype, workspace, workspace_bytes,
                        stream);
}

}  // extern "C"
