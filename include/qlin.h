/*
 * qlin.h -- C ABI of libqlin.so, the MI355X (gfx950) quantized linear layer.
 *
 * A linear layer computes Y = X W^T with X [m, k] (activations, row-major,
 * k contiguous) and W [n, k] (weights, row-major).  Two phases use two
 * weight formats, as in Disaggregated Quantization (singularity-lens: the
 * format-disaggregated variant runs prefill with NVFP4 compute and decode on
 * a weight-only path) and Mix-Quant (gist.science, section 2 "Method":
 * NVFP4 W4A4 prefill):
 *
 *   prefill  quantize_nvfp4(X) -> gemm_w4a4(codes, scales, s_t, W packed NVFP4)
 *   decode   gemm_w4a16(X bf16, W packed INT4 group-128)
 *            gemm_lut2 (X bf16, W packed 2-bit codebook)
 *
 * Offline weight preparation (not timed; the Disaggregated Quantization page
 * notes that its LUT speed comparison leaves out weight-format conversion):
 *   NVFP4: quantize_nvfp4(W fp32) then repack_weights(QL_NVFP4, ...)
 *   INT4 : quantize_int4_g128(W)  then repack_weights(QL_INT4_G128, ...)
 *   LUT2 : fit_lut2(W)            then repack_weights(QL_LUT2, ...)
 * The MARLIN article (abeam.tech, "オフラインで並べ替えておく") motivates
 * repacking weights and scales offline into the order the kernel reads.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated otherwise; `stream` is a
 *     hipStream_t passed as void* (NULL = the default stream).
 *   - Every call is asynchronous on `stream`.  No call allocates, frees or
 *     synchronises; the caller owns every buffer and keeps it alive until the
 *     stream work that uses it has completed.
 *   - Argument errors are reported synchronously, before any launch, as a
 *     ql_status; a failed launch returns QL_EHIP.  No call aborts and no C++
 *     exception crosses this interface.
 *   - m == 0 (or n == 0 for weight preparation) returns QL_OK and does nothing.
 *   - Buffers must be 16-byte aligned and contiguous.
 *   - Results are deterministic: fixed reduction order, no floating-point
 *     atomics, so repeated runs are bitwise identical.
 *   - Inputs must be finite (NaN/Inf are outside the method's domain).
 *   - Calls are stateless and may be issued from several host threads.
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QL_OK = 0,
  QL_EINVAL = 1,     /* null pointer, negative size or unknown flag          */
  QL_ESHAPE = 2,     /* shape constraint violated (see each call)            */
  QL_EALIGN = 3,     /* pointer not 16-byte aligned                          */
  QL_EDTYPE = 4,     /* unknown or unsupported dtype                         */
  QL_EWORKSPACE = 5, /* workspace or output buffer too small                 */
  QL_EHIP = 6,       /* a HIP launch failed                                  */
  QL_EFORMAT = 7     /* unknown weight format                                */
} ql_status;

typedef enum { QL_F32 = 0, QL_BF16 = 1 } ql_dtype;
typedef enum { QL_NVFP4 = 0, QL_INT4_G128 = 1, QL_LUT2 = 2, QL_INT4_SP24 = 3 } ql_format;

/* quantize_nvfp4 flag: read *tensor_scale as the (calibrated) tensor scale
 * instead of computing it from the tensor's absolute maximum. */
#define QL_STATIC_SCALE 1u

/* Human-readable name of a status code (static string; never NULL). */
const char *ql_status_str(int status);

/* Layout version of packed weight blobs produced by this library. */
int ql_version(void);

/* ------------------------------------------------------------------------
 * NVFP4 quantization, round to nearest (Mix-Quant, section 2: NVFP4 keeps a
 * local scale per 16-element group plus a tensor-level scale, and plain RTN
 * is enough for the format).  Element codes are E2M1, group scales E4M3
 * (OCP E4M3FN), the tensor scale fp32.  Operation order, all binary32 and
 * correctly rounded:
 *   amax = max|x|;  s_t = amax / 2688;  d = 6 * s_t
 *   per 16-group: s_g = E4M3(max|x_g| / d)   (RNE, saturating at 448; 0 if d == 0)
 *   p = s_g * s_t;  p == 0 -> codes are the sign bits alone
 *   else inv = 1 / p;  code = E2M1(x * inv)  (RNE, ties to even, saturating at 6)
 *
 * x            [rows, cols], dtype QL_F32 or QL_BF16.
 * codes        out [rows, cols/2]  : byte j holds column 2j (low nibble) and 2j+1.
 * scales       out [rows, cols/16] : E4M3 bit patterns.
 * tensor_scale device fp32 scalar: out (s_t) by default; in when
 *              flags & QL_STATIC_SCALE.
 * workspace    >= quantize_nvfp4_workspace(rows, cols) bytes of device memory
 *              (per-block partial maxima; may be NULL when that size is 0).
 * Shapes: cols % 16 == 0.  Errors: QL_EINVAL, QL_ESHAPE, QL_EALIGN,
 * QL_EDTYPE, QL_EWORKSPACE, QL_EHIP.
 * ---------------------------------------------------------------------- */
size_t quantize_nvfp4_workspace(int64_t rows, int64_t cols);
int quantize_nvfp4(const void *x, int x_dtype, int64_t rows, int64_t cols,
                   uint8_t *codes, uint8_t *scales, float *tensor_scale,
                   unsigned flags, void *workspace, size_t workspace_bytes,
                   void *stream);

/* ------------------------------------------------------------------------
 * quantize_nvfp4 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments, outputs and errors as quantize_nvfp4,
 * without the workspace.  The per-block partial maxima go to a 4 KiB array
 * (1024 x uint32) that the library keeps in each GPU's memory for the life of
 * the process; its device address is looked up once per device, at the first
 * call on that device (with that device current).  The call allocates and
 * frees nothing.  Nothing in the array needs clearing: every partial a call
 * reads is written by that call's own first pass.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that may overlap on one GPU (issued to different streams
 * without an ordering between them) race on it and may compute a wrong
 * tensor scale.  Calls on one stream are ordered and safe.
 *
 * Errors: as quantize_nvfp4 (no QL_EWORKSPACE for a missing workspace);
 * QL_EWORKSPACE if the input would need more than 1024 partial maxima (the
 * first pass never runs more than 1024 blocks, so no shape the other checks
 * accept does); QL_EHIP if the array's address cannot be looked up.
 * ---------------------------------------------------------------------- */
int quantize_nvfp4_noalloc(const void *x, int x_dtype, int64_t rows, int64_t cols,
                           uint8_t *codes, uint8_t *scales, float *tensor_scale,
                           unsigned flags, void *stream);

/* ------------------------------------------------------------------------
 * Symmetric INT4 weight quantization with groups of 128 along k (MARLIN
 * article, "データの扱い方": 4-bit weights, group size 128).  Per row and
 * group: a = max|w|; s = bf16(a / 7) (binary32 division, then RNE to bf16);
 * q = clamp(rne(w / s), -7, 7) (binary32 division by the stored scale);
 * q = 0 when s == 0.
 *
 * w       [n, k] fp32.
 * codes   out [n, k/2]   : u = q + 8 (1..15), column 2j in the low nibble.
 * scales  out [n, k/128] : bf16 bit patterns.
 * Shapes: k % 128 == 0.  Errors: QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EHIP.
 * ---------------------------------------------------------------------- */
int quantize_int4_g128(const float *w, int64_t n, int64_t k, uint8_t *codes,
                       uint16_t *scales, void *stream);

/* ------------------------------------------------------------------------
 * 2:4 structured-sparse INT4 group-128 quantization (MARLIN article,
 * "データの扱い方" and "実験と結果": Sparse-MARLIN combines the group-128
 * INT4 format with 2:4 structured sparsity).  The pages do not say how the
 * pattern is chosen; here: in every run of four consecutive columns of a row
 * the two entries of largest |w| are kept (ties to the lower column) and the
 * other two are set to zero, then the row is quantized exactly as by
 * quantize_int4_g128 (so pruned entries have q = 0, u = 8).
 *
 * Arguments, outputs, shapes and errors as quantize_int4_g128; the codes are
 * in the same dense canonical layout, with at most two nonzero q per quad.
 * ---------------------------------------------------------------------- */
int quantize_int4_g128_sp24(const float *w, int64_t n, int64_t k, uint8_t *codes,
                            uint16_t *scales, void *stream);

/* ------------------------------------------------------------------------
 * 2-bit codebook (LUT2) fit: per weight row, 4 centroids by 10 Lloyd
 * K-means iterations (KLLM article, aibr.jp, sections 1 and 3: K-means
 * quantization into centroids plus an index matrix; Disaggregated
 * Quantization: 2-bit LUT decode weights).  Centroids start at the
 * quantiles sorted(w)[floor((2j+1) k / 8)]; each iteration assigns every
 * weight to the nearest centroid in fp64 (ties to the lower index) and moves
 * each non-empty centroid to the fp64 mean of its weights, summed in
 * ascending column order.  Centroids are then rounded to bf16 (via binary32)
 * and every weight is re-assigned to the nearest rounded centroid.
 *
 * w          [n, k] fp32.
 * idx        out [n, k/4] : column 4b+i in bits 2i..2i+1 of byte b.
 * centroids  out [n, 4]   : bf16 bit patterns, ascending.
 * workspace  >= fit_lut2_workspace(n, k) bytes.
 * Shapes: k % 128 == 0, k <= 32768.  Errors: QL_EINVAL, QL_ESHAPE,
 * QL_EALIGN, QL_EWORKSPACE, QL_EHIP.
 * ---------------------------------------------------------------------- */
size_t fit_lut2_workspace(int64_t n, int64_t k);
int fit_lut2(const float *w, int64_t n, int64_t k, uint8_t *idx,
             uint16_t *centroids, void *workspace, size_t workspace_bytes,
             void *stream);

/* ------------------------------------------------------------------------
 * Offline repack of canonical quantized weights into the private gfx950
 * operand order read by the GEMM kernels (an opaque, versioned blob with a
 * header).  Pure data movement: values are not changed.
 *
 * fmt            QL_NVFP4 | QL_INT4_G128 | QL_LUT2 | QL_INT4_SP24.
 * codes          canonical codes as produced by quantize_nvfp4 (NVFP4, from
 *                W [n,k]), quantize_int4_g128 / quantize_int4_g128_sp24, or
 *                fit_lut2.  QL_INT4_SP24 keeps, in each run of four
 *                consecutive columns, the two codes of largest |q| (ties to
 *                the lower column) with their positions: every nonzero code
 *                when the codes come from quantize_int4_g128_sp24.
 * scales_or_lut  E4M3 [n, k/16] | bf16 [n, k/128] (INT4 and INT4_SP24) |
 *                bf16 centroids [n, 4].
 * tensor_scale   device fp32 s_t of the weights (NVFP4 only, else NULL);
 *                copied into the blob.
 * packed         out, >= repack_weights_bytes(fmt, n, k) bytes.
 * Shapes: n % 16 == 0, k % 128 == 0.  Errors: QL_EINVAL, QL_ESHAPE,
 * QL_EALIGN, QL_EFORMAT, QL_EWORKSPACE, QL_EHIP.
 * ---------------------------------------------------------------------- */
size_t repack_weights_bytes(int fmt, int64_t n, int64_t k);
int repack_weights(int fmt, int64_t n, int64_t k, const uint8_t *codes,
                   const void *scales_or_lut, const float *tensor_scale,
                   void *packed, size_t packed_bytes, void *stream);

/* ------------------------------------------------------------------------
 * W4A4 prefill GEMM (Mix-Quant, section 2, system-level deployment: the
 * prefill worker runs the NVFP4 W4A4 path):
 *   Y[m,n] = s_tA s_tW sum_g sA[m,g] sW[n,g] sum_{k in g} E2M1(a[m,k]) E2M1(w[n,k])
 * computed with exact fp16 dequantized operands on gfx950 MFMA and fp32
 * accumulation.
 *
 * a_codes, a_scales, a_tensor_scale : output of quantize_nvfp4 on X [m, k].
 * w_packed  NVFP4 blob of W [n, k] from repack_weights.
 * y         out [m, n], y_dtype QL_F32 or QL_BF16 (RNE).
 * Shapes: n % 16 == 0, k % 128 == 0, m >= 0.  n and k must be the values the
 * blob was packed with: the kernels read the blob header first, and a blob
 * that is not an NVFP4 blob of this (n, k) is not read further and leaves y
 * untouched (the host cannot detect it without synchronising, so no status
 * reports it).  Errors: QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EDTYPE,
 * QL_EHIP.
 * ---------------------------------------------------------------------- */
int gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales,
              const float *a_tensor_scale, const void *w_packed, int64_t m,
              int64_t n, int64_t k, void *y, int y_dtype, void *stream);

/* ------------------------------------------------------------------------
 * gemm_w4a4 with a caller-provided workspace that lets the last, partly
 * filled round of 256 x 256 output tiles (one tile per compute unit and
 * round), or a whole problem of at most half a round, be split along k over
 * the idle compute units: fp32 partial tiles go to the workspace and a
 * second launch adds them in a fixed order (so results stay deterministic;
 * they differ from gemm_w4a4's in fp32 rounding only).  Same arithmetic
 * definition and arguments as gemm_w4a4, plus:
 *
 * workspace        device memory of at least gemm_w4a4_workspace(m, n, k)
 *                  bytes, 16-byte aligned, not read before it is written;
 *                  may be NULL (then the call is gemm_w4a4).  Calls that
 *                  share one workspace must be ordered (same stream).
 * gemm_w4a4_workspace returns 0 when no split applies to the shape (the
 * tiles fill whole rounds, the last round is more than half full, or k is
 * too short for two slices), and depends on the current device's
 * compute-unit count.
 * Errors: as gemm_w4a4, and QL_EWORKSPACE when workspace is non-NULL and
 * smaller than gemm_w4a4_workspace(m, n, k).
 * ---------------------------------------------------------------------- */
size_t gemm_w4a4_workspace(int64_t m, int64_t n, int64_t k);
int gemm_w4a4_ws(const uint8_t *a_codes, const uint8_t *a_scales,
                 const float *a_tensor_scale, const void *w_packed, int64_t m,
                 int64_t n, int64_t k, void *y, int y_dtype, void *workspace,
                 size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Quantize folded into the W4A4 GEMM (Mix-Quant technical summary, section 2,
 * system-level deployment: the prefill path quantizes activations to NVFP4
 * and runs the W4A4 product): the result of quantize_nvfp4 on bf16 X followed
 * by gemm_w4a4 on its outputs, without materialising the activation codes.
 * The GEMM kernel quantizes each activation tile as it loads it, with the
 * quantizer's own operation order (quantize_nvfp4 above), so the codes, the
 * tensor scale and y are bit-identical to that pair of calls wherever
 * gemm_w4a4 runs its small-batch kernel (m <= 32) or its 128-row-tile kernel
 * (m <= 128, or few 256 x 256 tiles), whose quantizing variants this call
 * runs; gemm_w4a4's 256 x 256 kernel accumulates in another k order and
 * agrees in fp32 rounding only.  Every block that uses an activation group
 * quantizes it again (once per block of output columns): at m <= 32 this
 * costs about as much as the pair of calls (less on narrow layers), above
 * that about twice as much.  It is for callers that want no activation
 * codes in memory, or a single launch with a static tensor scale.  Two
 * launches (the amax pass, then the GEMM), or one with a static tensor
 * scale.
 *
 * x_bf16          [m, k] bf16, 16-byte aligned.
 * a_tensor_scale  device fp32 s_t of X: out by default; in when
 *                 flags & QL_STATIC_SCALE (as quantize_nvfp4).
 * w_packed        NVFP4 blob of W [n, k] from repack_weights.
 * y               out [m, n], y_dtype QL_F32 or QL_BF16 (RNE).
 * workspace       >= quantize_gemm_w4a4_workspace(m, k) bytes of device
 *                 memory (the amax pass's partial maxima), 16-byte aligned;
 *                 unused (may be NULL) with QL_STATIC_SCALE.  Calls sharing a
 *                 workspace must be ordered (same stream).
 * Shapes: n % 16 == 0, k % 128 == 0, m >= 0.  A blob that is not an NVFP4
 * blob of this (n, k) leaves y and the tensor scale untouched (as gemm_w4a4).
 * Errors: QL_EINVAL, QL_ESHAPE, QL_EALIGN, QL_EDTYPE, QL_EWORKSPACE, QL_EHIP.
 * ---------------------------------------------------------------------- */
size_t quantize_gemm_w4a4_workspace(int64_t m, int64_t k);
int quantize_gemm_w4a4(const void *x_bf16, int64_t m, int64_t k, float *a_tensor_scale,
                       unsigned flags, const void *w_packed, int64_t n, void *y,
                       int y_dtype, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ------------------------------------------------------------------------
 * W4A16 decode GEMV / skinny GEMM (weight-only decode: Disaggregated
 * Quantization; MARLIN article, "どんな技術か": 16-bit activations times
 * INT4 weights, dequantized in registers):
 *   Y[m,n] = sum_g s[n,g] sum_{k in g} x[m,k] q[n,k]   (fp32 accumulation)
 * x        [m, k] bf16.   w_packed: INT4 blob from repack_weights.
 * y        out [m, n], QL_F32 or QL_BF16.
 * Tuned for m <= 32 (decode batches); any m >= 0 is accepted.
 * Shapes: n % 16 == 0, k % 128 == 0.  Errors as gemm_w4a4.
 * The kernels read the blob header together with their first weight loads
 * and test it (magic, version, format, n, k) before their first store: a blob
 * that is not one of this format packed for this (n, k) leaves y untouched
 * (the host cannot detect it without synchronising, so no status reports
 * it).  It is read as a blob of this format and shape first, so the buffer
 * must hold at least repack_weights_bytes(format, n, k) bytes.
 * ---------------------------------------------------------------------- */
int gemm_w4a16(const void *x_bf16, const void *w_packed, int64_t m, int64_t n,
               int64_t k, void *y, int y_dtype, void *stream);

/* ------------------------------------------------------------------------
 * gemm_w4a16 with a caller-provided workspace that lets the k dimension be
 * split over blocks: each block takes one k slice of several 16-row weight
 * tiles, so the activation fragments it loads serve all of them (without a
 * split, narrow-n shapes run one row tile per block, and every block loads
 * the whole activation), and a second launch adds the slices' fp32 partial
 * sums in slice order (deterministic; results differ from gemm_w4a16's in
 * fp32 rounding only).  Same arithmetic definition and arguments as
 * gemm_w4a16, plus:
 *
 * workspace        device memory of at least gemm_w4a16_workspace(m, n, k)
 *                  bytes, 16-byte aligned, not read before it is written;
 *                  may be NULL (then the call is gemm_w4a16).  Calls that
 *                  share one workspace must be ordered (same stream).
 * gemm_w4a16_workspace returns 0 when no split applies to the shape (it
 * applies to 8 < m <= 32 with k > 4096, where it was measured faster), and
 * depends on the current device's compute-unit count.
 * Errors: as gemm_w4a16, and QL_EWORKSPACE when workspace is non-NULL and
 * smaller than gemm_w4a16_workspace(m, n, k).
 * ---------------------------------------------------------------------- */
size_t gemm_w4a16_workspace(int64_t m, int64_t n, int64_t k);
int gemm_w4a16_ws(const void *x_bf16, const void *w_packed, int64_t m, int64_t n,
                  int64_t k, void *y, int y_dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * LUT2 decode GEMV (2-bit codebook weights; KLLM article section 3 and
 * Disaggregated Quantization's LUT2 decode):
 *   Y[m,n] = sum_k x[m,k] C[n, idx[n,k]]   (fp32 accumulation)
 * x        [m, k] bf16.   w_packed: LUT2 blob from repack_weights.
 * y        out [m, n], QL_F32 or QL_BF16.
 * Shapes: n % 16 == 0, k % 128 == 0.  Errors as gemm_w4a4.
 * The kernels read the blob header together with their first weight loads
 * and test it (magic, version, format, n, k) before their first store: a blob
 * that is not one of this format packed for this (n, k) leaves y untouched
 * (the host cannot detect it without synchronising, so no status reports
 * it).  It is read as a blob of this format and shape first, so the buffer
 * must hold at least repack_weights_bytes(format, n, k) bytes.
 * ---------------------------------------------------------------------- */
int gemm_lut2(const void *x_bf16, const void *w_packed, int64_t m, int64_t n,
              int64_t k, void *y, int y_dtype, void *stream);

/* ------------------------------------------------------------------------
 * gemm_lut2 with a caller-provided workspace for a k split over blocks, as
 * gemm_w4a16_ws: same arithmetic definition and arguments as gemm_lut2, plus
 * the workspace (at least gemm_lut2_workspace(m, n, k) bytes, 16-byte
 * aligned, not read before it is written; NULL makes the call gemm_lut2;
 * calls sharing a workspace must be ordered).  gemm_lut2_workspace returns 0
 * when no split applies.  Errors: as gemm_lut2, and QL_EWORKSPACE when the
 * workspace is non-NULL and too small.
 * ---------------------------------------------------------------------- */
size_t gemm_lut2_workspace(int64_t m, int64_t n, int64_t k);
int gemm_lut2_ws(const void *x_bf16, const void *w_packed, int64_t m, int64_t n,
                 int64_t k, void *y, int y_dtype, void *workspace,
                 size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * 2:4 sparse W4A16 decode GEMV / skinny GEMM (MARLIN article, "実験と結果":
 * Sparse-MARLIN), on gfx950's 2:4 sparse MFMA:
 *   Y[m,n] = sum_g s[n,g] sum_{k in g, kept} x[m,k] q[n,k]   (fp32 accumulation)
 * x        [m, k] bf16.   w_packed: QL_INT4_SP24 blob from repack_weights.
 * y        out [m, n], QL_F32 or QL_BF16.
 * Tuned for m <= 32; any m >= 0 is accepted.
 * Shapes: n % 16 == 0, k % 128 == 0.  Errors as gemm_w4a4.
 * The kernels read the blob header together with their first weight loads
 * and test it (magic, version, format, n, k) before their first store: a blob
 * that is not one of this format packed for this (n, k) leaves y untouched
 * (the host cannot detect it without synchronising, so no status reports
 * it).  It is read as a blob of this format and shape first, so the buffer
 * must hold at least repack_weights_bytes(format, n, k) bytes.
 * ---------------------------------------------------------------------- */
int gemm_w4a16_sp24(const void *x_bf16, const void *w_packed, int64_t m, int64_t n,
                    int64_t k, void *y, int y_dtype, void *stream);

/* ------------------------------------------------------------------------
 * gemm_w4a16_sp24 with a caller-provided workspace for a k split over
 * blocks, as gemm_w4a16_ws: each block takes one k slice of several 16-row
 * weight tiles, and a second launch adds the slices' fp32 partial sums in
 * slice order (deterministic; results differ from gemm_w4a16_sp24's in fp32
 * rounding only).  Same arithmetic definition and arguments as
 * gemm_w4a16_sp24, plus the workspace (at least
 * gemm_w4a16_sp24_workspace(m, n, k) bytes, 16-byte aligned, not read before
 * it is written; NULL makes the call gemm_w4a16_sp24; calls sharing a
 * workspace must be ordered).  gemm_w4a16_sp24_workspace returns 0 when no
 * split applies (it applies to 8 < m <= 32 with k > 4096) and depends on the
 * current device's compute-unit count.  Errors: as gemm_w4a16_sp24, and
 * QL_EWORKSPACE when the workspace is non-NULL and too small.
 * ---------------------------------------------------------------------- */
size_t gemm_w4a16_sp24_workspace(int64_t m, int64_t n, int64_t k);
int gemm_w4a16_sp24_ws(const void *x_bf16, const void *w_packed, int64_t m,
                       int64_t n, int64_t k, void *y, int y_dtype, void *workspace,
                       size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
