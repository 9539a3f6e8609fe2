// Internal declarations shared by the libqlin.so translation units.
// Not part of the public ABI (include/qlin.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

namespace qlin {

// Streaming (non-temporal) vector loads: data read once should not displace
// reused data in the caches.
typedef uint32_t qlin_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t qlin_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  qlin_u32x4 v = __builtin_nontemporal_load(static_cast<const qlin_u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_nt8(const void* p) {
  qlin_u32x2 v = __builtin_nontemporal_load(static_cast<const qlin_u32x2*>(p));
  return make_uint2(v[0], v[1]);
}

// Compute units of the current device (cached per device; 0 if unknown).
// Host threads may call concurrently: the cache slots are atomics (a race
// only repeats the attribute query, which returns the same value).
inline int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Raise a kernel's dynamic-LDS limit on the current device, once per device
// (`done` is the caller's per-kernel flag array of 64 devices).  Host threads
// may race here; that only repeats the call.
inline hipError_t lds_limit_once(std::atomic<int>* done, const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev >= 0 && dev < 64) done[dev].store(1, std::memory_order_release);
  return e;
}

// fp32 -> bf16, round to nearest even, with v_cvt_pk_bf16_f32 (two values
// per instruction).  An exhaustive GPU check of every non-NaN binary32 bit
// pattern found it identical to the integer rounding
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16, denormals and overflow to infinity
// included.
typedef __bf16 qlin_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const qlin_bf16x2 r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ---------------------------------------------------------------------------
// Packed weight blob: a 256-byte header followed by the data regions.
// ---------------------------------------------------------------------------
constexpr uint32_t kBlobMagic = 0x4E494C51u;  // "QLIN"
constexpr int kBlobVersion = 2;   // 2: 2:4 codes and positions interleaved
constexpr size_t kHeaderBytes = 256;

struct BlobHeader {
  uint32_t magic;
  int32_t version;
  int32_t fmt;
  int32_t reserved;
  int64_t n;
  int64_t k;
  float tensor_scale;  // NVFP4 only
  uint32_t pad[(256 - 36) / 4];
};
static_assert(sizeof(BlobHeader) == 256, "header size");

// Device-side check of a blob against the call's format and shape.  The host
// cannot read the header without a synchronising copy, so the kernels test it
// themselves; the result is the same for every thread.  Words tested: 0
// magic, 1 version, 2 format, 4-5 n, 6-7 k (int64, little-endian; n and k of
// a call are below 2^31).
//
// The W4A4 kernels test it first (one scalar load, combined without branches
// so that no load waits for another) and, on a mismatch, return before any
// other memory access: a blob packed for another format or shape is never
// read past its end.
__device__ __forceinline__ bool blob_matches(const uint8_t* blob, int fmt, int n, int k) {
  const uint4* p = reinterpret_cast<const uint4*>(blob);
  const uint4 a = p[0], b = p[1];
  const uint32_t diff = (a.x ^ kBlobMagic) | (a.y ^ uint32_t(kBlobVersion)) | (a.z ^ uint32_t(fmt)) |
                        (b.x ^ uint32_t(n)) | b.y | (b.z ^ uint32_t(k)) | b.w;
  return diff == 0;
}

// The decode kernels cannot wait for the header ahead of their weights (that
// measured 2-23 % slower on their microsecond launches).  A scalar load
// cannot be left in flight either (scalar loads return out of order, so the
// next wait on any scalar load or LDS access would wait for it too), nor can
// an LDS-direct copy (the compiler then waits for every vector load before
// each LDS access).  So lane l loads header word l % 8 with a vector load
// issued with the first weight loads -- vector loads complete in order, so a
// wait for anything issued after it covers it -- and header_word_ok reads
// lanes 0-7 into scalar registers and tests them before the first store: one
// register per lane, 0.6 % of the decode time measured over the Qwen3-8B-like
// and Gemma3-like decode shapes.  On a mismatch the kernel stores nothing,
// after reading the buffer as a blob of the expected format and size.
__device__ __forceinline__ uint32_t header_word(const uint8_t* blob) {
  return reinterpret_cast<const uint32_t*>(blob)[threadIdx.x & 7];
}

__device__ __forceinline__ bool header_word_ok(uint32_t w, int fmt, int n, int k) {
  asm volatile("" : "+v"(w));   // tested here: the test and its wait stay at this point
  auto word = [&](int j) { return uint32_t(__builtin_amdgcn_readlane(int(w), j)); };
  const uint32_t diff = (word(0) ^ kBlobMagic) | (word(1) ^ uint32_t(kBlobVersion)) |
                        (word(2) ^ uint32_t(fmt)) | (word(4) ^ uint32_t(n)) | word(5) |
                        (word(6) ^ uint32_t(k)) | word(7);
  return diff == 0;
}

static_assert(offsetof(BlobHeader, n) == 16 && offsetof(BlobHeader, k) == 24, "header words");

// Region offsets (bytes from the start of the blob), shared by the repacker
// and the GEMM launchers.
struct BlobLayout {
  size_t codes_off, codes_bytes;
  size_t aux_off, aux_bytes;    // scales or codebook
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline BlobLayout blob_layout(int fmt, int64_t n, int64_t k) {
  BlobLayout L{};
  L.codes_off = kHeaderBytes;
  if (fmt == 0) {          // NVFP4: codes n*k/2, E4M3 scales n*k/16
    L.codes_bytes = size_t(n) * k / 2;
    L.aux_bytes = size_t(n) * k / 16;
  } else if (fmt == 1) {   // INT4 g128: codes n*k/2, bf16 scales n*k/128*2
    L.codes_bytes = size_t(n) * k / 2;
    L.aux_bytes = size_t(n) * (k / 128) * 2;
  } else if (fmt == 3) {   // 2:4 INT4 g128: kept codes n*k/4 interleaved with their
                           // positions n*k/8 (12 bytes per lane), scales
    L.codes_bytes = size_t(n) * k * 3 / 8;
    L.aux_bytes = size_t(n) * (k / 128) * 2;
  } else {                 // LUT2: indices n*k/4, codebook 8 bytes per row
    L.codes_bytes = size_t(n) * k / 4;
    L.aux_bytes = size_t(n) * 8;
  }
  L.aux_off = align256(L.codes_off + L.codes_bytes);
  L.total = align256(L.aux_off + L.aux_bytes);
  return L;
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files).  They assume validated arguments
// and return the hipError_t of the launch.
// ---------------------------------------------------------------------------
int quantize_blocks(int64_t rows, int64_t cols);
// quantize_nvfp4_noalloc: partial maxima in a library-held array per GPU.
int quantize_scratch_partials();
uint32_t* quantize_scratch();
hipError_t launch_quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                 bool static_scale, uint32_t* partial, hipStream_t s);

// Pass 1 of the quantizer alone on a bf16 tensor: quantize_blocks(rows, cols)
// partial maxima (their count is returned in *npartial).
hipError_t launch_amax_bf16(const void* x, int64_t rows, int64_t cols, uint32_t* partial,
                            int* npartial, hipStream_t s);
// The per-wave W4A4 kernel quantizing its activation operand as it loads it
// (bf16 X; partial: quantize_blocks(m, k) words unless static_scale).
hipError_t launch_quantize_gemm_w4a4(const void* x_bf16, int64_t m, int64_t k, float* ts,
                                     bool static_scale, uint32_t* partial, const void* w_packed,
                                     int64_t n, void* y, int y_dtype, hipStream_t s);

hipError_t launch_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* codes,
                                uint16_t* scales, bool prune24, hipStream_t s);
size_t lut2_workspace(int64_t n, int64_t k);
hipError_t launch_fit_lut2(const float* w, int64_t n, int64_t k, uint8_t* idx,
                           uint16_t* centroids, void* ws, hipStream_t s);

hipError_t launch_repack(int fmt, int64_t n, int64_t k, const uint8_t* codes,
                         const void* aux, const float* tensor_scale, void* packed,
                         hipStream_t s);

// W4A4: the block-cooperative kernel's last partial round of tiles can be
// split along k over the idle CUs; `ws` (fp32 partial tiles, may be null)
// enables that when it holds gemm_w4a4_ws_bytes(m, n, k) bytes.
size_t gemm_w4a4_ws_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                            const float* a_ts, const void* w_packed, int64_t m, int64_t n,
                            int64_t k, void* y, int y_dtype, void* ws, size_t ws_bytes,
                            hipStream_t s);
struct CoopSplit {
  int full;    // tiles computed whole (a multiple of the CU count)
  int tail;    // tiles of the last partial round, each split along k
  int splits;  // k slices per tail tile (1: no split)
};
CoopSplit coop_split_plan(int64_t m, int64_t n, int64_t k);
size_t coop_split_bytes(const CoopSplit& plan);
hipError_t launch_gemm_w4a4_coop(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* a_ts, const void* w_packed, int64_t m, int64_t n,
                                 int64_t k, void* y, int y_dtype, float* part, bool split,
                                 hipStream_t s);
// Decode: the k-sliced persistent plan of the workspace entry points (S < 2:
// no split for this shape; the plain kernels run).
struct DecodeSplit {
  int gw;  // groups per wave
  int mt;  // m-tiles of 16 tokens (1 or 2)
  int S;   // k slices
  int P;   // tile walkers per slice
};
DecodeSplit decode_split_plan(bool lut, int64_t m, int64_t n, int64_t k);
size_t decode_split_bytes(const DecodeSplit& p, int64_t m, int64_t n);
hipError_t launch_gemm_w4a16(const void* x, const void* w_packed, int64_t m, int64_t n,
                             int64_t k, void* y, int y_dtype, void* ws, size_t ws_bytes,
                             hipStream_t s);
hipError_t launch_gemm_w4a16_sp24(const void* x, const void* w_packed, int64_t m, int64_t n,
                                  int64_t k, void* y, int y_dtype, void* ws, size_t ws_bytes,
                                  hipStream_t s);
// 2:4 sparse decode: the k-sliced plan of its workspace entry point (S < 2:
// no split for this shape).
DecodeSplit sp24_split_plan(int64_t m, int64_t n, int64_t k);
// Sum of S slices of fp32 partial sums part[S][m][n] into y (format `fmt`'s
// blob header tested before the store), in slice order.
hipError_t launch_decode_reduce(const float* part, int S, int64_t m, int64_t n, void* y,
                                int y_dtype, const uint8_t* blob, int fmt, int64_t k,
                                hipStream_t s);
hipError_t launch_gemm_lut2(const void* x, const void* w_packed, int64_t m, int64_t n,
                            int64_t k, void* y, int y_dtype, void* ws, size_t ws_bytes,
                            hipStream_t s);

}  // namespace qlin
