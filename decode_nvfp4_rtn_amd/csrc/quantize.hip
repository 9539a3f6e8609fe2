// NVFP4 activation / weight quantizer for gfx950, two passes.
//
// Method: NVFP4 with one E4M3 scale per 16-element group plus an fp32
// tensor scale, quantized by plain round-to-nearest (Mix-Quant technical
// summary, gist.science, section 2 "Method", hybrid-precision strategy).
// Element format E2M1 and scale format E4M3 follow the OCP MX v1.0 and OFP8
// specifications.  The binary32 operation order is fixed by include/qlin.h.
//
// Pass 1 (amax): every block reduces max|x| over a grid-strided slice with
//   wavefront shuffles and writes one partial maximum (as the bit pattern of
//   a non-negative float, which orders like an unsigned integer).  Its loads
//   are non-temporal: measured, ordinary cached loads were 15-25 % slower
//   over both passes for tensors larger than the Infinity Cache and gained
//   nothing for smaller ones.
// Pass 2 (encode): every block first folds the partial maxima (a few KiB,
//   L2-resident) into amax and s_t -- so no third launch and no atomics are
//   needed and the result is deterministic -- then encodes (below).  Both
//   passes are streams with every wavefront access one contiguous run.
//
// This translation unit is compiled without fast-math and with
// -ffp-contract=off: every division is the correctly rounded binary32
// division and no multiply is fused into an add.
#include "nvfp4_encode.hpp"

#include <mutex>

namespace qlin {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 1024;
constexpr int kMaxEncodeBlocks = 2048;

// Partial maxima of quantize_nvfp4_noalloc, the entry point for callers that
// cannot allocate: one array in each GPU's memory for the life of the process
// (4 KiB, kMaxPartials uint32, enough for the amax pass of any input, which
// never runs more than kMaxPartials blocks).  In host code `scratch` names a
// host-side stand-in, never a device address: the launcher passes the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint32_t scratch[kMaxPartials];

// |x| as a binary32 bit pattern, for the two input dtypes.
__device__ __forceinline__ uint32_t abs_bits_bf16_pair(uint32_t w, uint32_t cur) {
  uint32_t lo = (w & 0x7FFFu) << 16;
  uint32_t hi = w & 0x7FFF0000u;
  cur = cur > lo ? cur : lo;
  return cur > hi ? cur : hi;
}

// Pass 1: partial[blockIdx.x] = max |x| over this block's grid-strided chunks
// of 16 bytes.  `nvec` counts 16-byte vectors of the whole tensor.
template <bool kBF16>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4* __restrict__ x, int64_t nvec,
                                                        uint32_t* __restrict__ partial) {
  uint32_t m = 0;
  auto fold = [&](const uint4& v) {
    if (kBF16) {
      m = abs_bits_bf16_pair(v.x, m);
      m = abs_bits_bf16_pair(v.y, m);
      m = abs_bits_bf16_pair(v.z, m);
      m = abs_bits_bf16_pair(v.w, m);
    } else {
      uint32_t a = v.x & 0x7FFFFFFFu, b = v.y & 0x7FFFFFFFu;
      uint32_t c = v.z & 0x7FFFFFFFu, d = v.w & 0x7FFFFFFFu;
      a = a > b ? a : b;
      c = c > d ? c : d;
      a = a > c ? a : c;
      m = m > a ? m : a;
    }
  };
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  // four independent 16-byte loads in flight per thread, then the remainder
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const uint4 v0 = load_nt16(&x[i]), v1 = load_nt16(&x[i + stride]);
    const uint4 v2 = load_nt16(&x[i + 2 * stride]), v3 = load_nt16(&x[i + 3 * stride]);
    fold(v0);
    fold(v1);
    fold(v2);
    fold(v3);
  }
  for (; i < nvec; i += stride) fold(load_nt16(&x[i]));
  m = block_max_u32<kThreads>(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Pass 2: tensor scale, then group scales and element codes.  Each lane
// loads one contiguous 16-byte vector (8 bf16 or 4 fp32 values) per step, U
// steps' loads issued before any is encoded, so a wavefront load is one
// contiguous 1 KiB run; the LPG lanes of a group (2 for bf16, 4 for fp32)
// exchange their partial maxima with lane shuffles, each computes the same
// group scale with the correctly rounded division, and each encodes its own
// values: multiplies by the reciprocal and paired E2M1 conversions.
//
// The reciprocal comes from a per-block table (fill_inv_table): the
// dequantized scale takes at most 127 values per tensor.  (Measured against
// two divisions per lane and one load in flight: both passes together
// 7-11 % faster at K = 4096 and 5120, equal at K = 12288, outputs
// bit-identical.)  The bf16 steps are encode8_bf16, which the W4A4 GEMM that
// quantizes its own activation operand shares.
template <bool kBF16, int U>
__global__ __launch_bounds__(kThreads) void encode_kernel(
    const uint4* __restrict__ x, int64_t nvec, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale, int static_scale,
    const uint32_t* __restrict__ partial, int npartial) {
  constexpr int LPG = kBF16 ? 2 : 4;   // lanes per 16-element group
  __shared__ float inv_tab[128];
  float s_t;
  if (static_scale) {
    s_t = *tensor_scale;
  } else {
    s_t = tensor_scale_from_partials<kThreads>(partial, npartial);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  }
  const float d = 6.0f * s_t;
  fill_inv_table(inv_tab, s_t);
  __syncthreads();
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i0 = int64_t(blockIdx.x) * kThreads + threadIdx.x; i0 < nvec; i0 += U * stride) {
    uint4 tv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) tv[u] = load_nt16(&x[min(i0 + u * stride, nvec - 1)]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      if (i >= nvec) break;
      const uint4 t = tv[u];
      uint32_t sc, w;
      if constexpr (kBF16) {
        w = encode8_bf16(t, d, inv_tab, sc);
        reinterpret_cast<uint32_t*>(codes)[i] = w;
      } else {
        // fp32: 4 values per lane, 4 lanes per group
        const float v[4] = {__uint_as_float(t.x), __uint_as_float(t.y), __uint_as_float(t.z),
                            __uint_as_float(t.w)};
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) a = __builtin_fmaxf(a, __builtin_fabsf(v[j]));
#pragma unroll
        for (int o = 1; o < LPG; o <<= 1) a = __builtin_fmaxf(a, __shfl_xor(a, o, 64));
        sc = (d == 0.0f) ? 0u : enc_e4m3(a / d);
        const float inv = inv_tab[sc];
        w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * inv, v[1] * inv, 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * inv, v[3] * inv, 1.0f, 1);
        reinterpret_cast<uint16_t*>(codes)[i] = static_cast<uint16_t>(w);
      }
      if ((i & (LPG - 1)) == 0) scales[i / LPG] = static_cast<uint8_t>(sc);
    }
  }
}

}  // namespace

int quantize_scratch_partials() { return kMaxPartials; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails
// (then it is tried again on the next call).  Host threads may call
// concurrently: the lookup runs under a lock, the kept addresses are atomics.
uint32_t* quantize_scratch() {
  static std::atomic<uint32_t*> addr[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  uint32_t* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    p = static_cast<uint32_t*>(q);
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

int quantize_blocks(int64_t rows, int64_t cols) {
  const int64_t vec = rows * cols / 8;  // 16-byte vectors of a bf16 tensor
  int64_t b = (vec + kThreads * 4 - 1) / (kThreads * 4);
  if (b < 1) b = 1;
  if (b > kMaxPartials) b = kMaxPartials;
  return static_cast<int>(b);
}

hipError_t launch_amax_bf16(const void* x, int64_t rows, int64_t cols, uint32_t* partial,
                            int* npartial, hipStream_t s) {
  const int npart = quantize_blocks(rows, cols);
  *npartial = npart;
  amax_kernel<true><<<npart, kThreads, 0, s>>>(static_cast<const uint4*>(x), rows * cols / 8,
                                               partial);
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                 bool static_scale, uint32_t* partial, hipStream_t s) {
  const bool bf16 = x_dtype == 1;
  const int64_t total = rows * cols;
  const int npart = quantize_blocks(rows, cols);
  if (!static_scale) {
    const int64_t nvec = bf16 ? total / 8 : total / 4;
    if (bf16)
      amax_kernel<true><<<npart, kThreads, 0, s>>>(static_cast<const uint4*>(x), nvec, partial);
    else
      amax_kernel<false><<<npart, kThreads, 0, s>>>(static_cast<const uint4*>(x), nvec, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nvec = bf16 ? total / 8 : total / 4;
  constexpr int U = 4;
  int64_t blocks = (nvec + kThreads * U - 1) / (kThreads * U);
  if (blocks > kMaxEncodeBlocks) blocks = kMaxEncodeBlocks;
  if (blocks < 1) blocks = 1;
  if (bf16)
    encode_kernel<true, U><<<static_cast<int>(blocks), kThreads, 0, s>>>(
        static_cast<const uint4*>(x), nvec, codes, scales, tensor_scale, static_scale,
        partial, npart);
  else
    encode_kernel<false, U><<<static_cast<int>(blocks), kThreads, 0, s>>>(
        static_cast<const uint4*>(x), nvec, codes, scales, tensor_scale, static_scale,
        partial, npart);
  return hipGetLastError();
}

}  // namespace qlin
