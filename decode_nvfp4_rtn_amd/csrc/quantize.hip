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
#include "qlin_internal.hpp"

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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t sh[kThreads / 64];
  v = wave_max_u32(v);
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  uint32_t r = sh[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = r > sh[i] ? r : sh[i];
  __syncthreads();
  return r;
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
  m = block_max_u32(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// E4M3 (OCP E4M3FN) encoding of a non-negative binary32 value: round to
// nearest, ties to even, saturating at 448 (0x7E).  The hardware converter
// rounds to nearest-even but does not saturate (it returns NaN above 464), so
// the value is clamped to 448 first; a NaN input also becomes 448 (fminf
// returns the other operand).  An exhaustive sweep of every non-negative
// binary32 pattern on gfx950 found this identical to the integer encoder
// (mantissa rounding, exponent rebias, subnormal quantum 2^-9, saturation).
__device__ __forceinline__ uint32_t enc_e4m3(float q) {
  const float c = __builtin_fminf(q, 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0u, false) & 0xFFu;
}

// Exact binary32 value of a non-negative E4M3 code (0..0x7E).
__device__ __forceinline__ float dec_e4m3(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 encoding uses v_cvt_scalef32_pk_fp4_f32 with scale 1.0: two binary32
// values per instruction (the first into the low nibble) into one byte of
// the destination: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code,
// saturating at 6, sign copied also for results that round to zero.  An
// exhaustive sweep of every non-NaN binary32 pattern on gfx950 found it
// identical to the comparison chain  code = (a>.25)+(a>=.75)+(a>1.25)+
// (a>=1.75)+(a>2.5)+(a>=3.5)+(a>5), a = |y|, with the sign bit of y.

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Pass 2: tensor scale, then group scales and element codes.  Each lane
// loads one contiguous 16-byte vector (8 bf16 or 4 fp32 values) per step, U
// steps' loads issued before any is encoded, so a wavefront load is one
// contiguous 1 KiB run; the LPG lanes of a group (2 for bf16, 4 for fp32)
// exchange their partial maxima with lane shuffles, each computes the same
// group scale with the correctly rounded division, and each encodes its own
// values: multiplies by the reciprocal and paired E2M1 conversions.
//
// The reciprocal comes from a per-block table: the dequantized scale
// p = RN32(E4M3(s_g) * s_t) takes at most 127 values per tensor (one per
// finite E4M3 code), so each block computes inv[c] = RN32(1/p_c) once, with
// the correctly rounded division, and every group looks its reciprocal up.  A
// zero p (zero group scale or zero tensor scale) gets inv = 0, which turns
// every element into a signed zero and hence into the code signbit(x) << 3,
// as the method requires.  (Measured against two divisions per lane and one
// load in flight: both passes together 7-11 % faster at K = 4096 and 5120,
// equal at K = 12288, outputs bit-identical.)
template <bool kBF16, int U>
__global__ __launch_bounds__(kThreads) void encode_kernel(
    const uint4* __restrict__ x, int64_t nvec, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale, int static_scale,
    const uint32_t* __restrict__ partial, int npartial) {
  constexpr int LPG = kBF16 ? 2 : 4;   // lanes per 16-element group
  constexpr int EPL = 16 / LPG;        // elements per lane
  __shared__ float inv_tab[128];
  float s_t;
  if (static_scale) {
    s_t = *tensor_scale;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) m = m > partial[i] ? m : partial[i];
    m = block_max_u32(m);
    s_t = __uint_as_float(m) / 2688.0f;  // 2688 = 6 * 448
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  }
  const float d = 6.0f * s_t;
  if (threadIdx.x < 128) {
    const float p = dec_e4m3(threadIdx.x) * s_t;
    inv_tab[threadIdx.x] = p == 0.0f ? 0.0f : 1.0f / p;
  }
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
      float v[EPL];
      float a;
      if (kBF16) {
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
        u16x2 mx = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
        for (int j = 1; j < 4; ++j)
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
        a = __uint_as_float(uint32_t(mx[0] > mx[1] ? mx[0] : mx[1]) << 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = __uint_as_float(w[j] << 16);
          v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
      } else {
        v[0] = __uint_as_float(t.x);
        v[1] = __uint_as_float(t.y);
        v[2] = __uint_as_float(t.z);
        v[3] = __uint_as_float(t.w);
        a = 0.0f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) a = __builtin_fmaxf(a, __builtin_fabsf(v[j]));
      }
#pragma unroll
      for (int o = 1; o < LPG; o <<= 1) a = __builtin_fmaxf(a, __shfl_xor(a, o, 64));
      const uint32_t sc = (d == 0.0f) ? 0u : enc_e4m3(a / d);
      const float inv = inv_tab[sc];
      float y[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) y[j] = v[j] * inv;
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
      if (kBF16) {
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4 % EPL], y[5 % EPL], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6 % EPL], y[7 % EPL], 1.0f, 3);
      }
      if (kBF16)
        reinterpret_cast<uint32_t*>(codes)[i] = w;
      else
        reinterpret_cast<uint16_t*>(codes)[i] = static_cast<uint16_t>(w);
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
