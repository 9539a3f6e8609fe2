// Offline weight preparation for the weight-only decode formats (not timed).
//
// INT4 group-128 (MARLIN article, abeam.tech, "データの扱い方": 4-bit weights
// with group size 128): symmetric round-to-nearest with a bf16 scale equal to
// the group's absolute maximum over 7.  One wavefront per group; lane l owns
// columns 2l and 2l+1 and writes one code byte, so stores are coalesced.
//
// LUT2 (KLLM article, aibr.jp, sections 1 and 3: K-means quantization into a
// codebook of centroids plus an index matrix; Disaggregated Quantization:
// 2-bit LUT decode weights): 4 centroids per row from 10 Lloyd iterations.
//   kernel 1  one workgroup per row selects the four quantile order
//             statistics sorted(w)[floor((2j+1) k/8)] by a 4 x 8-bit radix
//             select over monotone integer keys (LDS histograms).
//   kernel 2  one thread per row runs the Lloyd iterations in fp64.  The
//             cluster sums are taken one weight at a time in ascending
//             column order, which fixes the rounding of every mean.
//   kernel 3  one thread per output byte re-assigns 4 weights to the
//             nearest bf16 centroid (ties to the lower index).
// This translation unit is compiled with -ffp-contract=off.
#include "qlin_internal.hpp"

namespace qlin {
namespace {

// ------------------------------------------------------------------ INT4 --
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// kPrune: 2:4 magnitude pruning first (MARLIN article, "データの扱い方":
// Sparse-MARLIN's 2:4 structured sparsity).  Of every four consecutive
// columns the two of largest |w| are kept (ties to the lower column) and the
// other two become zero before the group is quantized; a quad spans lanes
// 2j and 2j+1, which swap their pair of values to rank all four.
template <bool kPrune>
__global__ __launch_bounds__(256) void int4_kernel(const float* __restrict__ w, int64_t n,
                                                   int64_t k, uint8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t G = k / 128;
  const int64_t grp = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (grp >= n * G) return;   // wave-uniform: whole wavefronts exit together
  const int64_t row = grp / G, g = grp % G;
  float2 v = reinterpret_cast<const float2*>(w + row * k + g * 128)[lane];
  if (kPrune) {
    const float o0 = __shfl_xor(v.x, 1, 64), o1 = __shfl_xor(v.y, 1, 64);
    // quad columns 0..3: this lane holds 2 (lane & 1) and 2 (lane & 1) + 1
    const int c0 = 2 * (lane & 1);
    const float q[4] = {(lane & 1) ? o0 : v.x, (lane & 1) ? o1 : v.y,
                        (lane & 1) ? v.x : o0, (lane & 1) ? v.y : o1};
    auto kept = [&](int c) {
      int beaten = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __builtin_fabsf(q[e]), ac = __builtin_fabsf(q[c]);
        beaten += (ae > ac || (ae == ac && e < c)) ? 1 : 0;
      }
      return beaten < 2;
    };
    if (!kept(c0)) v.x = 0.0f;
    if (!kept(c0 + 1)) v.y = 0.0f;
  }
  float a = __builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off, 64));
  const uint32_t sb = bf16_rne_bits(a / 7.0f);
  const float s = __uint_as_float(sb << 16);
  int q0 = 0, q1 = 0;
  if (s != 0.0f) {
    q0 = static_cast<int>(__builtin_rintf(v.x / s));
    q1 = static_cast<int>(__builtin_rintf(v.y / s));
    q0 = q0 < -7 ? -7 : (q0 > 7 ? 7 : q0);
    q1 = q1 < -7 ? -7 : (q1 > 7 ? 7 : q1);
  }
  codes[row * (k / 2) + g * 64 + lane] = static_cast<uint8_t>((q0 + 8) | ((q1 + 8) << 4));
  if (lane == 0) scales[row * G + g] = static_cast<uint16_t>(sb);
}

// ------------------------------------------------------------------ LUT2 --
constexpr int kSelThreads = 256;

// Monotone key: unsigned order of keys equals numeric order of floats, with
// -0.0 folded onto +0.0 so a zero quantile is always +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

__global__ __launch_bounds__(kSelThreads) void lut2_select_kernel(const float* __restrict__ w,
                                                                  int64_t k,
                                                                  double* __restrict__ cinit) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t prefix[4], rank[4];
  const int64_t row = blockIdx.x;
  const float* wr = w + row * k;
  if (threadIdx.x < 4) {
    prefix[threadIdx.x] = 0;
    rank[threadIdx.x] = static_cast<uint32_t>(((2 * threadIdx.x + 1) * k) / 8);
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 4 * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (32 - 8 * pass));
    for (int64_t i = threadIdx.x; i < k; i += kSelThreads) {
      const uint32_t key = float_key(wr[i]);
      const uint32_t digit = (key >> shift) & 0xFFu;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((key & hmask) == prefix[j]) atomicAdd(&hist[j][digit], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 4) {
      const int j = threadIdx.x;
      uint32_t r = rank[j], d = 0;
      while (d < 255 && hist[j][d] <= r) {
        r -= hist[j][d];
        ++d;
      }
      rank[j] = r;
      prefix[j] |= d << shift;
    }
    __syncthreads();
  }
  if (threadIdx.x < 4) cinit[row * 4 + threadIdx.x] = static_cast<double>(key_float(prefix[threadIdx.x]));
}

__device__ __forceinline__ int nearest4(double x, const double c[4]) {
  int best = 0;
  double bd = __builtin_fabs(x - c[0]);
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    const double d = __builtin_fabs(x - c[j]);
    if (d < bd) {
      bd = d;
      best = j;
    }
  }
  return best;
}

__global__ __launch_bounds__(64) void lut2_lloyd_kernel(const float* __restrict__ w, int64_t n,
                                                        int64_t k, const double* __restrict__ cinit,
                                                        uint16_t* __restrict__ centroids) {
  const int64_t row = int64_t(blockIdx.x) * 64 + threadIdx.x;
  if (row >= n) return;
  const float* wr = w + row * k;
  double c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = cinit[row * 4 + j];
  for (int it = 0; it < 10; ++it) {
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    int64_t cnt[4] = {0, 0, 0, 0};
    for (int64_t i = 0; i < k; ++i) {
      const double x = static_cast<double>(wr[i]);
      const int j = nearest4(x, c);
      // ascending-column sequential sum per cluster
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t == j) {
          s[t] = s[t] + x;
          cnt[t] += 1;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (cnt[j] > 0) c[j] = s[j] / static_cast<double>(cnt[j]) + 0.0;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    centroids[row * 4 + j] = static_cast<uint16_t>(bf16_rne_bits(static_cast<float>(c[j])));
}

__global__ __launch_bounds__(256) void lut2_assign_kernel(const float* __restrict__ w, int64_t n,
                                                          int64_t k,
                                                          const uint16_t* __restrict__ centroids,
                                                          uint8_t* __restrict__ idx) {
  const int64_t bytes = n * k / 4;
  for (int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b < bytes;
       b += int64_t(gridDim.x) * blockDim.x) {
    const int64_t row = b / (k / 4);
    double c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c[j] = static_cast<double>(__uint_as_float(uint32_t(centroids[row * 4 + j]) << 16));
    const float4 v = reinterpret_cast<const float4*>(w)[b];
    const uint32_t o = uint32_t(nearest4(v.x, c)) | (uint32_t(nearest4(v.y, c)) << 2) |
                       (uint32_t(nearest4(v.z, c)) << 4) | (uint32_t(nearest4(v.w, c)) << 6);
    idx[b] = static_cast<uint8_t>(o);
  }
}

}  // namespace

hipError_t launch_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* codes,
                                uint16_t* scales, bool prune24, hipStream_t s) {
  const int64_t groups = n * (k / 128);
  const int64_t blocks = (groups + 3) / 4;
  if (prune24)
    int4_kernel<true><<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, n, k, codes, scales);
  else
    int4_kernel<false><<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, n, k, codes, scales);
  return hipGetLastError();
}

size_t lut2_workspace(int64_t n, int64_t) { return size_t(n) * 4 * sizeof(double); }

hipError_t launch_fit_lut2(const float* w, int64_t n, int64_t k, uint8_t* idx,
                           uint16_t* centroids, void* ws, hipStream_t s) {
  double* cinit = static_cast<double*>(ws);
  lut2_select_kernel<<<static_cast<unsigned>(n), kSelThreads, 0, s>>>(w, k, cinit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lut2_lloyd_kernel<<<static_cast<unsigned>((n + 63) / 64), 64, 0, s>>>(w, n, k, cinit, centroids);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t blocks = (n * k / 4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  lut2_assign_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, n, k, centroids, idx);
  return hipGetLastError();
}

}  // namespace qlin
