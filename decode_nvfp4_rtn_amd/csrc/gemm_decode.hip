// Weight-only decode GEMV / skinny GEMM for gfx950: INT4 group-128 (W4A16)
// and 2-bit codebook (LUT2) weights against bf16 activations.
//
// Small-batch decode re-reads every weight for few tokens, so it is bound by
// weight reads from HBM (Disaggregated Quantization, opening paragraph;
// MARLIN article, "基本アイデア").  Shrinking weights to 4 or 2 bits cuts
// those reads; the kernel must then dequantize fast enough to keep the HBM
// stream saturated (MARLIN article, "課題": dequantization, operand loads and
// scale handling become the bottleneck).
//
// Design (gfx950):
// * Weights are streamed once, in the repacked lane order, with one 16-byte
//   (INT4) or 8-byte (LUT2) load per lane per (16-row tile, 128-k group):
//   each wavefront load is one contiguous 1 KiB / 512 B run.
// * Dequantization builds bf16 MFMA operands with a handful of bit
//   operations per pair of weights, no per-element conversion:
//     INT4: (dword >> 4j) & 0x000F000F | 0x43004300 is the bf16 pair
//           (128 + u0, 128 + u1), u = q + 8.  The MFMA then gives
//           sum x (128 + u); subtracting 136 * sum x (taken from one more
//           MFMA against an all-ones operand) yields sum x q exactly up to
//           fp32 rounding, and the group scale is applied in fp32 once per
//           128-k group.
//     LUT2: the row's 4 bf16 centroids, split into a low-byte and a
//           high-byte table, are looked up with v_perm_b32 (4 indices per
//           instruction) and interleaved into bf16 pairs with two more
//           v_perm_b32: 1.4 VALU operations per weight.
// * The multiply-adds run on v_mfma_f32_16x16x32_bf16 (weights are the A
//   operand, 16 rows; activations the B operand, up to 16 tokens per m-tile),
//   so the VALU only dequantizes.  Batches up to 32 tokens use two m-tiles per
//   pass; larger batches take several passes.
// * A block of KW wavefronts owns NTB row tiles; the waves split k (as
//   MARLIN splits one output tile over several warps, "スレッドブロックと
//   ワープの配置") and their partial sums are added in LDS in a fixed order,
//   so results are deterministic and no atomics are used.
#include "qlin_internal.hpp"

namespace qlin {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KW = 8;  // wavefronts per block (k split)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// bf16 MFMA B operand: 8 activations x[m][k0 .. k0+8) (zero when m >= M)
__device__ __forceinline__ bf16x8_t load_x(const uint16_t* __restrict__ x, int m, int M, int K,
                                           int k0) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M) {
    const uint4 t = *reinterpret_cast<const uint4*>(x + int64_t(m) * K + k0);
    v = u32x4{t.x, t.y, t.z, t.w};
  }
  return as_bf16x8(v);
}

// INT4: dword of 8 nibbles (pairs at bits (4j, 16+4j)) -> bf16 (128+u) x 8
__device__ __forceinline__ bf16x8_t int4_operand(uint32_t w) {
  u32x4 v;
  v[0] = (w & 0x000F000Fu) | 0x43004300u;
  v[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  v[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  v[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return as_bf16x8(v);
}

template <int MT, int NTB, bool kBF16Out>
__device__ __forceinline__ void reduce_store(floatx4 (&tot)[NTB][MT], int nt0, int m0, int M,
                                             int N, void* __restrict__ y) {
  __shared__ floatx4 red[KW][NTB][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][nt][mt][lane] = tot[nt][mt];
  __syncthreads();
  for (int t = threadIdx.x; t < NTB * MT * 64; t += KW * 64) {
    const int nt = t / (MT * 64), mt = (t / 64) % MT, ln = t % 64;
    floatx4 s = red[0][nt][mt][ln];
#pragma unroll
    for (int w = 1; w < KW; ++w) s += red[w][nt][mt][ln];
    const int n = (nt0 + nt) * 16 + 4 * (ln >> 4);
    const int m = m0 + mt * 16 + (ln & 15);
    if (m < M && n < N) {
      if (kBF16Out) {
        uint2 o;
        o.x = f32_to_bf16_rne(s[0]) | (f32_to_bf16_rne(s[1]) << 16);
        o.y = f32_to_bf16_rne(s[2]) | (f32_to_bf16_rne(s[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + int64_t(m) * N + n) = o;
      } else {
        *reinterpret_cast<floatx4*>(static_cast<float*>(y) + int64_t(m) * N + n) = s;
      }
    }
  }
}

template <int MT, int NTB, bool kBF16Out>
__global__ __launch_bounds__(KW * 64) void w4a16_kernel(const uint16_t* __restrict__ x,
                                                        const uint8_t* __restrict__ blob,
                                                        int64_t codes_off, int64_t sc_off, int M,
                                                        int m0, int N, int K,
                                                        void* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = K / 128;
  const int gpw = (G + KW - 1) / KW;
  const int g0 = wave * gpw, g1 = min(G, g0 + gpw);
  const int nt0 = blockIdx.x * NTB;
  const int NT16 = N / 16;
  const uint4* codes = reinterpret_cast<const uint4*>(blob + codes_off);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(blob + sc_off);
  const bf16x8_t ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  floatx4 tot[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int g = g0; g < g1; ++g) {
    uint4 wv[NTB];
    uint2 sv[NTB];
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt) {
      const int tile = min(nt0 + nt, NT16 - 1);
      wv[nt] = load_nt16(&codes[(int64_t(tile) * G + g) * 64 + lane]);
      sv[nt] = *reinterpret_cast<const uint2*>(scales + (int64_t(tile) * G + g) * 16 +
                                               4 * (lane >> 4));
    }
    bf16x8_t xf[4][MT];
    floatx4 xs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      xs[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        xf[s][mt] = load_x(x, m0 + mt * 16 + (lane & 15), M, K, g * 128 + 32 * s + 8 * (lane >> 4));
        xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, xf[s][mt], xs[mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt) {
      floatx4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      const uint32_t wd[4] = {wv[nt].x, wv[nt].y, wv[nt].z, wv[nt].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t a = int4_operand(wd[s]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xf[s][mt], acc[mt], 0, 0, 0);
      }
      const float sc[4] = {__uint_as_float(sv[nt].x << 16), __uint_as_float(sv[nt].x & 0xFFFF0000u),
                           __uint_as_float(sv[nt].y << 16), __uint_as_float(sv[nt].y & 0xFFFF0000u)};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float off = 136.0f * xs[mt][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[nt][mt][i] += sc[i] * (acc[mt][i] - off);
      }
    }
  }
  reduce_store<MT, NTB, kBF16Out>(tot, nt0, m0, M, N, y);
}

template <int MT, int NTB, bool kBF16Out>
__global__ __launch_bounds__(KW * 64) void lut2_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ blob,
                                                       int64_t codes_off, int64_t book_off, int M,
                                                       int m0, int N, int K,
                                                       void* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = K / 128;
  const int gpw = (G + KW - 1) / KW;
  const int g0 = wave * gpw, g1 = min(G, g0 + gpw);
  const int nt0 = blockIdx.x * NTB;
  const int NT16 = N / 16;
  const uint2* codes = reinterpret_cast<const uint2*>(blob + codes_off);
  const uint2* book = reinterpret_cast<const uint2*>(blob + book_off);

  uint32_t lo_t[NTB], hi_t[NTB];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int tile = min(nt0 + nt, NT16 - 1);
    const uint2 b = book[tile * 16 + (lane & 15)];
    lo_t[nt] = b.x;
    hi_t[nt] = b.y;
  }

  floatx4 tot[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int g = g0; g < g1; ++g) {
    uint2 wv[NTB];
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt) {
      const int tile = min(nt0 + nt, NT16 - 1);
      wv[nt] = load_nt8(&codes[(int64_t(tile) * G + g) * 64 + lane]);
    }
    bf16x8_t xf[4][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xf[s][mt] = load_x(x, m0 + mt * 16 + (lane & 15), M, K, g * 128 + 32 * s + 8 * (lane >> 4));
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt) {
      const uint32_t wd[2] = {wv[nt].x, wv[nt].y};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        u32x4 op[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t sel = (wd[d] >> (2 * j)) & 0x03030303u;
          const uint32_t lo = __builtin_amdgcn_perm(0u, lo_t[nt], sel);
          const uint32_t hi = __builtin_amdgcn_perm(0u, hi_t[nt], sel);
          op[j >> 1][2 * (j & 1)] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
          op[j >> 1][2 * (j & 1) + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
          const bf16x8_t a = as_bf16x8(op[sl]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            tot[nt][mt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xf[2 * d + sl][mt], tot[nt][mt], 0, 0, 0);
        }
      }
    }
  }
  reduce_store<MT, NTB, kBF16Out>(tot, nt0, m0, M, N, y);
}

template <bool kLut, int MT, int NTB>
hipError_t launch_decode(const void* x, const uint8_t* blob, const BlobLayout& L, int M, int m0,
                         int N, int K, void* y, int y_dtype, hipStream_t s) {
  const int blocks = (N / 16 + NTB - 1) / NTB;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (kLut) {
    if (y_dtype == 1)
      lut2_kernel<MT, NTB, true><<<blocks, KW * 64, 0, s>>>(xp, blob, L.codes_off, L.aux_off, M,
                                                            m0, N, K, y);
    else
      lut2_kernel<MT, NTB, false><<<blocks, KW * 64, 0, s>>>(xp, blob, L.codes_off, L.aux_off, M,
                                                             m0, N, K, y);
  } else {
    if (y_dtype == 1)
      w4a16_kernel<MT, NTB, true><<<blocks, KW * 64, 0, s>>>(xp, blob, L.codes_off, L.aux_off, M,
                                                             m0, N, K, y);
    else
      w4a16_kernel<MT, NTB, false><<<blocks, KW * 64, 0, s>>>(xp, blob, L.codes_off, L.aux_off,
                                                              M, m0, N, K, y);
  }
  return hipGetLastError();
}

template <bool kLut>
hipError_t launch_decode_all(const void* x, const void* w_packed, int64_t m, int64_t n, int64_t k,
                             void* y, int y_dtype, hipStream_t s) {
  const BlobLayout L = blob_layout(kLut ? 2 : 1, n, k);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  for (int64_t m0 = 0; m0 < m; m0 += 32) {
    const int rows = static_cast<int>(m - m0 < 32 ? m - m0 : 32);
    hipError_t e;
    if (rows <= 16)
      e = launch_decode<kLut, 1, 1>(x, blob, L, int(m), int(m0), int(n), int(k), y, y_dtype, s);
    else
      e = launch_decode<kLut, 2, 1>(x, blob, L, int(m), int(m0), int(n), int(k), y, y_dtype, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_w4a16(const void* x, const void* w_packed, int64_t m, int64_t n, int64_t k,
                             void* y, int y_dtype, hipStream_t s) {
  return launch_decode_all<false>(x, w_packed, m, n, k, y, y_dtype, s);
}

hipError_t launch_gemm_lut2(const void* x, const void* w_packed, int64_t m, int64_t n, int64_t k,
                            void* y, int y_dtype, hipStream_t s) {
  return launch_decode_all<true>(x, w_packed, m, n, k, y, y_dtype, s);
}

}  // namespace qlin
