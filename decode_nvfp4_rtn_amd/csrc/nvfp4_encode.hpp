// NVFP4 round-to-nearest encoding steps (Mix-Quant technical summary,
// gist.science, section 2 "Method", hybrid-precision strategy: one E4M3 scale
// per 16-element group plus an fp32 tensor scale), shared by the activation
// quantizer (quantize.hip) and the W4A4 GEMM that quantizes its activation
// operand as it loads it (gemm_w4a4.hip), so that both produce the same codes.
// The binary32 operation order is the one include/qlin.h states for
// quantize_nvfp4.  Translation units that include this header are compiled
// without fast-math and with -ffp-contract=off: every division is the
// correctly rounded binary32 division and no multiply is fused into an add.
#pragma once

#include "qlin_internal.hpp"

namespace qlin {

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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Maximum over a block of NT threads (all of them must call).
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t sh[NT / 64];
  v = wave_max_u32(v);
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  uint32_t r = sh[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = r > sh[i] ? r : sh[i];
  __syncthreads();
  return r;
}

// Tensor scale s_t = amax / (6 * 448) from the amax pass's partial maxima
// (bit patterns of non-negative floats, which order like unsigned integers);
// every thread of the block of NT threads returns it.
template <int NT>
__device__ __forceinline__ float tensor_scale_from_partials(const uint32_t* partial,
                                                            int npartial) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npartial; i += NT) m = m > partial[i] ? m : partial[i];
  m = block_max_u32<NT>(m);
  return __uint_as_float(m) / 2688.0f;  // 2688 = 6 * 448
}

// The reciprocal of every dequantized group scale: the scale p =
// RN32(E4M3(c) * s_t) takes at most 127 values per tensor (one per finite
// E4M3 code c), so inv[c] = RN32(1 / p) is computed once per block (threads
// 0..127; the caller synchronises before use) and every group looks its
// reciprocal up.  A zero p (zero group scale or zero tensor scale) gets
// inv = 0, which turns every element into a signed zero and hence into the
// code signbit(x) << 3, as the method requires.
__device__ __forceinline__ void fill_inv_table(float* inv_tab, float s_t) {
  if (threadIdx.x < 128) {
    const float p = dec_e4m3(threadIdx.x) * s_t;
    inv_tab[threadIdx.x] = p == 0.0f ? 0.0f : 1.0f / p;
  }
}

// E2M1 encoding uses v_cvt_scalef32_pk_fp4_f32 with scale 1.0: two binary32
// values per instruction (the first into the low nibble) into one byte of
// the destination: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code,
// saturating at 6, sign copied also for results that round to zero.  An
// exhaustive sweep of every non-NaN binary32 pattern on gfx950 found it
// identical to the comparison chain  code = (a>.25)+(a>=.75)+(a>1.25)+
// (a>=1.75)+(a>2.5)+(a>=3.5)+(a>5), a = |y|, with the sign bit of y.
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&y)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

typedef unsigned short qlin_u16x2 __attribute__((ext_vector_type(2)));

// Half of a 16-element group: 8 bf16 values (one 16-byte vector, element 2j
// in the low half of dword j) whose other 8 values the lane (lane ^ 1) holds;
// both lanes must be active.  Returns the 8 E2M1 codes (element 2j in the low
// nibble of byte j) and sets sc to the group's E4M3 scale code; d = 6 s_t.
__device__ __forceinline__ uint32_t encode8_bf16(const uint4& t, float d, const float* inv_tab,
                                                 uint32_t& sc) {
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
  // max |x| of the 8 values on the bf16 bit patterns (sign cleared)
  qlin_u16x2 mx = __builtin_bit_cast(qlin_u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int j = 1; j < 4; ++j)
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(qlin_u16x2, w[j] & 0x7FFF7FFFu));
  float a = __uint_as_float(uint32_t(mx[0] > mx[1] ? mx[0] : mx[1]) << 16);
  a = __builtin_fmaxf(a, __shfl_xor(a, 1, 64));
  sc = (d == 0.0f) ? 0u : enc_e4m3(a / d);
  const float inv = inv_tab[sc];
  float y[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    y[2 * j] = __uint_as_float(w[j] << 16) * inv;
    y[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u) * inv;
  }
  return e2m1_pack8(y);
}

// A whole 16-element group of bf16 values held by one lane (a: elements
// 0..7, b: 8..15, element 2j in the low half of dword j): the same steps as
// encode8_bf16, the two halves' maxima combined with the same fmaxf that
// combines the two lanes' there (so NaN inputs give the same scale).
// Returns the 16 E2M1 codes in two dwords (c0: elements 0..7, c1: 8..15)
// and sets sc to the E4M3 scale code.
__device__ __forceinline__ void encode16_bf16(const uint4& a, const uint4& b, float d,
                                              const float* inv_tab, uint32_t& c0, uint32_t& c1,
                                              uint32_t& sc) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  auto half_max = [&](int h) {
    qlin_u16x2 mx = __builtin_bit_cast(qlin_u16x2, w[4 * h] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 4; ++j)
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(qlin_u16x2, w[4 * h + j] & 0x7FFF7FFFu));
    return __uint_as_float(uint32_t(mx[0] > mx[1] ? mx[0] : mx[1]) << 16);
  };
  const float amax = __builtin_fmaxf(half_max(0), half_max(1));
  sc = (d == 0.0f) ? 0u : enc_e4m3(amax / d);
  const float inv = inv_tab[sc];
  float y[2][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    y[j >> 2][2 * (j & 3)] = __uint_as_float(w[j] << 16) * inv;
    y[j >> 2][2 * (j & 3) + 1] = __uint_as_float(w[j] & 0xFFFF0000u) * inv;
  }
  c0 = e2m1_pack8(y[0]);
  c1 = e2m1_pack8(y[1]);
}

}  // namespace qlin
