// Device helpers shared by the weight-only decode kernels (gemm_decode.hip,
// gemm_sparse.hip).  Internal; not part of the public ABI.
#pragma once

#include "qlin_internal.hpp"

namespace qlin {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KW = 8;  // wavefronts per block (k split)

// Buffer resource word 3 for raw 32-bit buffer loads, and the non-temporal
// cache policy for streamed weights (read once).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kPolicyNT = 2;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// A 32-bit constant held in a VGPR, so that two-constant operations such as
// (w & mask) | bias can use one v_and_or_b32 (VOP3 on this target accepts no
// literal constants and one scalar operand).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
  return v;
}

// INT4: dword of 8 nibbles (pairs at bits (4j, 16+4j)) -> bf16 (128+u) x 8
__device__ __forceinline__ bf16x8_t int4_operand(uint32_t w, uint32_t mask, uint32_t bias) {
  u32x4 v;
  v[0] = (w & mask) | bias;
  v[1] = ((w >> 4) & mask) | bias;
  v[2] = ((w >> 8) & mask) | bias;
  v[3] = ((w >> 12) & mask) | bias;
  return as_bf16x8(v);
}

// ---------------------------------------------------------------- host --

constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Chunk of groups whose weight loads a wave issues at once.  Loads in flight
// hide HBM latency; a chunk boundary costs roughly one extra round trip and a
// padded slot one wasted load, so pick the size that minimises the sum.
int pick_chunk(int gpw, int cap) {
  static const int kSizes[] = {2, 4, 6, 8, 12, 16};
  int best = 2, best_cost = 1 << 30;
  for (int w : kSizes) {
    if (w > cap) break;
    const int chunks = (gpw + w - 1) / w;
    const int cost = chunks * w + 2 * chunks;
    if (cost < best_cost) best = w, best_cost = cost;
  }
  return best;
}

}  // namespace
}  // namespace qlin
