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

// Activation fragments staged as whole rows.  A fragment load (lane l: token
// l % 16, k 32 s + 8 (l / 16)) sends adjacent lanes to different rows, which
// the L1 cannot merge: measured with a [16, K] bf16 activation read by every
// block, it costs 4x the L1 tag lookups and 2-2.8x the address-unit time of
// the same bytes loaded as rows (and, with rows 24-30 KiB apart, twice the
// time).  rows_load issues row loads instead -- lane l: token
// m0 + 16 mt + 4 q + l / 16 (clamped to a valid row) at k 8 (l % 16) of a
// group, for the NQ row quads that hold tokens, or with one token (NQ = 0)
// lane l: group l / 16 -- into the registers the fragments will occupy;
// rows_stage then sends each group through a wave-private LDS tile of 16 rows
// x 256 bytes whose 16-byte slots are XOR-swizzled by row (conflict-free row
// writes and fragment reads) and reads its four fragments back.  LDS
// operations of one wave run in order, so one tile serves all the groups and
// no barrier is needed.  Lanes of tokens past the staged rows read the last
// staged row: their outputs are never stored.  The NG groups are
// g0 + min(i, ng - 1), clamped to G - 1.
__device__ __forceinline__ int stage_slot(int row, int chunk) { return row * 256 + 16 * (chunk ^ row); }

template <int NG, int MT, int NQ>
__device__ __forceinline__ void rows_load(const uint16_t* __restrict__ x, int M, int m0, int K,
                                          int g0, int ng, int G, int lane,
                                          bf16x8_t (&f)[NG][4][MT]) {
  static_assert(NQ <= 4 && (NQ > 0 || (MT == 1 && NG <= 4)), "row quads");
  auto grp = [&](int i) { return min(g0 + min(i, ng - 1), G - 1); };
  auto ld = [](const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return as_bf16x8(u32x4{v.x, v.y, v.z, v.w});
  };
  if constexpr (NQ == 0) {
    f[0][0][0] = ld(x + int64_t(m0) * K + grp(lane >> 4) * 128 + 8 * (lane & 15));
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          f[i][q][mt] = ld(x + int64_t(min(m0 + 16 * mt + 4 * q + (lane >> 4), M - 1)) * K +
                           grp(i) * 128 + 8 * (lane & 15));
  }
}

// Fragment p of a group read back by rows_stage: dense MFMA operand p = s
// (lane l: chunk 4 s + l / 16, i.e. k 32 s + 8 (l / 16)); 2:4 sparse MFMA
// operand (kSp) piece p = 2 h + j of half h (lane l: chunk 8 h + 2 (l / 16)
// + j, i.e. k 64 h + 16 (l / 16) + 8 j).
template <bool kSp>
__device__ __forceinline__ int frag_chunk(int p, int lane) {
  return kSp ? 8 * (p >> 1) + 2 * (lane >> 4) + (p & 1) : 4 * p + (lane >> 4);
}

template <int NG, int MT, int NQ, bool kSp = false>
__device__ __forceinline__ void rows_stage(uint8_t* st, int lane, bf16x8_t (&f)[NG][4][MT]) {
  auto u4 = [](const bf16x8_t& v) { return __builtin_bit_cast(uint4, v); };
  auto rd = [&](int row, int chunk) {
    const uint4 v = *reinterpret_cast<const uint4*>(st + stage_slot(row, chunk));
    return as_bf16x8(u32x4{v.x, v.y, v.z, v.w});
  };
  if constexpr (NQ == 0) {
    *reinterpret_cast<uint4*>(st + stage_slot(lane >> 4, lane & 15)) = u4(f[0][0][0]);
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
      for (int p = 0; p < 4; ++p) f[i][p][0] = rd(i, frag_chunk<kSp>(p, lane));
  } else {
    const int row = min(lane & 15, 4 * NQ - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < NG; ++i) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          *reinterpret_cast<uint4*>(st + stage_slot(4 * q + (lane >> 4), lane & 15)) =
              u4(f[i][q][mt]);
#pragma unroll
        for (int p = 0; p < 4; ++p) f[i][p][mt] = rd(row, frag_chunk<kSp>(p, lane));
      }
  }
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
