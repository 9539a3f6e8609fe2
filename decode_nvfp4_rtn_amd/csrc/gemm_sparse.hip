// 2:4 sparse W4A16 decode GEMV / skinny GEMM for gfx950 on the sparse MFMA.
//
// The MARLIN article ("データの扱い方"; "実験と結果") names Sparse-MARLIN:
// INT4 group-128 weights with 2:4 structured sparsity, which reads a quarter
// fewer bytes per dense weight than dense INT4 (two 4-bit codes and two
// 2-bit positions per four weights, plus the group scales).  gfx950 runs 2:4
// sparse operands natively: v_smfmac_f32_16x16x64_bf16 takes the A operand
// compressed (8 bf16 per lane for 16 rows x 64 dense k) with a 2-bit position
// per value in an index register, and a dense 64 x 16 B operand.  The kept
// codes are dequantized as in dense INT4 (bf16 128 + u, half the VALU work
// per dense weight) and the positions go to the matrix core untouched.
//
// Operand layout of the sparse MFMA (measured on the device with one-hot
// operands; lane l, r = l % 16, q = l / 16): A element e = 2 (2h + b) + j
// (h, b, j in {0, 1}) of lane l is row r at dense k = 16 (2 (q % 2) + h) +
// 8 (q / 2) + 4 b + p_e, with the position p_e at bits 2e..2e+1 of the index
// operand; B lane l holds column l % 16 at k = 16 q + 0..15; D as the dense
// 16 x 16 MFMAs (lane l, register i: row 4 q + i, column r).  The repacker
// writes codes and positions in exactly this order.
//
// Offsets: dense INT4 seeds each group's MFMA chain with -136 * sum x, which
// depends only on the activations.  Here the kept positions differ per row,
// so each chain starts with one more sparse MFMA of an all -136 operand with
// the same positions (sum over the kept k of -136 x).
#include "qlin_internal.hpp"
#include <algorithm>
#include <climits>

#include "decode_ops.hpp"

namespace qlin {
namespace {

typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// B operand of the 64-k half s of group g (xr already points at row and
// k offset 16 (lane / 16)): 16 consecutive bf16, two 16-byte loads
__device__ __forceinline__ bf16x16_t load_xh(const uint16_t* xr, int g, int s) {
  const uint4* p = reinterpret_cast<const uint4*>(xr + g * 128 + 64 * s);
  const uint4 a = p[0], b = p[1];
  return __builtin_bit_cast(bf16x16_t, u32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w});
}

// two 8-element pieces -> one 16-element sparse-MFMA B operand
__device__ __forceinline__ bf16x16_t join16(bf16x8_t a, bf16x8_t b) {
  const uint4 u = __builtin_bit_cast(uint4, a), v = __builtin_bit_cast(uint4, b);
  return __builtin_bit_cast(bf16x16_t, u32x8{u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w});
}

// codes (dword per 64-k half), positions and the 4 scales of one
// (row tile, group) as this lane holds them
struct SpGroup {
  uint2 c;
  uint32_t m;
  uint2 s;
};

struct SpRsrc {
  __amdgpu_buffer_rsrc_t c, s;
};

// buffer resources of row tile t: scalar tile and group offsets
__device__ __forceinline__ SpRsrc sp_rsrc(const uint8_t* blob, int64_t codes_off, int64_t aux_off,
                                          int64_t t, int G) {
  SpRsrc R;
  R.c = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob + codes_off + t * G * 768), 0,
                                          G * 768, kRsrcWord3);
  R.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob + aux_off + t * G * 32), 0,
                                          G * 32, kRsrcWord3);
  return R;
}

// codes and positions of this lane in one 12-byte load, then the scales
__device__ __forceinline__ void sp_load(SpGroup& A, const SpRsrc& R, int lane, int gc) {
  const u32x3 c = __builtin_amdgcn_raw_buffer_load_b96(R.c, lane * 12, gc * 768, kPolicyNT);
  A.c = make_uint2(c[0], c[1]);
  A.m = c[2];
  const u32x2 s = __builtin_amdgcn_raw_buffer_load_b64(R.s, (lane >> 4) * 8, gc * 32, 0);
  A.s = make_uint2(s[0], s[1]);
}

// sum over the group's kept k of x q for 16 rows x 16 columns: per 64-k half,
// the -136 seed and the (128 + u) operand against the same positions
__device__ __forceinline__ floatx4 sp_group(const SpGroup& A, const bf16x16_t (&xh)[2],
                                            bf16x8_t neg136, uint32_t mask, uint32_t bias) {
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int idx = int(s ? (A.m >> 16) : (A.m & 0xFFFFu));
    acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(neg136, xh[s], acc, idx, 0, 0);
    acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(int4_operand(s ? A.c.y : A.c.x, mask, bias),
                                                    xh[s], acc, idx, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ void scale_add(floatx4& tot, const floatx4& acc, uint2 sc, bool live) {
  const uint32_t s01 = live ? sc.x : 0u, s23 = live ? sc.y : 0u;
  const float f[4] = {__uint_as_float(s01 << 16), __uint_as_float(s01 & 0xFFFF0000u),
                      __uint_as_float(s23 << 16), __uint_as_float(s23 & 0xFFFF0000u)};
#pragma unroll
  for (int r = 0; r < 4; ++r) tot[r] = fmaf(f[r], acc[r], tot[r]);
}

template <bool kBF16Out>
__device__ __forceinline__ void store_one(void* y, int64_t idx, float v) {
  if (kBF16Out)
    static_cast<uint16_t*>(y)[idx] = to_bf16(v);
  else
    static_cast<float*>(y)[idx] = v;
}

// Persistent kernel for MT m-tiles (M <= 16 MT), K <= 128 * KW * GW per k
// slice and at least two row tiles per block, organised as the dense
// persistent kernel: wave w owns groups [GW w, GW w + GW) of its slice in
// every row tile and keeps their activation fragments in registers; blocks
// walk the row tiles with the next tile's weights in flight; 4 MT waves add
// the eight partial sums of a tile (one component and m-tile each).  The
// dequantized operand of a group is shared by the m-tiles.  With S > 1 k
// slices (the workspace entry point), block b serves slice b % S, walks
// tiles b / S, + gridDim.x / S, ... and stores the slice's fp32 partial sums
// to part[slice][m][n]; a second launch adds the slices.
constexpr int sp_blocks_per_cu(int gw, int mt) { return gw == 2 && mt == 1 ? 2 : 1; }

template <int GW, int MT, int XQ, bool kBF16Out>
__global__ __launch_bounds__(KW * 64, KW / 4 * sp_blocks_per_cu(GW, MT))
void sp24_persist_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ blob,
                         int64_t codes_off, int64_t aux_off, int M, int N, int K,
                         void* __restrict__ y, int S, float* __restrict__ part) {
  const uint32_t hdr = header_word(blob);   // tested before the first store
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = K / 128;
  const int sl = blockIdx.x % S;          // k slice: groups [KW GW sl, KW GW (sl + 1))
  const int g0 = (sl * KW + wave) * GW;
  const int T = N / 16;
  const int stride = gridDim.x / S;       // tile walkers per slice
  const uint32_t m136 = vconst(0xC308C308u);
  const bf16x8_t neg136 = as_bf16x8(u32x4{m136, m136, m136, m136});
  const uint32_t nib_mask = vconst(0x000F000Fu), bf16_128 = vconst(0x43004300u);

  struct Tile {
    SpGroup g[GW];
  };
  auto load = [&](Tile& A, int t) {
    const SpRsrc R = sp_rsrc(blob, codes_off, aux_off, t, G);
#pragma unroll
    for (int i = 0; i < GW; ++i) sp_load(A.g[i], R, lane, min(g0 + i, G - 1));
  };

  // activation operands: XQ >= 0 loads whole rows (XQ row quads per m-tile,
  // 0 for one token) and stages them through a wave-private LDS tile
  // (rows_stage, decode_ops.hpp), issued before and finished after the first
  // tile's weight loads; XQ < 0 loads the operands directly
  __shared__ __attribute__((aligned(16))) uint8_t xst[XQ >= 0 ? KW : 1][4096];
  bf16x16_t xh[MT][GW][2];
  Tile A, B;
  int t = blockIdx.x / S;
  if constexpr (XQ >= 0) {
    bf16x8_t f[GW][4][MT];
    rows_load<GW, MT, XQ>(x, M, 0, K, g0, GW, G, lane, f);
    load(A, t);
    __builtin_amdgcn_sched_barrier(0);
    rows_stage<GW, MT, XQ, true>(xst[wave], lane, f);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) xh[mt][i][h] = join16(f[i][2 * h][mt], f[i][2 * h + 1][mt]);
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* xr = x + int64_t(min(mt * 16 + (lane & 15), M - 1)) * K + 16 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s) xh[mt][i][s] = load_xh(xr, min(g0 + i, G - 1), s);
    }
    load(A, t);
  }
  // the header was loaded ahead of the activations (which the staging above
  // waits for): tested once here, for every store below
  const bool hdr_ok = header_word_ok(hdr, 3, N, K);

  // 65-float rows with one m-tile: the row-wise final sums below read them
  // free of bank conflicts
  __shared__ float red[2][KW][MT][4][MT == 1 ? 65 : 64];
  auto finish = [&](const Tile& A, int t, int slot, bool store) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      floatx4 acc[GW];
#pragma unroll
      for (int i = 0; i < GW; ++i)
        acc[i] = sp_group(A.g[i], xh[mt][i], neg136, nib_mask, bf16_128);
      floatx4 tot = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < GW; ++i) scale_add(tot, acc[i], A.g[i].s, g0 + i < G);
#pragma unroll
      for (int r = 0; r < 4; ++r) red[slot][wave][mt][r][lane] = tot[r];
    }
    __syncthreads();
    // (a blob of another format or shape is read but never stored from)
    // One m-tile: wave rq adds token rows 4 rq .. 4 rq + 3, all 16 columns,
    // so each store writes whole 32-byte row pieces (accumulator lane row +
    // 16 (column / 4), component column % 4, held that output), as in the
    // dense persistent kernel; two m-tiles keep one component per wave.
    if (wave < 4 * MT && store && hdr_ok) {
      const int mt = wave >> 2;
      const int mrow = MT == 1 ? 4 * (wave & 3) + (lane >> 4) : (lane & 15);
      const int col = MT == 1 ? (lane & 15) : 4 * (lane >> 4) + (wave & 3);
      const int r = col & 3, src = mrow + 16 * (col >> 2);
      float v[KW];
#pragma unroll
      for (int w = 0; w < KW; ++w) v[w] = red[slot][w][mt][r][src];
#pragma unroll
      for (int h = KW / 2; h >= 1; h /= 2)
#pragma unroll
        for (int w = 0; w < h; ++w) v[w] += v[w + h];
      const int m = mt * 16 + mrow, n = t * 16 + col;
      if (m < M) {
        if (S > 1)
          part[(int64_t(sl) * M + m) * N + n] = v[0];   // this slice's partial sum
        else
          store_one<kBF16Out>(y, int64_t(m) * N + n, v[0]);
      }
    }
  };

  // the launch guarantees gridDim.x / S <= T; the second tile of an iteration is
  // computed from clamped loads but not stored when it does not exist (no
  // branch around the waits, which would also wait for the prefetch)
  for (; t < T; t += 2 * stride) {
    load(B, min(t + stride, T - 1));
    __builtin_amdgcn_sched_barrier(0);
    finish(A, t, 0, true);
    load(A, min(t + 2 * stride, T - 1));
    __builtin_amdgcn_sched_barrier(0);
    finish(B, t + stride, 1, t + stride < T);
  }
}

// k-split kernel for every other shape: a block of KW waves owns NTB row tiles
// and MT m-tiles of the batch (rows m0 ..), the waves split k and walk their
// groups in chunks of WMAX whose weight loads are issued at once; the
// activation fragments of a group follow (small, cached).  Slots past the
// wave's range or past k read a clamped group and contribute zero.
template <int MT, int NTB, int WMAX, int XQ, bool kBF16Out>
__global__ __launch_bounds__(KW * 64) void sp24_ksplit_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ blob, int64_t codes_off,
    int64_t aux_off, int M, int m0, int N, int K, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = K / 128;
  const int gpw = (G + KW - 1) / KW;
  const int g0 = wave * gpw;
  const int nt0 = blockIdx.x * NTB;
  const int T = N / 16;
  const uint32_t m136 = vconst(0xC308C308u);
  const bf16x8_t neg136 = as_bf16x8(u32x4{m136, m136, m136, m136});
  const uint32_t nib_mask = vconst(0x000F000Fu), bf16_128 = vconst(0x43004300u);

  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xr[mt] = x + int64_t(min(m0 + mt * 16 + (lane & 15), M - 1)) * K + 16 * (lane >> 4);
  SpRsrc R[NTB];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
    R[nt] = sp_rsrc(blob, codes_off, aux_off, min(nt0 + nt, T - 1), G);

  floatx4 tot[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // XQ >= 0: the activation rows of a chunk's groups are loaded first and
  // staged (rows_stage) once the chunk's weight loads are in flight -- per
  // chunk with one m-tile; with two (whose registers hold one chunk's rows
  // only next to the rest) the launcher takes this form only when the
  // wave's groups fit one chunk, loaded ahead of the loop.  XQ < 0 loads
  // each group's operands directly.
  __shared__ __attribute__((aligned(16))) uint8_t xst[XQ >= 0 ? KW : 1][4096];
  bf16x8_t xpre[XQ >= 0 ? WMAX : 1][4][MT];
  if constexpr (XQ >= 0 && MT == 2) rows_load<WMAX, MT, XQ>(x, M, m0, K, g0, gpw, G, lane, xpre);

  uint32_t hdr = 0;   // header words (lane l: word l % 8)
  for (int c0 = 0; c0 < gpw; c0 += WMAX) {
    if constexpr (XQ >= 0 && MT == 1)
      rows_load<WMAX, MT, XQ>(x, M, m0, K, g0 + c0, gpw - c0, G, lane, xpre);
    SpGroup w[WMAX][NTB];
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int gc = min(g0 + min(c0 + i, gpw - 1), G - 1);
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) sp_load(w[i][nt], R[nt], lane, gc);
    }
    if (c0 == 0) hdr = header_word(blob);   // behind the first weights; tested before the store
    if constexpr (XQ >= 0) {
      __builtin_amdgcn_sched_barrier(0);   // the weight loads go out before the staging
      rows_stage<WMAX, MT, XQ, true>(xst[wave], lane, xpre);
    }
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int gc = min(g0 + min(c0 + i, gpw - 1), G - 1);
      const bool live = c0 + i < gpw && g0 + c0 + i < G;
      bf16x16_t xh[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          xh[mt][s] = XQ >= 0 ? join16(xpre[XQ >= 0 ? i : 0][2 * s][mt],
                                       xpre[XQ >= 0 ? i : 0][2 * s + 1][mt])
                              : load_xh(xr[mt], gc, s);
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          scale_add(tot[nt][mt], sp_group(w[i][nt], xh[mt], neg136, nib_mask, bf16_128),
                    w[i][nt].s, live);
    }
  }

  if (!header_word_ok(hdr, 3, N, K)) return;   // uniform: before the barrier below
  // KW partial sums -> LDS; wave c handles (row tile, m-tile, component) c, c + KW, ...
  __shared__ float red[KW][NTB][MT][4][64];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][nt][mt][r][lane] = tot[nt][mt][r];
  __syncthreads();
  for (int c = wave; c < NTB * MT * 4; c += KW) {
    const int nt = c / (MT * 4), mt = (c / 4) % MT, r = c % 4;
    float v[KW];
#pragma unroll
    for (int w = 0; w < KW; ++w) v[w] = red[w][nt][mt][r][lane];
#pragma unroll
    for (int h = KW / 2; h >= 1; h /= 2)
#pragma unroll
      for (int w = 0; w < h; ++w) v[w] += v[w + h];
    const int tile = nt0 + nt, m = m0 + mt * 16 + (lane & 15), n = tile * 16 + 4 * (lane >> 4) + r;
    if (tile < T && m < M) store_one<kBF16Out>(y, int64_t(m) * N + n, v[0]);
  }
}

// chunk cap: the chunk's weights (5 registers per group and row tile) and the
// accumulators must fit next to the fragments at two waves per SIMD
constexpr int sp_cap(int mt, int ntb) { return mt * ntb == 1 ? 8 : (mt * ntb == 2 ? 6 : 4); }

// row quads staged for `rows` tokens of one pass: 0 for one token, else
// 1, 2 or 4 per m-tile (-1: no staging)
inline int stage_quads(int rows, int mt) { return mt == 2 ? 4 : rows == 1 ? 0 : rows <= 4 ? 1 : rows <= 8 ? 2 : 4; }

template <int MT, int NTB, int W, int XQ>
hipError_t launch_sp24_ksplit_xq(const uint16_t* x, const uint8_t* blob, const BlobLayout& L,
                                 int M, int m0, int N, int K, void* y, int y_dtype, hipStream_t s) {
  const int blocks = (N / 16 + NTB - 1) / NTB;
  if (y_dtype == 1)
    sp24_ksplit_kernel<MT, NTB, W, XQ, true><<<blocks, KW * 64, 0, s>>>(
        x, blob, L.codes_off, L.aux_off, M, m0, N, K, y);
  else
    sp24_ksplit_kernel<MT, NTB, W, XQ, false><<<blocks, KW * 64, 0, s>>>(
        x, blob, L.codes_off, L.aux_off, M, m0, N, K, y);
  return hipGetLastError();
}

template <int MT, int NTB, int W>
hipError_t launch_sp24_ksplit_w(const uint16_t* x, const uint8_t* blob, const BlobLayout& L,
                                int M, int m0, int N, int K, void* y, int y_dtype, hipStream_t s) {
  const int gpw = (K / 128 + KW - 1) / KW;
  const int rows = M - m0 < 16 * MT ? M - m0 : 16 * MT;
  // one m-tile: rows staged per chunk (chunks of up to six groups); two
  // m-tiles: only when the wave's groups fit one chunk of up to four
  if constexpr (MT == 1 ? W <= 6 : W <= 4) {
    if (MT == 2 && gpw > W) return launch_sp24_ksplit_xq<MT, NTB, W, -1>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    switch (stage_quads(rows, MT)) {
      case 0:   // one token: a lane per group for up to four groups, else one row quad
        if constexpr (MT == 1 && W <= 4)
          return launch_sp24_ksplit_xq<MT, NTB, W, 0>(x, blob, L, M, m0, N, K, y, y_dtype, s);
        return launch_sp24_ksplit_xq<MT, NTB, W, 1>(x, blob, L, M, m0, N, K, y, y_dtype, s);
      case 1: return launch_sp24_ksplit_xq<MT, NTB, W, 1>(x, blob, L, M, m0, N, K, y, y_dtype, s);
      case 2: return launch_sp24_ksplit_xq<MT, NTB, W, 2>(x, blob, L, M, m0, N, K, y, y_dtype, s);
      default: return launch_sp24_ksplit_xq<MT, NTB, W, 4>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    }
  }
  return launch_sp24_ksplit_xq<MT, NTB, W, -1>(x, blob, L, M, m0, N, K, y, y_dtype, s);
}

template <int MT, int NTB>
hipError_t launch_sp24_ksplit(const uint16_t* x, const uint8_t* blob, const BlobLayout& L, int M,
                              int m0, int N, int K, void* y, int y_dtype, hipStream_t s) {
  constexpr int kCap = sp_cap(MT, NTB);
  switch (pick_chunk((K / 128 + KW - 1) / KW, kCap)) {
    case 2: return launch_sp24_ksplit_w<MT, NTB, cmin(2, kCap)>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    case 4: return launch_sp24_ksplit_w<MT, NTB, cmin(4, kCap)>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    case 6: return launch_sp24_ksplit_w<MT, NTB, cmin(6, kCap)>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    default: return launch_sp24_ksplit_w<MT, NTB, cmin(8, kCap)>(x, blob, L, M, m0, N, K, y, y_dtype, s);
  }
}

// grid: S k slices x tile walkers (at most T per slice); part: the fp32
// partial sums when S > 1
template <int GW, int MT, int XQ>
hipError_t launch_sp24_persist_xq(const uint16_t* x, const uint8_t* blob, const BlobLayout& L,
                                  int M, int N, int K, void* y, int y_dtype, int grid, int S,
                                  float* part, hipStream_t s) {
  if (y_dtype == 1)
    sp24_persist_kernel<GW, MT, XQ, true><<<grid, KW * 64, 0, s>>>(
        x, blob, L.codes_off, L.aux_off, M, N, K, y, S, part);
  else
    sp24_persist_kernel<GW, MT, XQ, false><<<grid, KW * 64, 0, s>>>(
        x, blob, L.codes_off, L.aux_off, M, N, K, y, S, part);
  return hipGetLastError();
}

template <int GW, int MT>
hipError_t launch_sp24_persist(const uint16_t* x, const uint8_t* blob, const BlobLayout& L, int M,
                               int N, int K, void* y, int y_dtype, int grid, int S, float* part,
                               hipStream_t s) {
  if constexpr (MT == 2)
    return launch_sp24_persist_xq<GW, MT, 4>(x, blob, L, M, N, K, y, y_dtype, grid, S, part, s);
  switch (stage_quads(M, MT)) {
    case 0:
      if constexpr (MT == 1)
        return launch_sp24_persist_xq<GW, MT, 0>(x, blob, L, M, N, K, y, y_dtype, grid, S, part, s);
      break;
    case 1: return launch_sp24_persist_xq<GW, MT, 1>(x, blob, L, M, N, K, y, y_dtype, grid, S, part, s);
    case 2: return launch_sp24_persist_xq<GW, MT, 2>(x, blob, L, M, N, K, y, y_dtype, grid, S, part, s);
    default: break;
  }
  return launch_sp24_persist_xq<GW, MT, 4>(x, blob, L, M, N, K, y, y_dtype, grid, S, part, s);
}

}  // namespace

// Plan of the k-sliced persistent kernel for the workspace entry point: GW
// groups per wave (2 or 4), S slices of KW GW groups, P tile walkers per
// slice, one block per CU (S P = CUs), as the dense plan.  Long k and
// 8 < m <= 32 only, where every block loading the whole activation dominates.
DecodeSplit sp24_split_plan(int64_t m, int64_t n, int64_t k) {
  DecodeSplit best{0, 0, 0, 0};
  const int cus = device_cu_count();
  if (m < 1 || m > 32 || cus <= 0 || n % 16 != 0 || k % 128 != 0) return best;
  const int64_t T = n / 16, G = k / 128;
  if (G <= KW * 4 || m <= 8) return best;
  int64_t best_cost = INT64_MAX;
  for (int gw = 2; gw <= 4; gw += 2) {
    const int64_t S = (G + KW * gw - 1) / (KW * gw);
    if (S < 2) continue;
    const int64_t P = std::min<int64_t>(T, cus / S);
    if (P < 1) continue;
    // (row tile, group) units per CU, plus a round trip per pair of tiles
    const int64_t tiles = (T + P - 1) / P;
    const int64_t cost = tiles * KW * gw + 32 * ((tiles + 1) / 2);
    if (cost < best_cost) {
      best_cost = cost;
      best = DecodeSplit{gw, m > 16 ? 2 : 1, int(S), int(P)};
    }
  }
  return best;
}

hipError_t launch_gemm_w4a16_sp24(const void* x, const void* w_packed, int64_t m, int64_t n,
                                  int64_t k, void* y, int y_dtype, void* ws, size_t ws_bytes,
                                  hipStream_t s) {
  const BlobLayout L = blob_layout(3, n, k);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const int M = int(m), N = int(n), K = int(k), G = int(k / 128), T = int(n / 16);
  const int cus = device_cu_count();
  // k split over blocks with the caller's workspace: the slices' fp32
  // partial sums, added by a second launch
  const DecodeSplit sp = sp24_split_plan(m, n, k);
  if (sp.S >= 2 && ws != nullptr && ws_bytes >= decode_split_bytes(sp, m, n)) {
    float* part = static_cast<float*>(ws);
    const int grid = sp.S * sp.P;
    hipError_t e;
    if (sp.mt == 1)
      e = sp.gw == 2 ? launch_sp24_persist<2, 1>(xp, blob, L, M, N, K, y, y_dtype, grid, sp.S, part, s)
                     : launch_sp24_persist<4, 1>(xp, blob, L, M, N, K, y, y_dtype, grid, sp.S, part, s);
    else
      e = sp.gw == 2 ? launch_sp24_persist<2, 2>(xp, blob, L, M, N, K, y, y_dtype, grid, sp.S, part, s)
                     : launch_sp24_persist<4, 2>(xp, blob, L, M, N, K, y, y_dtype, grid, sp.S, part, s);
    if (e != hipSuccess) return e;
    return launch_decode_reduce(part, sp.S, m, n, y, y_dtype, blob, 3, k, s);
  }
  if (m <= 32 && G <= KW * 4 && cus > 0 && T >= 2 * cus) {
    // every block owns at least two tiles, and the grid never exceeds T
    auto grid_of = [&](int per_cu) { return T >= 2 * per_cu * cus ? per_cu * cus : cus; };
    if (m <= 16)
      return G <= KW * 2
                 ? launch_sp24_persist<2, 1>(xp, blob, L, M, N, K, y, y_dtype,
                                             grid_of(sp_blocks_per_cu(2, 1)), 1, nullptr, s)
                 : launch_sp24_persist<4, 1>(xp, blob, L, M, N, K, y, y_dtype,
                                             grid_of(sp_blocks_per_cu(4, 1)), 1, nullptr, s);
    return G <= KW * 2
               ? launch_sp24_persist<2, 2>(xp, blob, L, M, N, K, y, y_dtype,
                                           grid_of(sp_blocks_per_cu(2, 2)), 1, nullptr, s)
               : launch_sp24_persist<4, 2>(xp, blob, L, M, N, K, y, y_dtype,
                                           grid_of(sp_blocks_per_cu(4, 2)), 1, nullptr, s);
  }
  const bool wide = T >= 384;   // two row tiles per block still give >= 192 blocks
  for (int64_t m0 = 0; m0 < m; m0 += 32) {
    const int rows = int(m - m0 < 32 ? m - m0 : 32), b = int(m0);
    hipError_t e;
    if (rows <= 16)
      e = wide ? launch_sp24_ksplit<1, 2>(xp, blob, L, M, b, N, K, y, y_dtype, s)
               : launch_sp24_ksplit<1, 1>(xp, blob, L, M, b, N, K, y, y_dtype, s);
    else
      e = wide ? launch_sp24_ksplit<2, 2>(xp, blob, L, M, b, N, K, y, y_dtype, s)
               : launch_sp24_ksplit<2, 1>(xp, blob, L, M, b, N, K, y, y_dtype, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qlin
