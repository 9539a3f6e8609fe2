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
#include "decode_ops.hpp"

#include <algorithm>
#include <climits>
#include <type_traits>

namespace qlin {
namespace {

// LUT2: 16 2-bit indices (layout of the repacked blob) -> two bf16x8 operands
// (sub-steps 2d and 2d+1) looked up in the row's codebook with v_perm_b32.
__device__ __forceinline__ void lut2_operands(uint32_t w, uint32_t lo_t, uint32_t hi_t,
                                              bf16x8_t& a0, bf16x8_t& a1) {
  u32x4 op[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = (w >> (2 * j)) & 0x03030303u;
    const uint32_t lo = __builtin_amdgcn_perm(0u, lo_t, sel);
    const uint32_t hi = __builtin_amdgcn_perm(0u, hi_t, sel);
    op[j >> 1][2 * (j & 1)] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    op[j >> 1][2 * (j & 1) + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  a0 = as_bf16x8(op[0]);
  a1 = as_bf16x8(op[1]);
}

template <int MT, int NTB, int KWT, bool kBF16Out>
__device__ __forceinline__ void reduce_store(floatx4 (&tot)[NTB][MT], int nt0, int m0, int M,
                                             int N, void* __restrict__ y) {
  __shared__ floatx4 red[KWT][NTB][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][nt][mt][lane] = tot[nt][mt];
  __syncthreads();
  for (int t = threadIdx.x; t < NTB * MT * 64; t += KWT * 64) {
    const int nt = t / (MT * 64), mt = (t / 64) % MT, ln = t % 64;
    floatx4 s = red[0][nt][mt][ln];
#pragma unroll
    for (int w = 1; w < KWT; ++w) s += red[w][nt][mt][ln];
    const int n = (nt0 + nt) * 16 + 4 * (ln >> 4);
    const int m = m0 + mt * 16 + (ln & 15);
    if (m < M && n < N) {
      if (kBF16Out) {
        uint2 o;
        o.x = pack_bf16x2(s[0], s[1]);
        o.y = pack_bf16x2(s[2], s[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + int64_t(m) * N + n) = o;
      } else {
        *reinterpret_cast<floatx4*>(static_cast<float*>(y) + int64_t(m) * N + n) = s;
      }
    }
  }
}

// Activation fragments of one 128-k group for MT m-tiles: lane l holds row
// m0 + 16 mt + l % 16 (clamped to the last valid row: columns m >= M are
// computed but never stored, so they need no zeroing) and k = 128 g + 32 s +
// 8 (l / 16) + t.
template <int MT>
struct XFrag {
  bf16x8_t f[4][MT];
};
template <int MT>
__device__ __forceinline__ void load_xfrag(XFrag<MT>& X, const uint16_t* const (&xr)[MT], int g) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 t = *reinterpret_cast<const uint4*>(xr[mt] + g * 128 + 32 * s);
      X.f[s][mt] = as_bf16x8(u32x4{t.x, t.y, t.z, t.w});
    }
}

// Each wave owns groups g0 .. g0 + gpw - 1 of NTB row tiles and walks them in
// chunks of WMAX groups.  A chunk's weight loads (HBM) are issued at once;
// activation fragments (small, L2-resident) follow one group ahead.  The
// arithmetic of a chunk runs in two phases so that no VALU instruction waits
// on an MFMA it has just issued: first every group's MFMA chains (independent,
// so they stream through the matrix core back to back), then every group's
// fp32 scale multiply-add.  Slots past the wave's range or past k are clamped
// to a valid address and contribute zero (their scales are replaced by 0),
// so the loop has no branches and the compiler can count outstanding loads.
// XQ >= 0: the activation rows of the wave's groups are loaded first and
// staged with rows_stage (NQ = XQ) once the chunk's weight loads are in
// flight -- all of them before the loop when they fit one chunk, else
// (kRowsPerChunk) each chunk's at the top of its iteration.
template <int MT, int NTB, int WMAX, int KWT, int XQ, bool kBF16Out, bool kRowsPerChunk = false>
__global__ __launch_bounds__(KWT * 64) void w4a16_kernel(const uint16_t* __restrict__ x,
                                                        const uint8_t* __restrict__ blob,
                                                        int64_t codes_off, int64_t sc_off, int M,
                                                        int m0, int N, int K,
                                                        void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = K / 128;
  const int gpw = (G + KWT - 1) / KWT;
  const int g0 = wave * gpw;
  const int nt0 = blockIdx.x * NTB;
  const int NT16 = N / 16;
  // -136 in every bf16 lane: an MFMA chain against it yields -136 * sum x, the
  // start value that turns sum x (128 + u) into sum x q (u = q + 8)
  const uint32_t m136 = vconst(0xC308C308u);
  const bf16x8_t neg136 = as_bf16x8(u32x4{m136, m136, m136, m136});
  const uint32_t nib_mask = vconst(0x000F000Fu), bf16_128 = vconst(0x43004300u);

  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xr[mt] = x + int64_t(min(m0 + mt * 16 + (lane & 15), M - 1)) * K + 8 * (lane >> 4);
  const uint4* wp[NTB];
  const uint2* sp[NTB];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int64_t tile = min(nt0 + nt, NT16 - 1);
    wp[nt] = reinterpret_cast<const uint4*>(blob + codes_off) + tile * G * 64 + lane;
    sp[nt] = reinterpret_cast<const uint2*>(blob + sc_off + (tile * G * 16 + 4 * (lane >> 4)) * 2);
  }

  floatx4 tot[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  __shared__ __attribute__((aligned(16))) uint8_t xst[XQ >= 0 ? KWT : 1][4096];
  bf16x8_t xpre[XQ >= 0 ? WMAX : 1][4][MT];
  if constexpr (XQ >= 0 && !kRowsPerChunk) rows_load<WMAX, MT, XQ>(x, M, m0, K, g0, gpw, G, lane, xpre);

  uint32_t hdr = 0;   // header words (lane l: word l % 8)
  for (int c0 = 0; c0 < gpw; c0 += WMAX) {
    if constexpr (XQ >= 0 && kRowsPerChunk)
      rows_load<WMAX, MT, XQ>(x, M, m0, K, g0 + c0, gpw - c0, G, lane, xpre);
    uint4 wv[WMAX][NTB];
    uint2 sv[WMAX][NTB];
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int gc = min(g0 + min(c0 + i, gpw - 1), G - 1);
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        wv[i][nt] = load_nt16(wp[nt] + gc * 64);
        sv[i][nt] = sp[nt][gc * 4];
      }
    }
    if (c0 == 0) hdr = header_word(blob);   // behind the first weights; tested before the store
    if constexpr (XQ >= 0) {
      __builtin_amdgcn_sched_barrier(0);   // the weight loads go out before the staging
      rows_stage<WMAX, MT, XQ>(xst[wave], lane, xpre);
    }
    // phase 1: MFMA chains of every group of the chunk
    floatx4 acc[WMAX][NTB][MT];
    XFrag<MT> xf;
    if constexpr (XQ < 0) load_xfrag<MT>(xf, xr, min(g0 + c0, G - 1));
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      XFrag<MT> xn;
      if constexpr (XQ >= 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xf.f[s][mt] = xpre[i][s][mt];
      } else if (i + 1 < WMAX) {
        load_xfrag<MT>(xn, xr, min(g0 + c0 + i + 1, G - 1));   // compile-time
      }
      floatx4 xs[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        xs[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg136, xf.f[s][mt], xs[mt], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[i][nt][mt] = xs[mt];
        const uint32_t wd[4] = {wv[i][nt].x, wv[i][nt].y, wv[i][nt].z, wv[i][nt].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t a = int4_operand(wd[s], nib_mask, bf16_128);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[i][nt][mt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xf.f[s][mt], acc[i][nt][mt], 0, 0, 0);
        }
      }
      if constexpr (XQ < 0) {
        if (i + 1 < WMAX) xf = xn;
      }
    }
    // phase 2: tot += group scale * (sum x q), in fp32, per group
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const bool live = c0 + i < gpw && g0 + c0 + i < G;
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        const uint32_t s01 = live ? sv[i][nt].x : 0u, s23 = live ? sv[i][nt].y : 0u;
        const float sc[4] = {__uint_as_float(s01 << 16), __uint_as_float(s01 & 0xFFFF0000u),
                             __uint_as_float(s23 << 16), __uint_as_float(s23 & 0xFFFF0000u)};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            tot[nt][mt][r] = fmaf(sc[r], acc[i][nt][mt][r], tot[nt][mt][r]);
      }
    }
  }
  if (!header_word_ok(hdr, 1, N, K)) return;   // uniform: no wave reaches the barrier in reduce_store
  reduce_store<MT, NTB, KWT, kBF16Out>(tot, nt0, m0, M, N, y);
}

template <int MT, int NTB, int WMAX, int KWT, int XQ, bool kBF16Out>
__global__ __launch_bounds__(KWT * 64) void lut2_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ blob,
                                                       int64_t codes_off, int64_t book_off, int M,
                                                       int m0, int N, int K,
                                                       void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = K / 128;
  const int gpw = (G + KWT - 1) / KWT;
  const int g0 = wave * gpw;
  const int nt0 = blockIdx.x * NTB;
  const int NT16 = N / 16;

  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xr[mt] = x + int64_t(min(m0 + mt * 16 + (lane & 15), M - 1)) * K + 8 * (lane >> 4);
  const uint2* wp[NTB];
  uint32_t lo_t[NTB], hi_t[NTB];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int64_t tile = min(nt0 + nt, NT16 - 1);
    wp[nt] = reinterpret_cast<const uint2*>(blob + codes_off) + tile * G * 64 + lane;
    const uint2 b = reinterpret_cast<const uint2*>(blob + book_off)[tile * 16 + (lane & 15)];
    lo_t[nt] = b.x;
    hi_t[nt] = b.y;
  }

  // two accumulator sets, even and odd groups, so consecutive MFMAs of a tile
  // do not wait on each other's results
  floatx4 tot2[2][NTB][MT];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) tot2[e][nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  __shared__ __attribute__((aligned(16))) uint8_t xst[XQ >= 0 ? KWT : 1][4096];
  bf16x8_t xpre[XQ >= 0 ? WMAX : 1][4][MT];
  if constexpr (XQ >= 0) rows_load<WMAX, MT, XQ>(x, M, m0, K, g0, gpw, G, lane, xpre);

  uint32_t hdr = 0;   // header words (lane l: word l % 8)
  for (int c0 = 0; c0 < gpw; c0 += WMAX) {
    uint2 wv[WMAX][NTB];
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int gc = min(g0 + min(c0 + i, gpw - 1), G - 1);
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) wv[i][nt] = load_nt8(wp[nt] + gc * 64);
    }
    if (c0 == 0) hdr = header_word(blob);   // behind the first weights; tested before the store
    if constexpr (XQ >= 0) {
      __builtin_amdgcn_sched_barrier(0);   // the weight loads go out before the staging
      rows_stage<WMAX, MT, XQ>(xst[wave], lane, xpre);
    }
    XFrag<MT> xf;
    if constexpr (XQ < 0) load_xfrag<MT>(xf, xr, min(g0 + c0, G - 1));
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int g = g0 + c0 + i;
      XFrag<MT> xn;
      if constexpr (XQ >= 0) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xf.f[s][mt] = xpre[i][s][mt];
      } else if (i + 1 < WMAX) {
        load_xfrag<MT>(xn, xr, min(g + 1, G - 1));   // compile-time condition
      }
      const uint32_t keep = (c0 + i < gpw && g < G) ? 0xFFFFFFFFu : 0u;  // else zero codebook
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        const uint32_t lo = lo_t[nt] & keep, hi = hi_t[nt] & keep;
        bf16x8_t a[4];
        lut2_operands(wv[i][nt].x, lo, hi, a[0], a[1]);
        lut2_operands(wv[i][nt].y, lo, hi, a[2], a[3]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            tot2[i & 1][nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a[s], xf.f[s][mt], tot2[i & 1][nt][mt], 0, 0, 0);
      }
      if constexpr (XQ < 0) {
        if (i + 1 < WMAX) xf = xn;
      }
    }
  }
  floatx4 tot[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[nt][mt] = tot2[0][nt][mt] + tot2[1][nt][mt];
  if (!header_word_ok(hdr, 2, N, K)) return;   // uniform: no wave reaches the barrier in reduce_store
  reduce_store<MT, NTB, KWT, kBF16Out>(tot, nt0, m0, M, N, y);
}

// Pipelined k-split variant for one m-tile (M <= 16) and long K (at least
// two chunks of W groups per wave): a block of 8 waves owns one row tile and
// the waves split k, as above, but each wave walks its groups in chunks of W
// with the next chunk's loads in flight while it computes the current one
// (two register sets).  A chunk's activation rows travel in the same batch
// as its weights: loads complete in issue order for the wait counter, so
// rows fetched later would make the arithmetic wait for the next chunk's
// weights as well.
//
// Activations are loaded as whole rows and turned into MFMA fragments in LDS.
// A fragment load (lane l: token l % 16, k 32 s + 8 (l / 16)) sends adjacent
// lanes to different rows, so the L1 cannot merge them: measured with rows
// 24-30 KiB apart (K = 12288, 15360), fragment loads cost 4x the L1 tag
// lookups and 2.5-2.8x the address-unit time of the same bytes loaded as
// rows, and twice the time.  Here lane l loads token 4 q + l / 16 at k
// 8 (l % 16) of a group (row quad q: 256 contiguous bytes per token), only
// the NQ quads that hold tokens < M, writes them to a wave-private LDS tile
// [4 NQ tokens][128 k] (rows padded to 272 bytes) and reads the fragments
// back, lanes of tokens >= 4 NQ reading the last staged row (its outputs are
// not stored).  With one token (NQ = 0) a single load brings the chunk's four
// groups (lane l: group l / 16).  The INT4 group scales of a chunk's four
// groups (4 x 32 contiguous bytes) also come with one load (lane l: group
// (l / 2) % 4, half l % 2) and reach their lanes through LDS.  LDS
// operations of one wave run in order, so none of this needs a barrier.
constexpr int kXRow = 272;               // LDS bytes per staged token row

template <int NQ>
constexpr int pipe_xrows() { return NQ == 0 ? 1 : 4 * NQ; }
// LDS bytes of one wave: activation tiles (two groups' tiles, or with one
// token the four groups of a chunk) and the chunk's scales
template <int NQ>
constexpr int pipe_xbytes() { return NQ == 0 ? 4 * kXRow : 2 * 4 * NQ * kXRow; }
constexpr int kSBytes = 128;

template <int W, bool kLut, int NQ>
struct PipeBatch;
template <int W, int NQ>
struct PipeBatch<W, false, NQ> {
  uint4 w[W];
  uint4 s;
  uint4 x[NQ == 0 ? 1 : W][NQ == 0 ? 1 : NQ];
};
template <int W, int NQ>
struct PipeBatch<W, true, NQ> {
  uint2 w[W];
  uint4 x[NQ == 0 ? 1 : W][NQ == 0 ? 1 : NQ];
};

template <int W, bool kLut, int NQ, bool kBF16Out>
__global__ __launch_bounds__(KW * 64) void decode_pipe_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ blob, int64_t codes_off,
    int64_t aux_off, int M, int N, int K, void* __restrict__ y) {
  static_assert(W == 4, "a chunk is four groups: one scale load, one single-token row load");
  __shared__ __attribute__((aligned(16))) uint8_t xt[KW][pipe_xbytes<NQ>()];
  __shared__ __attribute__((aligned(16))) uint8_t st[KW][kSBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = K / 128;
  const int gpw = (G + KW - 1) / KW;
  const int g0 = wave * gpw;
  const int64_t tile = blockIdx.x;
  const uint32_t m136 = vconst(0xC308C308u);
  const bf16x8_t neg136 = as_bf16x8(u32x4{m136, m136, m136, m136});
  const uint32_t nib_mask = vconst(0x000F000Fu), bf16_128 = vconst(0x43004300u);
  // byte offset of this lane's token of each row quad (clamped to a valid
  // row) and k position: 32 bits, added to the uniform group address
  constexpr int NQR = NQ == 0 ? 1 : NQ;
  uint32_t xq[NQR];
#pragma unroll
  for (int q = 0; q < NQR; ++q)
    xq[q] = 2u * (uint32_t(NQ == 0 ? 0 : min(4 * q + (lane >> 4), M - 1)) * uint32_t(K) +
                  8u * uint32_t(lane & 15));
  auto xrow = [&](int q, int g) {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(x) + int64_t(g) * 256 +
                                           xq[q]);
  };
  uint32_t lo_t = 0, hi_t = 0;
  if constexpr (kLut) {
    const uint2 b = reinterpret_cast<const uint2*>(blob + aux_off)[tile * 16 + (lane & 15)];
    lo_t = b.x;
    hi_t = b.y;
  }
  auto gclamp = [&](int c0, int i) { return min(g0 + min(c0 + i, gpw - 1), G - 1); };

  auto load = [&](PipeBatch<W, kLut, NQ>& B, int c0) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int64_t gi = tile * G + gclamp(c0, i);
      if constexpr (kLut)
        B.w[i] = load_nt8(reinterpret_cast<const uint2*>(blob + codes_off) + gi * 64 + lane);
      else
        B.w[i] = load_nt16(reinterpret_cast<const uint4*>(blob + codes_off) + gi * 64 + lane);
    }
    if constexpr (!kLut) {
      const int64_t gs = tile * G + gclamp(c0, (lane >> 1) & 3);
      B.s = *reinterpret_cast<const uint4*>(blob + aux_off + gs * 32 + 16 * (lane & 1));
    }
    if constexpr (NQ == 0) {
      B.x[0][0] = xrow(0, gclamp(c0, lane >> 4));
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q) B.x[i][q] = xrow(q, gclamp(c0, i));
    }
  };

  uint8_t* const xw = xt[wave];
  // a chunk's shared stores (single-token rows, scales) before its groups
  auto stage = [&](const PipeBatch<W, kLut, NQ>& B) {
    if constexpr (NQ == 0)
      *reinterpret_cast<uint4*>(xw + (lane >> 4) * kXRow + 16 * (lane & 15)) = B.x[0][0];
    if constexpr (!kLut) {
      if (lane < 8) *reinterpret_cast<uint4*>(st[wave] + 16 * lane) = B.s;
    }
  };
  // fragments of group i of the chunk
  auto fragments = [&](const PipeBatch<W, kLut, NQ>& B, int i, bf16x8_t (&f)[4]) {
    const uint8_t* t;
    int row;
    if constexpr (NQ == 0) {
      t = xw + i * kXRow;
      row = 0;
    } else {
      uint8_t* tw = xw + (i & 1) * (4 * NQ * kXRow);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        *reinterpret_cast<uint4*>(tw + (4 * q + (lane >> 4)) * kXRow + 16 * (lane & 15)) =
            B.x[i][q];
      t = tw;
      row = min(lane & 15, 4 * NQ - 1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 v = *reinterpret_cast<const uint4*>(t + row * kXRow + 64 * s + 16 * (lane >> 4));
      f[s] = as_bf16x8(u32x4{v.x, v.y, v.z, v.w});
    }
  };

  floatx4 tot[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  auto compute = [&](const PipeBatch<W, kLut, NQ>& B, int c0) {
    stage(B);
    if constexpr (kLut) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        const int g = g0 + c0 + i;
        const uint32_t keep = (c0 + i < gpw && g < G) ? 0xFFFFFFFFu : 0u;   // else zero codebook
        bf16x8_t f[4];
        fragments(B, i, f);
        bf16x8_t a[4];
        lut2_operands(B.w[i].x, lo_t & keep, hi_t & keep, a[0], a[1]);
        lut2_operands(B.w[i].y, lo_t & keep, hi_t & keep, a[2], a[3]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          tot[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], f[s], tot[i & 1], 0, 0, 0);
      }
    } else {
      floatx4 acc[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        bf16x8_t f[4];
        fragments(B, i, f);
        acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg136, f[s], acc[i], 0, 0, 0);
        const uint32_t wd[4] = {B.w[i].x, B.w[i].y, B.w[i].z, B.w[i].w};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(int4_operand(wd[s], nib_mask, bf16_128),
                                                           f[s], acc[i], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < W; ++i) {
        // this lane's rows 4 (l / 16) .. + 3 of group i: 8 bytes of the staged scales
        const uint2 sv = *reinterpret_cast<const uint2*>(st[wave] + 32 * i + 8 * (lane >> 4));
        const bool live = c0 + i < gpw && g0 + c0 + i < G;
        const uint32_t s01 = live ? sv.x : 0u, s23 = live ? sv.y : 0u;
        const float sc[4] = {__uint_as_float(s01 << 16), __uint_as_float(s01 & 0xFFFF0000u),
                             __uint_as_float(s23 << 16), __uint_as_float(s23 & 0xFFFF0000u)};
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[0][r] = fmaf(sc[r], acc[i][r], tot[0][r]);
      }
    }
  };

  // (the scheduling barriers keep each batch's loads ahead of the arithmetic
  // on the previous one; the compiler would otherwise sink them below it)
  PipeBatch<W, kLut, NQ> A, B;
  load(A, 0);
  const uint32_t hdr = header_word(blob);   // behind the first weights; tested before the store
  int c0 = 0;
  for (; c0 + W < gpw; c0 += 2 * W) {   // chunks c0 (in A) and c0 + W (in B)
    load(B, c0 + W);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, c0);
    load(A, c0 + 2 * W);                 // clamped when past the range
    __builtin_amdgcn_sched_barrier(0);
    compute(B, c0 + W);
  }
  if (c0 < gpw) compute(A, c0);          // wave-uniform: an odd last chunk
  floatx4 t1[1][1] = {{tot[0] + tot[1]}};
  if (!header_word_ok(hdr, kLut ? 2 : 1, N, K)) return;   // uniform: no wave reaches the barrier in reduce_store
  reduce_store<1, 1, KW, kBF16Out>(t1, int(tile), 0, M, N, y);
}

// Persistent variant for M <= 32 and K <= 128 * KW * GW.  Wave w owns groups
// [GW w, GW w + GW) of every row tile, so its activation fragments -- and, for
// INT4, the -136 * sum x seeds -- are the same for all tiles: they are loaded
// and computed once per wave.  One or two blocks per CU walk the row tiles
// t = blockIdx.x, + gridDim.x, ... with the next tile's weights (two register
// sets) in flight while the current one is dequantized, multiplied and
// reduced; no activation load sits between them in the load queue, so the
// arithmetic waits only for its own tile.  Used when every block gets at
// least two tiles.
//
// Weights are read through a buffer resource made per tile, so tile and group
// offsets are scalar and no vector instruction computes an address.  The
// first tile's loads are issued before the seed MFMAs (which wait only for
// the activation loads ahead of them).  The eight (sixteen) partial sums of a
// tile are added by four (eight) waves at once, one accumulator component
// each.  INT4 with two m-tiles keeps the second m-tile's fragments in LDS
// (lane-private, so they need no barrier): in registers they would not fit
// next to the two weight sets at two waves per SIMD.
template <int GW, bool kLut>
struct PersistTile;
template <int GW>
struct PersistTile<GW, false> {
  uint4 w[GW];
  uint2 s[GW];
};
template <int GW>
struct PersistTile<GW, true> {
  uint2 w[GW];
  uint2 book;
};

// waves per block: 8, or 16 for LUT2 with two m-tiles (two groups per wave)
constexpr int persist_waves(int mt, bool lut) { return mt == 2 && lut ? 2 * KW : KW; }
// Blocks of this kernel that fit on one CU: two when the registers allow four
// waves per SIMD (one m-tile with LUT2, or INT4 with at most three groups per
// wave: 116 VGPRs), else one.
constexpr int persist_blocks_per_cu(int gw, int mt, bool lut) {
  return mt == 1 && (lut || gw <= 3) ? 2 : 1;
}
constexpr bool persist_x_in_lds(int mt, bool lut) { return mt == 2 && !lut; }
// dynamic LDS: two reduction slots [2][waves][MT][4][64] floats, then (INT4,
// two m-tiles) the second m-tile's fragments [waves][GW][4][64] x 16 bytes
// floats per (wave, m-tile, component) row of a reduction slot: with one
// m-tile 65, which keeps the row-wise final sums' reads free of bank
// conflicts; with two, 64 (INT4 then fills the 160 KiB of LDS)
constexpr int persist_red_stride(int mt, bool lut) { return mt == 1 ? 65 : 64; }
constexpr size_t persist_red_bytes(int mt, bool lut) {
  return size_t(2) * persist_waves(mt, lut) * mt * 4 * persist_red_stride(mt, lut) * 4;
}
// one m-tile: the activation rows are staged through a wave-private LDS tile
// of 16 rows x 256 bytes at the start, in the space of the reduction slots
constexpr size_t persist_stage_bytes(int mt, bool lut) {
  return mt == 1 ? size_t(persist_waves(mt, lut)) * 4096 : 0;
}
constexpr size_t persist_lds_bytes(int gw, int mt, bool lut) {
  return (persist_red_bytes(mt, lut) > persist_stage_bytes(mt, lut)
              ? persist_red_bytes(mt, lut) : persist_stage_bytes(mt, lut)) +
         (persist_x_in_lds(mt, lut) ? size_t(persist_waves(mt, lut)) * gw * 4 * 64 * 16 : 0);
}

template <int GW, int MT, bool kLut, bool kBF16Out>
__global__ __launch_bounds__(persist_waves(MT, kLut) * 64,
                             persist_waves(MT, kLut) / 4 * persist_blocks_per_cu(GW, MT, kLut))
void decode_persist_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ blob,
                           int64_t codes_off, int64_t aux_off, int M, int N, int K,
                           void* __restrict__ y, int S, float* __restrict__ part) {
  const uint32_t hdr = header_word(blob);   // tested before the first store
  constexpr int NW = persist_waves(MT, kLut);
  constexpr bool kXL = persist_x_in_lds(MT, kLut);
  constexpr int MR = kXL ? 1 : MT;         // m-tiles whose fragments stay in registers
  constexpr int CB = kLut ? 512 : 1024;    // code bytes per (row tile, group)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* const red = reinterpret_cast<float*>(smem);
  bf16x8_t* const xl = reinterpret_cast<bf16x8_t*>(smem + persist_red_bytes(MT, kLut));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int G = K / 128;
  // block = (tile walker, k slice): slice sl owns groups [NW GW sl, NW GW (sl + 1))
  const int sl = blockIdx.x % S;
  const int g0 = (sl * NW + wave) * GW;
  const int T = N / 16;
  const int stride = gridDim.x / S;   // tile walkers
  const uint32_t m136 = vconst(0xC308C308u);
  const bf16x8_t neg136 = as_bf16x8(u32x4{m136, m136, m136, m136});
  const uint32_t nib_mask = vconst(0x000F000Fu), bf16_128 = vconst(0x43004300u);

  auto load = [&](PersistTile<GW, kLut>& A, int t) {
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(blob + codes_off + int64_t(t) * G * CB), 0, G * CB, kRsrcWord3);
    if constexpr (kLut) {
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, lane * 8, min(g0 + i, G - 1) * CB,
                                                             kPolicyNT);
        A.w[i] = make_uint2(v[0], v[1]);
      }
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(blob + aux_off + int64_t(t) * 128), 0, 128, kRsrcWord3);
      const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(rb, (lane & 15) * 8, 0, 0);
      A.book = make_uint2(b[0], b[1]);
    } else {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(blob + aux_off + int64_t(t) * G * 32), 0, G * 32, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int gc = min(g0 + i, G - 1);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16, gc * CB, kPolicyNT);
        A.w[i] = make_uint4(v[0], v[1], v[2], v[3]);
        const u32x2 s = __builtin_amdgcn_raw_buffer_load_b64(rs, (lane >> 4) * 8, gc * 32, 0);
        A.s[i] = make_uint2(s[0], s[1]);
      }
    }
  };

  // activation fragments (issued first), then the first tile's weights
  bf16x8_t xf[GW][4][MR];
  bf16x8_t xt[kXL ? GW : 1][4];
  // One m-tile: the rows are loaded whole (lane l: token 4 q + l / 16 at k
  // 8 (l % 16) of a group; with one token, lane l: group l / 16) and turned
  // into fragments through a wave-private LDS tile [16 rows][256 B] whose
  // 16-byte slots are XOR-swizzled by row (conflict-free writes and fragment
  // reads).  A fragment load sends adjacent lanes to different rows, which
  // the L1 cannot merge (4x the tag lookups of row loads).  Two m-tiles load
  // fragments directly (their registers would not hold a row batch).
  if constexpr (MT != 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* xr = x + int64_t(min(mt * 16 + (lane & 15), M - 1)) * K + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int gc = min(g0 + i, G - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 v = *reinterpret_cast<const uint4*>(xr + gc * 128 + 32 * s);
          if (kXL && mt == 1)
            xt[kXL ? i : 0][s] = as_bf16x8(u32x4{v.x, v.y, v.z, v.w});
          else
            xf[i][s][mt < MR ? mt : 0] = as_bf16x8(u32x4{v.x, v.y, v.z, v.w});
        }
      }
    }
  }
  // one m-tile with NQ row quads (NQ = 0: one token): the rows (loaded before
  // the first tile's weights) go through the wave's LDS staging tile once
  // those weights are in flight
  uint8_t* const xstage = smem + size_t(wave) * 4096;
  auto stage_rows = [&](auto nq_c, PersistTile<GW, kLut>& A0, int t0) __attribute__((always_inline)) {
    constexpr int NQ = decltype(nq_c)::value;
    rows_load<GW, 1, NQ>(x, M, 0, K, g0, GW, G, lane, xf);
    load(A0, t0);
    __builtin_amdgcn_sched_barrier(0);   // keep the tile loads ahead of the staging
    rows_stage<GW, 1, NQ>(xstage, lane, xf);
  };
  PersistTile<GW, kLut> A, B;
  int t = blockIdx.x / S;
  if constexpr (MT == 1) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    if (M == 1) stage_rows(I0{}, A, t);
    else if (M <= 4) stage_rows(I1{}, A, t);
    else if (M <= 8) stage_rows(I2{}, A, t);
    else if (M <= 12) stage_rows(I3{}, A, t);
    else stage_rows(I4{}, A, t);
    __syncthreads();   // the staging tiles share their space with the reduction slots
  } else {
    load(A, t);
    __builtin_amdgcn_sched_barrier(0);   // keep the tile loads ahead of the seed arithmetic
  }

  // slots past the last group (g0 + i >= G: the last k slice, or K not a
  // multiple of the groups a block covers) loaded a clamped copy of group
  // G - 1; their activation fragments are zeroed here, once, so that their
  // products vanish in every tile with no per-tile masking of the weights
  // (finite codebook entries and scales times zero)
  const bf16x8_t zero8 = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    if (g0 + i >= G) {   // wave-uniform
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mt = 0; mt < MR; ++mt) xf[i][s][mt] = zero8;
        if constexpr (kXL) xt[i][s] = zero8;
      }
    }
  }

  floatx4 xs[GW][MT];
  if constexpr (!kLut) {
#pragma unroll
    for (int i = 0; i < GW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        xs[i][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xs[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              neg136, (kXL && mt == 1) ? xt[kXL ? i : 0][s] : xf[i][s][mt < MR ? mt : 0],
              xs[i][mt], 0, 0, 0);
      }
  }
  if constexpr (kXL) {
#pragma unroll
    for (int i = 0; i < GW; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) xl[((wave * GW + i) * 4 + s) * 64 + lane] = xt[i][s];
  }
  // the header was loaded ahead of the activations, which the code above has
  // waited for: tested once here, for every store below
  const bool hdr_ok = header_word_ok(hdr, kLut ? 2 : 1, N, K);

  auto finish = [&](const PersistTile<GW, kLut>& A, int t, int slot, bool store) {
    floatx4 tot[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kLut) {
      floatx4 t2[2][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) t2[0][mt] = t2[1][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        bf16x8_t a[4];
        lut2_operands(A.w[i].x, A.book.x, A.book.y, a[0], a[1]);
        lut2_operands(A.w[i].y, A.book.x, A.book.y, a[2], a[3]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            t2[i & 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], xf[i][s][mt], t2[i & 1][mt], 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) tot[mt] = t2[0][mt] + t2[1][mt];
    } else {
      // every group's MFMA chains first, then the fp32 scale arithmetic, so
      // no VALU instruction waits on an MFMA it has just issued
      floatx4 acc[GW][MT];
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[i][mt] = xs[i][mt];
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const uint32_t wd[4] = {A.w[i].x, A.w[i].y, A.w[i].z, A.w[i].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t op = int4_operand(wd[s], nib_mask, bf16_128);
          acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, xf[i][s][0], acc[i][0], 0, 0, 0);
          if constexpr (MT == 2)
            acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                op, kXL ? xl[((wave * GW + i) * 4 + s) * 64 + lane] : xf[i][s][MR - 1], acc[i][1],
                0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const uint32_t s01 = A.s[i].x, s23 = A.s[i].y;
        const float sc[4] = {__uint_as_float(s01 << 16), __uint_as_float(s01 & 0xFFFF0000u),
                             __uint_as_float(s23 << 16), __uint_as_float(s23 & 0xFFFF0000u)};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) tot[mt][r] = fmaf(sc[r], acc[i][mt][r], tot[mt][r]);
      }
    }
    // partial sums -> LDS slot; 4 * MT waves each add one component
    constexpr int kRedStride = persist_red_stride(MT, kLut);
    float* rs = red + size_t(slot) * NW * MT * 4 * kRedStride;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) rs[((wave * MT + mt) * 4 + r) * kRedStride + lane] = tot[mt][r];
    __syncthreads();
    // (a blob of another format or shape is read but never stored from)
    // One m-tile: wave rq adds the partial sums of token rows 4 rq .. 4 rq + 3,
    // all 16 columns (lane: row lane / 16, column lane % 16; accumulator lane
    // row + 16 (column / 4), component column % 4, held that output), so each
    // store instruction writes 4 whole 32-byte row pieces of the tile:
    // 1.003-1.023x on gate_up and LUT2 30720 x 3840 at M = 1-16, against one
    // component (every fourth column, 2-byte pieces) per wave.  Two m-tiles
    // keep the component-per-wave form (0.98x the other way).
    if (wave < 4 * MT && store && hdr_ok) {
      const int mt = wave >> 2;
      const int mrow = MT == 1 ? 4 * (wave & 3) + (lane >> 4) : (lane & 15);
      const int col = MT == 1 ? (lane & 15) : 4 * (lane >> 4) + (wave & 3);
      const int src = ((mt * 4 + (col & 3)) * kRedStride) + mrow + 16 * (col >> 2);
      float v[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) v[w] = rs[w * MT * 4 * kRedStride + src];
#pragma unroll
      for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
        for (int w = 0; w < h; ++w) v[w] += v[w + h];
      const int m = mt * 16 + mrow, n = t * 16 + col;
      if (m < M) {
        if (S > 1)
          part[(int64_t(sl) * M + m) * N + n] = v[0];   // this slice's partial sum
        else if (kBF16Out)
          static_cast<uint16_t*>(y)[int64_t(m) * N + n] = to_bf16(v[0]);
        else
          static_cast<float*>(y)[int64_t(m) * N + n] = v[0];
      }
    }
  };

  // the launch guarantees gridDim.x / S <= T, so every block has a first tile.
  // The second tile of an iteration may not exist (t + stride >= T): it is
  // then computed from the clamped (valid) loads but not stored.  Keeping the
  // arithmetic unconditional keeps the loop free of branches around waits,
  // which would make the compiler wait for the in-flight prefetch as well.
  // (the scheduling barriers keep each prefetch ahead of the arithmetic; the
  // compiler would otherwise sink it below, to save registers)
  for (; t < T; t += 2 * stride) {
    load(B, min(t + stride, T - 1));
    __builtin_amdgcn_sched_barrier(0);
    finish(A, t, 0, true);
    load(A, min(t + 2 * stride, T - 1));
    __builtin_amdgcn_sched_barrier(0);
    finish(B, t + stride, 1, t + stride < T);
  }
}

// The dynamic-LDS limit is a per-function attribute: raised once per
// instantiation that needs more than the default 64 KiB.
template <int GW, int MT, bool kLut, bool kBF16Out>
hipError_t persist_lds_attr() {
  static std::atomic<int> done[64];
  if (persist_lds_bytes(GW, MT, kLut) <= 65536) return hipSuccess;
  return lds_limit_once(done,
                        reinterpret_cast<const void*>(decode_persist_kernel<GW, MT, kLut, kBF16Out>),
                        int(persist_lds_bytes(GW, MT, kLut)));
}

// Sum of the k slices' fp32 partial sums, in slice order: y = part[0] + ...
// + part[S-1] (deterministic), four outputs per thread.
template <bool kBF16Out>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part, int S,
                                                            int64_t n4, void* __restrict__ y,
                                                            const uint8_t* __restrict__ blob,
                                                            int fmt, int N, int K) {
  // the partial sums were not written when the blob does not match (tested
  // before the store, as in the main kernel)
  const uint32_t hdr = header_word(blob);   // tested before the store
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const floatx4* p = reinterpret_cast<const floatx4*>(part);
  floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
  if (i < n4) {
    v = p[i];
    for (int j = 1; j < S; ++j) v += p[int64_t(j) * n4 + i];
  }
  if (!header_word_ok(hdr, fmt, N, K) || i >= n4) return;
  if (kBF16Out) {
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    reinterpret_cast<uint2*>(y)[i] = o;
  } else {
    reinterpret_cast<floatx4*>(y)[i] = v;
  }
}

template <bool kLut, int MT, int NTB, int WMAX, int KWT, int XQ, bool kRowsPerChunk = false>
hipError_t launch_decode_xq(const void* x, const uint8_t* blob, const BlobLayout& L, int M,
                            int m0, int N, int K, void* y, int y_dtype, hipStream_t s) {
  const int blocks = (N / 16 + NTB - 1) / NTB;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if constexpr (kLut) {
    if (y_dtype == 1)
      lut2_kernel<MT, NTB, WMAX, KWT, XQ, true><<<blocks, KWT * 64, 0, s>>>(
          xp, blob, L.codes_off, L.aux_off, M, m0, N, K, y);
    else
      lut2_kernel<MT, NTB, WMAX, KWT, XQ, false><<<blocks, KWT * 64, 0, s>>>(
          xp, blob, L.codes_off, L.aux_off, M, m0, N, K, y);
  } else {
    if (y_dtype == 1)
      w4a16_kernel<MT, NTB, WMAX, KWT, XQ, true, kRowsPerChunk><<<blocks, KWT * 64, 0, s>>>(
          xp, blob, L.codes_off, L.aux_off, M, m0, N, K, y);
    else
      w4a16_kernel<MT, NTB, WMAX, KWT, XQ, false, kRowsPerChunk><<<blocks, KWT * 64, 0, s>>>(
          xp, blob, L.codes_off, L.aux_off, M, m0, N, K, y);
  }
  return hipGetLastError();
}

// Chunks of at most four groups: the activation rows are staged (XQ = row
// quads of this pass's tokens, 0 for a single token) -- once, when a wave's
// groups fit one chunk, else per chunk (INT4 with two m-tiles: 32-token
// passes); otherwise fragments are loaded per group (XQ = -1).
template <bool kLut, int MT, int NTB, int WMAX, int KWT>
hipError_t launch_decode(const void* x, const uint8_t* blob, const BlobLayout& L, int M, int m0,
                         int N, int K, void* y, int y_dtype, hipStream_t s) {
  const int gpw = (K / 128 + KWT - 1) / KWT;
  const int rows = M - m0 < 16 * MT ? M - m0 : 16 * MT;
  if constexpr (WMAX <= 4) {
    if (gpw <= WMAX) {
      if constexpr (MT == 1) {
        if (rows == 1)
          return launch_decode_xq<kLut, MT, NTB, WMAX, KWT, 0>(x, blob, L, M, m0, N, K, y, y_dtype, s);
        if (rows <= 4)
          return launch_decode_xq<kLut, MT, NTB, WMAX, KWT, 1>(x, blob, L, M, m0, N, K, y, y_dtype, s);
        if (rows <= 8)
          return launch_decode_xq<kLut, MT, NTB, WMAX, KWT, 2>(x, blob, L, M, m0, N, K, y, y_dtype, s);
      }
      return launch_decode_xq<kLut, MT, NTB, WMAX, KWT, 4>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    }
    if constexpr (!kLut && MT == 2)
      return launch_decode_xq<kLut, MT, NTB, WMAX, KWT, 4, true>(x, blob, L, M, m0, N, K, y,
                                                                  y_dtype, s);
  }
  return launch_decode_xq<kLut, MT, NTB, WMAX, KWT, -1>(x, blob, L, M, m0, N, K, y, y_dtype, s);
}

// Largest chunk whose weight registers fit without spilling (the INT4 operand
// is 16 bytes per lane and group per row tile, the LUT2 one 8).
// Largest chunk whose registers fit without spilling (8 waves per block may
// use up to 256 VGPRs; 16 waves per block, up to 128).
constexpr int chunk_cap(bool lut, int mt, int ntb, int kwt) {
  return kwt == 16 ? (lut ? 8 : (mt * ntb == 1 ? 6 : 2))
                   : (lut ? 16 : (mt * ntb == 1 ? 16 : (mt * ntb == 2 ? 8 : 2)));
}

template <bool kLut, int MT, int NTB, int KWT>
hipError_t launch_decode_w(const void* x, const uint8_t* blob, const BlobLayout& L, int M,
                           int m0, int N, int K, void* y, int y_dtype, hipStream_t s) {
  constexpr int kCap = chunk_cap(kLut, MT, NTB, KWT);
  switch (pick_chunk((K / 128 + KWT - 1) / KWT, kCap)) {
    // pick_chunk never exceeds kCap; the min() only keeps unused cases from
    // instantiating kernels that would spill
    case 2: return launch_decode<kLut, MT, NTB, 2, KWT>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    case 4: return launch_decode<kLut, MT, NTB, cmin(4, kCap), KWT>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    case 6: return launch_decode<kLut, MT, NTB, cmin(6, kCap), KWT>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    case 8: return launch_decode<kLut, MT, NTB, cmin(8, kCap), KWT>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    case 12: return launch_decode<kLut, MT, NTB, cmin(12, kCap), KWT>(x, blob, L, M, m0, N, K, y, y_dtype, s);
    default: return launch_decode<kLut, MT, NTB, cmin(16, kCap), KWT>(x, blob, L, M, m0, N, K, y, y_dtype, s);
  }
}

}  // namespace

// Plan of the k-sliced persistent kernel: GW groups per wave, S k slices of
// NW GW groups, P tile walkers per slice (S P blocks).  S == 0: no plan.
DecodeSplit decode_split_plan(bool lut, int64_t m, int64_t n, int64_t k) {
  DecodeSplit best{0, 0, 0, 0};
  const int cus = device_cu_count();
  if (m < 1 || m > 32 || cus <= 0 || n % 16 != 0 || k % 128 != 0) return best;
  const int64_t T = n / 16, G = k / 128;
  const int mt = m > 16 ? 2 : 1;
  const int nw = persist_waves(mt, lut);
  // Measured against the unsplit kernels (graph replay over rotating weight
  // copies, Qwen3-8B-like and Gemma3-like decode shapes): the split pays only
  // where k is long and the batch large enough that every block loading the
  // whole activation dominates -- W4A16 4096 x 12288 at M = 9 / 16 / 32:
  // 11.9 / 12.4 / 27.7 us unsplit, 10.5 / 11.4 / 16.3 us split; LUT2
  // 3840 x 15360 at M = 9 / 16: 12.2 / 13.5 us unsplit, 11.2 / 12.0 us split
  // -- and costs 0.6-0.9x at M <= 8 and on K <= 4096 (the second launch adds
  // ~1.7 us).  One block per CU (S P = CUs) measured best: walkers sharing a
  // CU slowed every split plan by 5-30 %.
  if (G <= KW * 4 || m <= 8) return best;
  int64_t best_cost = INT64_MAX;
  for (int gw = 1; gw <= 4; ++gw) {
    if (mt == 2 && lut && gw > 2) break;
    const int64_t S = (G + nw * gw - 1) / (nw * gw);
    if (S < 2) continue;
    const int64_t P = std::min<int64_t>(T, cus / S);
    if (P < 1) continue;
    // (row tile, group) units per CU, plus a round trip per pair of tiles
    const int64_t tiles = (T + P - 1) / P;
    const int64_t cost = tiles * nw * gw + 32 * ((tiles + 1) / 2);
    if (cost < best_cost) {
      best_cost = cost;
      best = DecodeSplit{gw, mt, int(S), int(P)};
    }
  }
  return best;
}

size_t decode_split_bytes(const DecodeSplit& p, int64_t m, int64_t n) {
  return p.S < 2 ? 0 : size_t(p.S) * size_t(m) * size_t(n) * sizeof(float);
}

namespace {

template <bool kLut>
hipError_t launch_decode_all(const void* x, const void* w_packed, int64_t m, int64_t n, int64_t k,
                             void* y, int y_dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  const BlobLayout L = blob_layout(kLut ? 2 : 1, n, k);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  // two row tiles per block when there are enough tiles to keep every CU busy
  // (N >= 6144 gives at least 192 blocks of 512 threads)
  const bool wide = n / 16 >= 384;
  const int G = static_cast<int>(k / 128);
  const int cus = device_cu_count();
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  auto run = [&](auto kern, int waves, int grid, size_t lds, hipError_t attr, int S,
                 float* part) {
    if (attr != hipSuccess) return attr;
    kern<<<grid, waves * 64, lds, s>>>(xp, blob, L.codes_off, L.aux_off, int(m), int(n),
                                       int(k), y, S, part);
    return hipGetLastError();
  };
#define QL_PERSIST_RUN(GW, MT, GRID, S, PART)                                                \
  (y_dtype == 1                                                                             \
       ? run(decode_persist_kernel<GW, MT, kLut, true>, persist_waves(MT, kLut), GRID,       \
             persist_lds_bytes(GW, MT, kLut), persist_lds_attr<GW, MT, kLut, true>(), S, PART) \
       : run(decode_persist_kernel<GW, MT, kLut, false>, persist_waves(MT, kLut), GRID,      \
             persist_lds_bytes(GW, MT, kLut), persist_lds_attr<GW, MT, kLut, false>(), S, PART))
  // k-sliced persistent kernel with the caller's workspace: each block owns
  // one k slice of several row tiles, so its activation fragments serve all
  // of them; the slices' fp32 partial sums are added by a second launch
  const DecodeSplit sp = decode_split_plan(kLut, m, n, k);
  if (sp.S >= 2 && ws != nullptr && ws_bytes >= decode_split_bytes(sp, m, n)) {
    float* part = static_cast<float*>(ws);
    const int grid = sp.S * sp.P;
    hipError_t e = hipSuccess;
    if (sp.mt == 1) {
      switch (sp.gw) {
        case 1: e = QL_PERSIST_RUN(1, 1, grid, sp.S, part); break;
        case 2: e = QL_PERSIST_RUN(2, 1, grid, sp.S, part); break;
        case 3: e = QL_PERSIST_RUN(3, 1, grid, sp.S, part); break;
        default: e = QL_PERSIST_RUN(4, 1, grid, sp.S, part); break;
      }
    } else if constexpr (kLut) {
      e = sp.gw == 1 ? QL_PERSIST_RUN(1, 2, grid, sp.S, part)
                     : QL_PERSIST_RUN(2, 2, grid, sp.S, part);
    } else {
      switch (sp.gw) {
        case 1: e = QL_PERSIST_RUN(1, 2, grid, sp.S, part); break;
        case 2: e = QL_PERSIST_RUN(2, 2, grid, sp.S, part); break;
        case 3: e = QL_PERSIST_RUN(3, 2, grid, sp.S, part); break;
        default: e = QL_PERSIST_RUN(4, 2, grid, sp.S, part); break;
      }
    }
    if (e != hipSuccess) return e;
    return launch_decode_reduce(part, sp.S, m, n, y, y_dtype, blob, kLut ? 2 : 1, k, s);
  }
  // one pass over the batch (M <= 32), K <= 4096 and at least two row tiles
  // per CU: persistent kernel
  if (m <= 32 && G <= KW * 4 && cus > 0 && n / 16 >= 2 * cus) {
    const int T = int(n / 16);
    // every block must own at least two tiles, and the grid never exceeds T
    auto grid_of = [&](int per_cu) { return T >= 2 * per_cu * cus ? per_cu * cus : cus; };
#define QL_PERSIST(GW, MT) \
    return QL_PERSIST_RUN(GW, MT, grid_of(persist_blocks_per_cu(GW, MT, kLut)), 1, nullptr)
    if (m > 16) {
      if constexpr (kLut) {
        QL_PERSIST(2, 2);   // 16 waves: two groups per wave cover K <= 4096
      } else {
        if (G <= KW * 2) QL_PERSIST(2, 2);
        QL_PERSIST(4, 2);
      }
    }
    if (G <= KW * 2) {
      QL_PERSIST(2, 1);
    }
    QL_PERSIST(4, 1);
#undef QL_PERSIST
  }
#undef QL_PERSIST_RUN
  // one m-tile, one row tile per block and long K: pipelined k-split kernel
  const int gpw8 = (G + KW - 1) / KW;
  if (m <= 16 && !wide && gpw8 >= 8) {
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const int M = int(m), N = int(n), K = int(k), T = int(n / 16);
    // chunks of 4 groups
#define QL_PIPE_NQ(W, NQ)                                                                   \
    {                                                                                      \
      if (y_dtype == 1)                                                                    \
        decode_pipe_kernel<W, kLut, NQ, true><<<T, KW * 64, 0, s>>>(xp, blob, L.codes_off, \
                                                                   L.aux_off, M, N, K, y); \
      else                                                                                 \
        decode_pipe_kernel<W, kLut, NQ, false><<<T, KW * 64, 0, s>>>(xp, blob, L.codes_off,\
                                                                    L.aux_off, M, N, K, y);\
      return hipGetLastError();                                                            \
    }
#define QL_PIPE(W)                       \
    {                                    \
      if (M == 1) QL_PIPE_NQ(W, 0)       \
      if (M <= 4) QL_PIPE_NQ(W, 1)       \
      if (M <= 8) QL_PIPE_NQ(W, 2)       \
      QL_PIPE_NQ(W, 4)                   \
    }
    QL_PIPE(4)
#undef QL_PIPE
#undef QL_PIPE_NQ
  }
  for (int64_t m0 = 0; m0 < m; m0 += 32) {
    const int rows = static_cast<int>(m - m0 < 32 ? m - m0 : 32);
    const int a = int(m), b = int(m0), c = int(n), d = int(k);
    hipError_t e;
    if (rows <= 16)
      e = wide ? launch_decode_w<kLut, 1, 2, KW>(x, blob, L, a, b, c, d, y, y_dtype, s)
               : launch_decode_w<kLut, 1, 1, KW>(x, blob, L, a, b, c, d, y, y_dtype, s);
    else
      e = wide ? launch_decode_w<kLut, 2, 2, KW>(x, blob, L, a, b, c, d, y, y_dtype, s)
               : launch_decode_w<kLut, 2, 1, KW>(x, blob, L, a, b, c, d, y, y_dtype, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode_reduce(const float* part, int S, int64_t m, int64_t n, void* y,
                                int y_dtype, const uint8_t* blob, int fmt, int64_t k,
                                hipStream_t s) {
  const int64_t n4 = m * n / 4;
  const int rb = int((n4 + 255) / 256);
  if (y_dtype == 1)
    decode_reduce_kernel<true><<<rb, 256, 0, s>>>(part, S, n4, y, blob, fmt, int(n), int(k));
  else
    decode_reduce_kernel<false><<<rb, 256, 0, s>>>(part, S, n4, y, blob, fmt, int(n), int(k));
  return hipGetLastError();
}

hipError_t launch_gemm_w4a16(const void* x, const void* w_packed, int64_t m, int64_t n, int64_t k,
                             void* y, int y_dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  return launch_decode_all<false>(x, w_packed, m, n, k, y, y_dtype, ws, ws_bytes, s);
}

hipError_t launch_gemm_lut2(const void* x, const void* w_packed, int64_t m, int64_t n, int64_t k,
                            void* y, int y_dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  return launch_decode_all<true>(x, w_packed, m, n, k, y, y_dtype, ws, ws_bytes, s);
}

}  // namespace qlin
