// NVFP4 W4A4 prefill GEMM for gfx950, block-cooperative dequantization.
//
//   Y[m,n] = s_tA s_tW sum_g sA[m,g] sW[n,g] sum_{k in g} E2M1(a[m,k]) E2M1(w[n,k])
//
// Same exact arithmetic as the register-dequant kernel (fp16 operands that
// hold E2M1 * E4M3 exactly, v_mfma_f32_16x16x32_f16, fp32 accumulation, the
// tensor scales in the epilogue), organised so that every code is dequantized
// once per 256 x 256 block instead of once per wavefront that uses it.  On
// gfx950 VALU work and MFMA work share the SIMD issue slots (measured:
// non-interleaved they simply add up), so dequantization per MFMA is the
// quantity to minimise: 1 VALU op per MFMA here against 4 in the
// register-dequant design.
//
// Block 256 (n) x 256 (m), 8 wavefronts in 2 (n) x 4 (m), each 128 x 64
// (8 x 4 MFMA tiles, 128 fp32 accumulators per lane; 2 waves per SIMD).  K
// advances 64 per stage.  Per stage every thread owns one of the 512 rows (256
// weight rows, then 256 activation rows):
//   global -> registers: 32 code bytes + 4 E4M3 scale bytes,
//   registers -> fp16: 64 values (cvt fp4->f16, exact pk_mul by the scale),
//   registers -> LDS: 8 x 16 bytes.
// The fp16 tiles are double buffered in LDS (2 stages x 2 operands x 256 rows
// x 160 bytes = 160 KiB, one block per CU); stage s+1 is dequantized while
// the MFMAs of stage s run, one 16-byte dequant store after every MFMA row.
// Codes for stage s+2 are loaded at the start of stage s (two register sets).
// LDS rows are padded from 128 to 160 bytes, which measured fewest bank
// conflicts for the 16-byte fragment reads and the row-wise stores together.
// Tiles are visited XCD-major (consecutive workgroups go to different XCDs,
// so each XCD gets a contiguous run of tiles) and in groups of 4 m-tiles, so
// the 32 tiles in flight on one XCD span 4 activation and 8 weight panels
// that they share in L2.  Measured against groups of 1, 2, 3, 6 and 8 (one
// process, interleaved, outputs bit-identical): 4 was fastest or within 1 %
// on the Qwen3-8B-like prefill set (against 8: o_proj +15 %, gate_up +2.5 %,
// down +2 %) and on the 27B-class gate_up (+7 %); only the 27B-class down
// (K = 17408) was 4 % slower.
#include "qlin_internal.hpp"

namespace qlin {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 256, BM = 256, BK = 64;
constexpr int GROUP_M = 4;

__device__ __forceinline__ half2_t cvt2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// 8 codes -> 8 exact fp16 products with the group scale, packed for one store
__device__ __forceinline__ u32x4 dequant8(uint32_t w, half2_t s) {
  return u32x4{__builtin_bit_cast(uint32_t, cvt2(w, 0) * s),
               __builtin_bit_cast(uint32_t, cvt2(w, 1) * s),
               __builtin_bit_cast(uint32_t, cvt2(w, 2) * s),
               __builtin_bit_cast(uint32_t, cvt2(w, 3) * s)};
}

// E4M3 scale g (0..3) of a dword of four, as an fp16 pair: one packed
// conversion per two scales (exact: every E4M3 value is an fp16 value; an
// exhaustive GPU check of all byte pairs agreed), broadcast by the multiply
__device__ __forceinline__ half2_t scale_h2(uint32_t w4, int g) {
  const half2_t two = g < 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w4, 1.0f, false)
                            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w4, 1.0f, true);
  const _Float16 h = two[g & 1];
  return half2_t{h, h};
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// tile t (0 .. tiles_m * tiles_n - 1, after any XCD remap) -> its origin:
// groups of GROUP_M m-tiles, n-tiles in order within a group
__device__ __forceinline__ void coop_tile_origin(int t, int tiles_m, int tiles_n, int& m0,
                                                 int& n0) {
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (t / in_group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  m0 = (first_m + (t % in_group) % gsz) * BM;
  n0 = ((t % in_group) / gsz) * BN;
}

// WAVES = 4: 2 x 2 waves of 128 x 128 (1 wave per SIMD);
// WAVES = 8: 2 (n) x 4 (m) waves of 128 x 64 (2 waves per SIMD).
template <int WAVES, int RS, bool kBF16Out>
__global__ __launch_bounds__(WAVES * 64, 1) void w4a4_coop_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ blob, int64_t wc_off,
    int64_t ws_off, int M, int N, int K, void* __restrict__ y, int full, int tail, int splits,
    float* __restrict__ part) {
  if (!blob_matches(blob, 0, N, K)) return;   // before any barrier: uniform
  constexpr int NTHR = WAVES * 64;
  constexpr int TILE_BYTES = 256 * RS;
  constexpr int WGM = WAVES / 2;          // waves along m
  constexpr int TN = 8;                   // 16-row MFMA tiles per wave along n (128)
  constexpr int TM = BM / WGM / 16;       // along m: 8 (128) or 4 (64)
  constexpr int ROWS = 512 / NTHR;        // rows each thread dequantizes per stage (2 or 1)
  constexpr int DW = 8 * ROWS;            // dwords of codes per thread per stage
  constexpr int STEP = 2 * TN / DW;       // fragment iterations per dequantized dword
  static_assert(STEP >= 1 && (2 * TN) % DW == 0, "dequant interleave");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [2][W tile, X tile]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;

  const int KT = K / 128;
  const int S = K / BK;
  const int NT16 = N / 16;

  // Blocks [0, full) take whole tiles; blocks past that take one k slice of
  // one of the `tail` last tiles (slice-major, so the slices of a tile run on
  // different CUs) and leave an fp32 partial tile for the reduction kernel.
  int t = blockIdx.x;
  int st_begin = 0, st_end = S, slot = -1, slice = 0;
  if (t >= full) {
    const int u = t - full;
    slot = u % tail;
    slice = u / tail;
    t = full + slot;
    const int pairs = S / 2;             // the loop advances two stages at a time
    st_begin = 2 * (slice * pairs / splits);
    st_end = 2 * ((slice + 1) * pairs / splits);
  } else if ((full & 7) == 0) {
    t = (t & 7) * (full >> 3) + (t >> 3);
  }
  int m0, n0;
  coop_tile_origin(t, tiles_m, tiles_n, m0, n0);

  // dequantization rows of this thread: row j of 512 = tid + j * NTHR; rows < 256
  // are weight rows n0 + row, the rest activation rows m0 + row - 256 (the same
  // kind for a whole wavefront).  Rows past N or M are clamped to the last
  // valid one: their products only reach outputs that are never stored, and
  // the loads stay unconditional (a load under a branch makes the compiler
  // wait for every outstanding load where the branch rejoins, which would
  // expose the prefetch latency each stage).  Loads go through buffer
  // resources: the row offset is a per-thread constant, the stage offset
  // and the operand are wave-uniform, so no vector instruction computes an
  // address (offsets fit 31 bits; the launcher checks).
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t rcw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(blob + wc_off), 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(blob + ws_off), 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rcx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(xcodes), 0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(xscales), 0, 0x7FFFFFFF, 0x00020000);
  bool isw[ROWS];
  int lrow[ROWS];
  uint32_t vc[ROWS], vs[ROWS];
#pragma unroll
  for (int j = 0; j < ROWS; ++j) {
    const int row = tid + j * NTHR;
    isw[j] = wave_u * 64 + j * NTHR < 256;   // wave-uniform
    lrow[j] = row & 255;
    if (isw[j]) {
      const int wrow = n0 + row;
      const uint32_t wt = uint32_t(min(wrow >> 4, NT16 - 1));
      vc[j] = (wt * uint32_t(KT) * 16u + uint32_t(wrow & 15)) * 64u;
      vs[j] = (wt * uint32_t(KT) * 16u + uint32_t(wrow & 15)) * 8u;
    } else {
      const uint32_t xrow = uint32_t(min(m0 + row - 256, M - 1));
      vc[j] = xrow * uint32_t(K / 2);
      vs[j] = xrow * uint32_t(K / 16);
    }
  }

  // codes + scales of one stage for this thread's rows; two sets (ping-pong) so
  // the loads for stage st+2 are issued at the start of stage st
  struct Regs {
    uint4 c[ROWS][2];
    uint32_t sc[ROWS];
  };
  Regs ra, rb;
  auto gload = [&](Regs& R, int st) {
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
      const int co = isw[j] ? (st >> 1) * 1024 + (st & 1) * 32 : st * 32;
      const int so = isw[j] ? (st >> 1) * 128 + (st & 1) * 4 : st * 4;
      const __amdgpu_buffer_rsrc_t rc = isw[j] ? rcw : rcx, rs = isw[j] ? rsw : rsx;
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rc, vc[j], co, 0);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rc, vc[j], co + 16, 0);
      R.c[j][0] = make_uint4(a[0], a[1], a[2], a[3]);
      R.c[j][1] = make_uint4(b[0], b[1], b[2], b[3]);
      R.sc[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs[j], so, 0);
    }
  };
  // dequantize dword e (0 .. DW-1) of this thread's rows into LDS buffer buf
  auto dq_store = [&](const Regs& R, int buf, int e) {
    const int j = e >> 3, d = e & 7;
    const u32x4 h = dequant8(pick(R.c[j][d >> 2], d & 3), scale_h2(R.sc[j], d >> 1));
    uint8_t* dst = smem + buf * 2 * TILE_BYTES + (isw[j] ? 0 : TILE_BYTES) + lrow[j] * RS + d * 16;
    *reinterpret_cast<u32x4*>(dst) = h;
  };

  floatx4 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  gload(ra, st_begin);
#pragma unroll
  for (int e = 0; e < DW; ++e) dq_store(ra, 0, e);
  gload(rb, st_begin + 1);   // every range holds an even number >= 2 of stages
  __syncthreads();

  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, q = lane >> 4;
  const int wbase = (wn * 128 + r) * RS + q * 16;
  const int xbase = (wm * (TM * 16) + r) * RS + q * 16;

  // one stage: MFMAs on LDS buffer `buf` while `nxt` (stage st+1's codes) is
  // dequantized into the other buffer
  auto stage = [&](int buf, const Regs& nxt) {
    const uint8_t* wt = smem + buf * 2 * TILE_BYTES;
    const uint8_t* xt = wt + TILE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8_t xf[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j)
        xf[j] = *reinterpret_cast<const half8_t*>(xt + xbase + j * 16 * RS + s * 64);
      half8_t wf = *reinterpret_cast<const half8_t*>(wt + wbase + s * 64);
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        half8_t wn_f = wf;
        if (i + 1 < TN)
          wn_f = *reinterpret_cast<const half8_t*>(wt + wbase + (i + 1) * 16 * RS + s * 64);
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf[j], acc[i][j], 0, 0, 0);
        // on the last stage this writes the idle buffer, which nothing reads again
        const int it = s * TN + i;
        if (it % STEP == 0) dq_store(nxt, buf ^ 1, it / STEP);
        wf = wn_f;
      }
    }
  };
  // The prefetches are unconditional (the stage index is clamped; reloading the
  // last stage is harmless): a load under a branch makes the compiler wait for
  // every outstanding load at the join, which would expose the full latency.
  for (int st = st_begin; st < st_end; st += 2) {
    // even stage: buffer 0; rb holds stage st+1; ra is free -> stage st+2
    gload(ra, min(st + 2, st_end - 1));
    __builtin_amdgcn_sched_barrier(0);   // issue the prefetch here, not after the stage
    stage(0, rb);
    __syncthreads();
    // odd stage: buffer 1; ra holds stage st+2; rb is free -> stage st+3
    gload(rb, min(st + 3, st_end - 1));
    __builtin_amdgcn_sched_barrier(0);
    stage(1, ra);
    __syncthreads();
  }

  if (slot >= 0) {
    // partial tile, unscaled, in the accumulators' own order: each wavefront
    // store is one contiguous 1 KiB run
    floatx4* dst = reinterpret_cast<floatx4*>(part) +
                   (int64_t(slot * splits + slice) * WAVES + wave) * (TN * TM * 64) + lane;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) dst[(i * TM + j) * 64] = acc[i][j];
    return;
  }
  const float stv = a_ts[0] * reinterpret_cast<const BlobHeader*>(blob)->tensor_scale;
  if constexpr (kBF16Out) {
    // The accumulators hold 4 consecutive columns of one row per lane, so a
    // direct store instruction writes 16 rows x 32 bytes: every 128-byte line
    // of the output is written in four partial pieces.  Each wave instead
    // passes its 128 (n) x 64 (m) bf16 tile through a private LDS region
    // (row-major, 288-byte rows: conflict-free 8-byte writes and 16-byte
    // reads) and stores whole rows, 4 rows x 256 bytes per instruction.  LDS
    // is idle here (every wave has passed the last stage's barrier), and one
    // wave's LDS operations complete in order, so no barrier is needed.
    constexpr int ORS = 288;
    static_assert(WAVES * TM * 16 * ORS <= 2 * 2 * TILE_BYTES, "output staging fits in LDS");
    uint8_t* const ot = smem + wave * (TM * 16 * ORS);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const floatx4 v = acc[i][j] * stv;
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(ot + (16 * j + r) * ORS + (16 * i + 4 * q) * 2) = o;
      }
    __asm__ volatile("" ::: "memory");   // keep the reads below the writes
    const int n = n0 + wn * 128 + 8 * (lane & 15);
#pragma unroll
    for (int it = 0; it < TM * 4; ++it) {
      const int rr = 4 * it + (lane >> 4);
      const uint4 v = *reinterpret_cast<const uint4*>(ot + rr * ORS + 16 * (lane & 15));
      const int m = m0 + wm * (TM * 16) + rr;
      if (m < M && n < N)   // N is a multiple of 16: a lane's 8 columns are all in or all out
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + int64_t(m) * N + n) = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int n = n0 + wn * 128 + i * 16 + 4 * q;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + wm * (TM * 16) + j * 16 + r;
        if (m >= M) continue;
        *reinterpret_cast<floatx4*>(static_cast<float*>(y) + int64_t(m) * N + n) = acc[i][j] * stv;
      }
    }
  }
}

// Sum of the k slices of the split tiles, in slice order (deterministic),
// times the tensor scales, stored like the main epilogue.  Block = (tail
// slot, 16-column strip i of each wave's 128 columns), so the reduction
// spreads over tail * 8 blocks; each thread loads all MAXS slices of its four
// accumulators before adding (slice indices past `splits` re-read the last
// slice and are not added), so one memory round trip serves the whole sum.
template <int WAVES, int MAXS, bool kBF16Out>
__global__ __launch_bounds__(WAVES * 64) void w4a4_split_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ a_ts,
    const uint8_t* __restrict__ blob, int M, int N, int K, int full, int splits,
    void* __restrict__ y) {
  if (!blob_matches(blob, 0, N, K)) return;
  constexpr int WGM = WAVES / 2, TN = 8, TM = BM / WGM / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = blockIdx.x / TN, i = blockIdx.x % TN;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int m0, n0;
  coop_tile_origin(full + slot, tiles_m, tiles_n, m0, n0);
  const floatx4* src = reinterpret_cast<const floatx4*>(part) +
                       (int64_t(slot * splits) * WAVES + wave) * (TN * TM * 64) + i * TM * 64 +
                       lane;
  const int64_t slice_stride = int64_t(WAVES) * TN * TM * 64;
  floatx4 v[MAXS][TM];
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int j = 0; j < TM; ++j) v[sl][j] = src[min(sl, splits - 1) * slice_stride + j * 64];
  const float stv = a_ts[0] * reinterpret_cast<const BlobHeader*>(blob)->tensor_scale;
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, q = lane >> 4;
  const int n = n0 + wn * 128 + i * 16 + 4 * q;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    floatx4 a = v[0][j];
#pragma unroll
    for (int sl = 1; sl < MAXS; ++sl)
      if (sl < splits) a += v[sl][j];
    const int m = m0 + wm * (TM * 16) + j * 16 + r;
    if (n >= N || m >= M) continue;
    const floatx4 o = a * stv;
    if (kBF16Out) {
      uint2 h;
      h.x = pack_bf16x2(o[0], o[1]);
      h.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + int64_t(m) * N + n) = h;
    } else {
      *reinterpret_cast<floatx4*>(static_cast<float*>(y) + int64_t(m) * N + n) = o;
    }
  }
}

template <int WAVES, bool kBF16Out>
void launch_split_reduce(const float* part, const float* a_ts, const uint8_t* blob, int64_t m,
                         int64_t n, int64_t k, void* y, const CoopSplit& P, hipStream_t s) {
  const dim3 grid(P.tail * 8), block(WAVES * 64);
  if (P.splits <= 2)
    w4a4_split_reduce_kernel<WAVES, 2, kBF16Out><<<grid, block, 0, s>>>(
        part, a_ts, blob, int(m), int(n), int(k), P.full, P.splits, y);
  else if (P.splits <= 4)
    w4a4_split_reduce_kernel<WAVES, 4, kBF16Out><<<grid, block, 0, s>>>(
        part, a_ts, blob, int(m), int(n), int(k), P.full, P.splits, y);
  else
    w4a4_split_reduce_kernel<WAVES, 8, kBF16Out><<<grid, block, 0, s>>>(
        part, a_ts, blob, int(m), int(n), int(k), P.full, P.splits, y);
}

template <int WAVES, int RS>
hipError_t launch_coop(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                       const uint8_t* blob, const BlobLayout& L, int64_t m, int64_t n,
                       int64_t k, void* y, int y_dtype, float* part, const CoopSplit& P,
                       hipStream_t s) {
  const int blocks = P.full + P.tail * P.splits;
  const size_t lds = 2 * 2 * 256 * RS;
  // the dynamic-LDS limit is a per-kernel, per-device attribute
  static std::atomic<int> done_bf16[64], done_f32[64];
  const hipError_t attr =
      y_dtype == 1
          ? lds_limit_once(done_bf16, reinterpret_cast<const void*>(w4a4_coop_kernel<WAVES, RS, true>),
                           int(lds))
          : lds_limit_once(done_f32, reinterpret_cast<const void*>(w4a4_coop_kernel<WAVES, RS, false>),
                           int(lds));
  if (attr != hipSuccess) return attr;
  if (y_dtype == 1)
    w4a4_coop_kernel<WAVES, RS, true><<<blocks, WAVES * 64, lds, s>>>(
        a_codes, a_scales, a_ts, blob, L.codes_off, L.aux_off, int(m), int(n), int(k), y, P.full,
        P.tail, P.splits, part);
  else
    w4a4_coop_kernel<WAVES, RS, false><<<blocks, WAVES * 64, lds, s>>>(
        a_codes, a_scales, a_ts, blob, L.codes_off, L.aux_off, int(m), int(n), int(k), y, P.full,
        P.tail, P.splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.tail == 0) return e;
  if (y_dtype == 1)
    launch_split_reduce<WAVES, true>(part, a_ts, blob, m, n, k, y, P, s);
  else
    launch_split_reduce<WAVES, false>(part, a_ts, blob, m, n, k, y, P, s);
  return hipGetLastError();
}

}  // namespace

// Tiles are dispatched in rounds of one per CU.  When the last round (or a
// problem of less than one round) is at most half full, its tiles are split
// along k into `splits` slices (pairs of stages, at most 8 slices) so that
// the round occupies the CUs; the slices' fp32 partial tiles are summed by a
// second launch.  Measured on the 27B-class layers at M = 4096: o_proj
// (5120 x 5120, 1.25 rounds) 863 -> 992 TFLOP/s, down (5120 x 17408, 1.25
// rounds) 943 -> 1279, gate_up (8.5 rounds) +2 %.
CoopSplit coop_split_plan(int64_t m, int64_t n, int64_t k) {
  const int tiles = static_cast<int>(((m + BM - 1) / BM) * ((n + BN - 1) / BN));
  const int cus = device_cu_count();
  CoopSplit P{tiles, 0, 1};
  if (cus <= 0) return P;
  const int tail = tiles % cus;
  if (tail == 0) return P;
  int splits = cus / tail;
  const int pairs = static_cast<int>(k / (2 * BK));
  if (splits > pairs) splits = pairs;
  if (splits > 8) splits = 8;
  if (splits < 2) return P;
  return CoopSplit{tiles - tail, tail, splits};
}

size_t coop_split_bytes(const CoopSplit& P) {
  return size_t(P.tail) * P.splits * BM * BN * sizeof(float);
}

hipError_t launch_gemm_w4a4_coop(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const float* a_ts, const void* w_packed, int64_t m, int64_t n,
                                 int64_t k, void* y, int y_dtype, float* part, bool split,
                                 hipStream_t s) {
  const BlobLayout L = blob_layout(0, n, k);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  const int tiles = static_cast<int>(((m + BM - 1) / BM) * ((n + BN - 1) / BN));
  const CoopSplit P = split ? coop_split_plan(m, n, k) : CoopSplit{tiles, 0, 1};
  return launch_coop<8, 160>(a_codes, a_scales, a_ts, blob, L, m, n, k, y, y_dtype, part, P, s);
}

}  // namespace qlin
