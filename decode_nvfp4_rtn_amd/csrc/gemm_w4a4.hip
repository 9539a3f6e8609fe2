// NVFP4 W4A4 prefill GEMM for gfx950 (CDNA4).
//
//   Y[m,n] = s_tA s_tW sum_g sA[m,g] sW[n,g] sum_{k in g} E2M1(a[m,k]) E2M1(w[n,k])
//
// Prefill runs both operands in NVFP4 (Mix-Quant technical summary,
// gist.science, section 2, system-level deployment; Disaggregated
// Quantization, format disaggregation).  Prefill is compute-bound because the
// same weights serve every token (Disaggregated Quantization, opening
// paragraph), so the contraction belongs on the matrix cores.
//
// Reconciling NVFP4 with gfx950.  gfx950's scaled MFMA applies power-of-two
// (E8M0) scales per 32 k, while NVFP4 has E4M3 scales (4 significant bits)
// per 16 k.  A dequantized element E2M1 * E4M3 needs up to 6 significant
// bits, so it is NOT exact in FP8/FP6/FP4, but it IS exact in fp16 (11 bits;
// the range 2^-10 .. 2688 is all normal).  This kernel therefore
//   1. converts each 4-bit code to fp16 with the hardware converter
//      (v_cvt_scalef32_pk_f16_fp4, scale 1.0: two codes per instruction),
//   2. multiplies by the group scale with v_pk_mul_f16 (exact product),
//   3. runs v_mfma_f32_16x16x32_f16 with fp32 accumulation,
//   4. multiplies by s_tA * s_tW in the epilogue.
// Products of dequantized operands are exact in fp32; only the accumulation
// rounds.  The ceiling of this exact formulation is the dense fp16 MFMA rate.
//
// Three kernels share this arithmetic.  The block-cooperative kernel
// (gemm_w4a4_coop.hip) dequantizes each code once per block into fp16 LDS
// tiles of 256 x 256; it runs every problem with m > 128 and more 256 x 256
// tiles than half the CUs (use_coop below), and a smaller problem when the
// caller's workspace lets its tiles be split along k and the split pays
// (split_pays: m > 128, or k >= 8192 for problems of at most half a round).
// Batches of up to 32 tokens take the small-batch kernel (w4a4_small_kernel,
// the decode kernels' k split over waves), and every other problem the
// per-wave kernel below, whose 4x (or, with fewer 128 x 128 tiles than CUs,
// 16x) smaller tiles keep every CU busy.
//
// Tiling.  Block tile 128 (n) x 128 (m), k-step 128, four waves in 2 x 2,
// each wave 64 x 64 = 4 x 4 MFMA tiles.  Codes and scales of both operands are
// staged through LDS (double buffered, one barrier per k-step) in their
// packed 4-bit form, so LDS traffic is a quarter of an fp16 GEMM's; every wave
// dequantizes its own fragments in registers.  MFMA operand k-mapping: lane
// (r = l%16, q = l/16) holds groups 2q and 2q+1 of the k-step (16 contiguous
// code bytes, one 16-byte LDS read), and MFMA (c, s) (c, s in {0,1}) uses the
// 8 codes of group 2q+c, half s.  Both operands use the same mapping, so the
// sum over k is unchanged.  Weights are the A operand (16 n-rows) and
// activations the B operand, so each lane owns 4 consecutive n of one m in
// the output and stores them with one vector store.
//
// Block order: tiles are grouped 8 m-tiles wide for L2 reuse, and block ids
// are remapped so that consecutive tiles land on the same XCD (the hardware
// deals workgroups round-robin over the 8 XCDs, each with its own L2).
//
// Quantize folded into the activation load (kFuse, quantize_gemm_w4a4): the
// per-wave kernel can take X itself (bf16) instead of its NVFP4 codes and
// quantize each k-step's activation tile as it stages it: every thread loads
// 16-byte vectors of 8 bf16 values (unit v: row v / 16, k 8 (v % 16) of the
// step), and with its partner lane, which holds the other half of the
// 16-element group, computes the group's E4M3 scale and the 8 E2M1 codes
// with the quantizer's own steps (nvfp4_encode.hpp), then writes codes and
// scale to the same LDS tiles the code loads fill.  The tensor scale comes
// from the amax pass's partial maxima (each block folds them, as the encode
// pass does) or is the caller's static scale.  The MFMA work is unchanged,
// so outputs are bit-identical to quantize_nvfp4 followed by this kernel;
// the encode is repeated by every block that uses an activation tile.  The
// small-batch kernel has the same variant: each lane loads the 32 bf16
// values of its two groups in a k-step and encodes each group whole
// (encode16_bf16), so it needs no partner lane.
#include "nvfp4_encode.hpp"

namespace qlin {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int RS = 80;             // LDS row stride in bytes (64 data + 16 pad)
constexpr int kThreads = 256;      // 4 waves, 2 (n) x 2 (m)
constexpr int GROUP_M = 8;

__device__ __forceinline__ half2_t h2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// 8 E2M1 codes (low nibble first) times an fp16 group scale -> 8 exact fp16.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s) {
  half2_t a = h2(w, 0) * s, b = h2(w, 1) * s, c = h2(w, 2) * s, d = h2(w, 3) * s;
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E4M3 byte `sel` of `w` as an fp16 pair (exact: E4M3 values are fp16 values).
__device__ __forceinline__ half2_t scale2(uint32_t w, int sel) {
  float f = sel == 0 ? __builtin_amdgcn_cvt_f32_fp8(w, 0) : __builtin_amdgcn_cvt_f32_fp8(w, 1);
  _Float16 h = static_cast<_Float16>(f);
  return half2_t{h, h};
}

__device__ __forceinline__ uint32_t dword(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// WN x WM MFMA tiles (16 x 16 each) per wave; block tile BN x BM with 2 x 2 waves.
// kFuse: xcodes is X itself (bf16 [M, K]) and xscales is unused; the tensor
// scale is folded from partial[0 .. npartial) and stored to *ts by block 0,
// or read from *ts when npartial == 0 (a static scale).  Otherwise xcodes,
// xscales and a_ts are quantize_nvfp4's outputs.
template <int WN, int WM, bool kBF16Out, bool kFuse>
__global__ __launch_bounds__(kThreads) void w4a4_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ blob, int64_t wc_off,
    int64_t ws_off, int M, int N, int K, void* __restrict__ y,
    const uint32_t* __restrict__ partial, int npartial, float* __restrict__ ts) {
  if (!blob_matches(blob, 0, N, K)) return;
  constexpr int BN = 32 * WN, BM = 32 * WM;
  constexpr int WU = BN * 4 / kThreads;   // 16-byte W code units per thread per stage
  constexpr int XU = kFuse ? 1 : BM * 4 / kThreads;   // 16-byte X code units per thread per stage
  constexpr int XB = kFuse ? BM * 16 / kThreads : 1;  // kFuse: 16-byte bf16 X units
  constexpr int SROWS = kFuse ? BN : BN + BM;         // scale rows loaded from memory
  constexpr int SU = (SROWS + kThreads - 1) / kThreads;  // 8-byte scale rows per thread
  static_assert(XB >= 1 && (BM * 16) % kThreads == 0, "activation units");
  __shared__ __attribute__((aligned(16))) uint8_t wc_s[2][BN * RS];
  __shared__ __attribute__((aligned(16))) uint8_t xc_s[2][BM * RS];
  __shared__ __attribute__((aligned(16))) uint8_t sc_s[2][(BN + BM) * 8];
  __shared__ float inv_tab[kFuse ? 128 : 1];
  float s_t = 0.0f, d = 0.0f;
  if constexpr (kFuse) {
    if (npartial > 0) {
      s_t = tensor_scale_from_partials<kThreads>(partial, npartial);
      if (blockIdx.x == 0 && threadIdx.x == 0) *ts = s_t;
    } else {
      s_t = *ts;
    }
    d = 6.0f * s_t;
    fill_inv_table(inv_tab, s_t);
    __syncthreads();
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;

  // XCD-aware remap, then GROUP_M-wide grouped order
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (t / in_group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (t % in_group) % gsz;
  const int tn = (t % in_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int KT = K / 128;
  const int NT16 = N / 16;
  const int wn = wave & 1, wm = wave >> 1;
  const uint8_t* wcodes = blob + wc_off;
  const uint8_t* wscales = blob + ws_off;

  floatx4 acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  uint4 pw[WU], px[XU], pxb[XB];
  uint2 ps[SU];
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      const int u = i * kThreads + tid;
      const int nt = tn * (BN / 16) + (u >> 6);
      pw[i] = nt < NT16 ? *reinterpret_cast<const uint4*>(
                              wcodes + (int64_t(nt) * KT + ks) * 1024 + (u & 63) * 16)
                        : make_uint4(0, 0, 0, 0);
    }
    if constexpr (kFuse) {
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int v = i * kThreads + tid;
        const int m = m0 + (v >> 4);
        pxb[i] = m < M ? *reinterpret_cast<const uint4*>(
                             xcodes + (int64_t(m) * K + ks * 128 + (v & 15) * 8) * 2)
                       : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < XU; ++i) {
        const int u = i * kThreads + tid;
        const int m = m0 + (u >> 2);
        px[i] = m < M ? *reinterpret_cast<const uint4*>(xcodes + int64_t(m) * (K / 2) +
                                                        ks * 64 + (u & 3) * 16)
                      : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int r = i * kThreads + tid;   // 0 .. SROWS-1; W rows first
      if (r >= SROWS) {
        ps[i] = make_uint2(0, 0);
      } else if (r < BN) {
        const int nt = tn * (BN / 16) + (r >> 4);
        ps[i] = nt < NT16 ? *reinterpret_cast<const uint2*>(
                                wscales + (int64_t(nt) * KT + ks) * 128 + (r & 15) * 8)
                          : make_uint2(0, 0);
      } else {
        const int m = m0 + r - BN;
        ps[i] = m < M ? *reinterpret_cast<const uint2*>(xscales + int64_t(m) * (K / 16) + ks * 8)
                      : make_uint2(0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      const int u = i * kThreads + tid;
      const int wr = (u >> 6) * 16 + ((u & 63) >> 2);
      *reinterpret_cast<uint4*>(&wc_s[buf][wr * RS + (u & 3) * 16]) = pw[i];
    }
    if constexpr (kFuse) {
      // quantize the activation tile: a wavefront's 64 units are 4 rows;
      // rows past M (zeros) are encoded unless the whole wavefront is past M
      const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int v = i * kThreads + tid;
        const int row = v >> 4, k8 = v & 15;
        uint32_t c = 0, sc = 0;
        if (m0 + ((i * kThreads + wave_u * 64) >> 4) < M) c = encode8_bf16(pxb[i], d, inv_tab, sc);
        *reinterpret_cast<uint32_t*>(&xc_s[buf][row * RS + k8 * 4]) = c;
        if ((k8 & 1) == 0) sc_s[buf][(BN + row) * 8 + (k8 >> 1)] = uint8_t(sc);
      }
    } else {
#pragma unroll
      for (int i = 0; i < XU; ++i) {
        const int u = i * kThreads + tid;
        *reinterpret_cast<uint4*>(&xc_s[buf][(u >> 2) * RS + (u & 3) * 16]) = px[i];
      }
    }
#pragma unroll
    for (int i = 0; i < SU; ++i)
      if (i * kThreads + tid < SROWS)
        *reinterpret_cast<uint2*>(&sc_s[buf][(i * kThreads + tid) * 8]) = ps[i];
  };

  gload(0);
  sstore(0);
  __syncthreads();

  const int r = lane & 15, q = lane >> 4;
  for (int ks = 0; ks < KT; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < KT) gload(ks + 1);

    uint4 wraw[WN], xraw[WM];
    uint32_t wsc[WN], xsc[WM];
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int row = wn * (BN / 2) + i * 16 + r;
      wraw[i] = *reinterpret_cast<const uint4*>(&wc_s[buf][row * RS + q * 16]);
      wsc[i] = *reinterpret_cast<const uint16_t*>(&sc_s[buf][row * 8 + 2 * q]);
    }
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int row = wm * (BM / 2) + j * 16 + r;
      xraw[j] = *reinterpret_cast<const uint4*>(&xc_s[buf][row * RS + q * 16]);
      xsc[j] = *reinterpret_cast<const uint16_t*>(&sc_s[buf][(BN + row) * 8 + 2 * q]);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {          // d = 2c + s: group 2q + c, half s
      half8_t xf[WM];
#pragma unroll
      for (int j = 0; j < WM; ++j) xf[j] = dequant8(dword(xraw[j], d), scale2(xsc[j], d >> 1));
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        const half8_t wf = dequant8(dword(wraw[i], d), scale2(wsc[i], d >> 1));
#pragma unroll
        for (int j = 0; j < WM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf[j], acc[i][j], 0, 0, 0);
      }
    }

    if (ks + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: scale by s_tA * s_tW.  The accumulators hold 4 consecutive n of
  // one row per lane, so a direct bf16 store instruction writes 16 rows x 32
  // bytes, each output line in several partial pieces; bf16 tiles are
  // instead staged per wave in LDS (the code tiles are idle after the last
  // barrier; row stride 32 WN + 16 bytes: conflict-free 8-byte writes) and
  // stored as whole wave rows, 64 / (2 WN) rows of 32 WN bytes per
  // instruction.  One wave's LDS operations complete in order: no barrier.
  const float st = (kFuse ? s_t : a_ts[0]) * reinterpret_cast<const BlobHeader*>(blob)->tensor_scale;
  if constexpr (kBF16Out) {
    constexpr int RB = 32 * WN;            // bytes of one wave row (16 WN columns)
    constexpr int ORS = RB + 16;
    constexpr int WBYTES = 16 * WM * ORS;  // one wave's staging tile
    static_assert(2 * WBYTES <= 2 * BN * RS && 2 * WBYTES <= 2 * BM * RS, "staging fits");
    uint8_t* const ot = (wave < 2 ? &wc_s[0][0] : &xc_s[0][0]) + (wave & 1) * WBYTES;
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        const floatx4 v = acc[i][j] * st;
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(ot + (16 * j + r) * ORS + (16 * i + 4 * q) * 2) = o;
      }
    __asm__ volatile("" ::: "memory");   // keep the reads below the writes
    constexpr int CPR = RB / 16;           // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;          // rows per store instruction
    const int c = lane % CPR;
    const int n = n0 + wn * (BN / 2) + 8 * c;
#pragma unroll
    for (int it = 0; it < 16 * WM / RPI; ++it) {
      const int rr = RPI * it + lane / CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(ot + rr * ORS + 16 * c);
      const int m = m0 + wm * (BM / 2) + rr;
      if (m < M && n < N)   // N is a multiple of 16: a lane's 8 columns are all in or all out
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + int64_t(m) * N + n) = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int n = n0 + wn * (BN / 2) + i * 16 + 4 * q;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        const int m = m0 + wm * (BM / 2) + j * 16 + r;
        if (m >= M) continue;
        *reinterpret_cast<floatx4*>(static_cast<float*>(y) + int64_t(m) * N + n) = acc[i][j] * st;
      }
    }
  }
}

// Small batches (a pass of up to 16 MT tokens): the decode kernels'
// organisation with NVFP4 operands.  At a few tokens the per-wave kernel's
// blocks are few and each wave's dequantization chain sets the pace; here a
// block of 8 waves owns NTB 16-row weight tiles and the waves split k: each
// lane loads its fragment bytes straight from the blob (row r = l % 16,
// bytes 16 q .. 16 q + 15 of a 128-k step, q = l / 16, i.e. groups 2q and
// 2q + 1 -- the per-wave kernel's fragment mapping, read from the blob's
// [tile][step][16 rows][64 B] order instead of from LDS) and the activation
// fragments of the same k from the code rows, dequantizes both exactly to
// fp16 and runs v_mfma_f32_16x16x32_f16; a chunk of WMAX steps' loads is
// issued at once.  The waves' partial sums meet in LDS in a fixed order, and
// the tensor scales are applied to the sum, as in the other kernels.  Slots
// past the wave's range or past k read a clamped step with a zero scale, so
// they contribute nothing and the loop has no branches around loads.
constexpr int kSmallWaves = 8;
// Batches of up to 32 tokens take this kernel: measured against the per-wave
// kernel on the Qwen3-8B-like and 27B-class layers (interleaved, bf16 out),
// 1.3-4.3x faster at M = 1-32 (down 4096 x 12288 at M = 1: 18 against 79
// us); from M = 64 the per-wave kernel's 64- or 128-row tiles, which read
// each weight once per 64 or 128 tokens, win on the wide and long layers.
constexpr int64_t kSmallMaxM = 32;

// kFuse: xcodes is X itself (bf16 [M, K]) and xscales is unused; each lane
// loads its two groups' 32 bf16 values of a step and encodes them whole
// (encode16_bf16, the quantizer's steps), with the tensor scale folded from
// partial[0 .. npartial) (block 0 stores it to *ts) or read from *ts.
template <int MT, int NTB, int WMAX, bool kBF16Out, bool kFuse = false>
__global__ __launch_bounds__(kSmallWaves * 64) void w4a4_small_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ blob, int64_t wc_off,
    int64_t ws_off, int M, int m0, int N, int K, void* __restrict__ y,
    const uint32_t* __restrict__ partial = nullptr, int npartial = 0,
    float* __restrict__ ts = nullptr) {
  if (!blob_matches(blob, 0, N, K)) return;   // before any barrier: uniform
  constexpr int NW = kSmallWaves;
  __shared__ float inv_tab[kFuse ? 128 : 1];
  float s_t = 0.0f, d6 = 0.0f;
  if constexpr (kFuse) {
    if (npartial > 0) {
      s_t = tensor_scale_from_partials<NW * 64>(partial, npartial);
      if (blockIdx.x == 0 && threadIdx.x == 0 && m0 == 0) *ts = s_t;
    } else {
      s_t = *ts;
    }
    d6 = 6.0f * s_t;
    fill_inv_table(inv_tab, s_t);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int r = lane & 15, q = lane >> 4;
  const int KT = K / 128;
  const int gpw = (KT + NW - 1) / NW;
  const int g0 = wave * gpw;
  const int nt0 = blockIdx.x * NTB;
  const int NT16 = N / 16;

  const uint8_t* wc[NTB];
  const uint8_t* wsc[NTB];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int64_t tile = min(nt0 + nt, NT16 - 1);
    wc[nt] = blob + wc_off + tile * KT * 1024 + r * 64 + q * 16;
    wsc[nt] = blob + ws_off + tile * KT * 128 + r * 8 + 2 * q;
  }
  const uint8_t* xc[MT];
  const uint8_t* xs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t row = min(m0 + mt * 16 + r, M - 1);   // rows past M: computed, not stored
    if constexpr (kFuse) {
      xc[mt] = xcodes + (row * K + q * 32) * 2;          // bf16 elements 32 q .. of a step
      xs[mt] = nullptr;
    } else {
      xc[mt] = xcodes + row * (K / 2) + q * 16;
      xs[mt] = xscales + row * (K / 16) + 2 * q;
    }
  }

  floatx4 acc[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < gpw; c0 += WMAX) {
    uint4 wv[WMAX][NTB], xv[WMAX][MT];
    uint32_t wsv[WMAX][NTB], xsv[WMAX][MT];
    uint4 xb[kFuse ? WMAX : 1][kFuse ? MT : 1][4];
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const int g = min(g0 + min(c0 + i, gpw - 1), KT - 1);
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        wv[i][nt] = load_nt16(wc[nt] + int64_t(g) * 1024);
        wsv[i][nt] = *reinterpret_cast<const uint16_t*>(wsc[nt] + int64_t(g) * 128);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (kFuse) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            xb[i][mt][u] = *reinterpret_cast<const uint4*>(xc[mt] + int64_t(g) * 256 + u * 16);
        } else {
          xv[i][mt] = *reinterpret_cast<const uint4*>(xc[mt] + int64_t(g) * 64);
          xsv[i][mt] = *reinterpret_cast<const uint16_t*>(xs[mt] + int64_t(g) * 8);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // the chunk's loads go out before its arithmetic
    if constexpr (kFuse) {
      // the lane's two groups (2q, 2q + 1) of each step, encoded whole
#pragma unroll
      for (int i = 0; i < WMAX; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          uint32_t c[4], s0, s1;
          encode16_bf16(xb[i][mt][0], xb[i][mt][1], d6, inv_tab, c[0], c[1], s0);
          encode16_bf16(xb[i][mt][2], xb[i][mt][3], d6, inv_tab, c[2], c[3], s1);
          xv[i][mt] = make_uint4(c[0], c[1], c[2], c[3]);
          xsv[i][mt] = s0 | (s1 << 8);
        }
    }
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      const bool live = c0 + i < gpw && g0 + c0 + i < KT;   // wave-uniform
#pragma unroll
      for (int d = 0; d < 4; ++d) {          // d = 2c + s: group 2q + c, half s
        half8_t xf[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          xf[mt] = dequant8(dword(xv[i][mt], d), scale2(xsv[i][mt], d >> 1));
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt) {
          const half8_t wf = dequant8(dword(wv[i][nt], d), scale2(live ? wsv[i][nt] : 0u, d >> 1));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf[mt], acc[nt][mt], 0, 0, 0);
        }
      }
    }
  }

  // partial sums of the waves -> LDS; sum in wave order, scale, store
  __shared__ floatx4 red[NW][NTB][MT][64];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][nt][mt][lane] = acc[nt][mt];
  __syncthreads();
  const float st = (kFuse ? s_t : a_ts[0]) * reinterpret_cast<const BlobHeader*>(blob)->tensor_scale;
  for (int t = threadIdx.x; t < NTB * MT * 64; t += NW * 64) {
    const int nt = t / (MT * 64), mt = (t / 64) % MT, ln = t % 64;
    floatx4 v = red[0][nt][mt][ln];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][nt][mt][ln];
    v = v * st;
    const int n = (nt0 + nt) * 16 + 4 * (ln >> 4);
    const int m = m0 + mt * 16 + (ln & 15);
    if (m < M && n < N) {
      if (kBF16Out) {
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + int64_t(m) * N + n) = o;
      } else {
        *reinterpret_cast<floatx4*>(static_cast<float*>(y) + int64_t(m) * N + n) = v;
      }
    }
  }
}

template <int MT, int NTB, bool kFuse = false>
hipError_t launch_small_pass(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                             const uint8_t* blob, const BlobLayout& L, int M, int m0, int N,
                             int K, void* y, int y_dtype, hipStream_t s,
                             const uint32_t* partial = nullptr, int npartial = 0,
                             float* ts = nullptr) {
  constexpr int WMAX = kFuse ? 2 : 4;   // the bf16 rows of a chunk take 4x the registers of codes
  const int blocks = (N / 16 + NTB - 1) / NTB;
  if (y_dtype == 1)
    w4a4_small_kernel<MT, NTB, WMAX, true, kFuse><<<blocks, kSmallWaves * 64, 0, s>>>(
        a_codes, a_scales, a_ts, blob, L.codes_off, L.aux_off, M, m0, N, K, y, partial, npartial,
        ts);
  else
    w4a4_small_kernel<MT, NTB, WMAX, false, kFuse><<<blocks, kSmallWaves * 64, 0, s>>>(
        a_codes, a_scales, a_ts, blob, L.codes_off, L.aux_off, M, m0, N, K, y, partial, npartial,
        ts);
  return hipGetLastError();
}

// passes of up to 32 tokens (two m-tiles), two row tiles per block when that
// still leaves at least 192 blocks
template <bool kFuse = false>
hipError_t launch_small_all(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                            const uint8_t* blob, const BlobLayout& L, int64_t m, int64_t n,
                            int64_t k, void* y, int y_dtype, hipStream_t s,
                            const uint32_t* partial = nullptr, int npartial = 0,
                            float* ts = nullptr) {
  const bool wide = n / 16 >= 384;
  for (int64_t m0 = 0; m0 < m; m0 += 32) {
    const int rows = int(m - m0 < 32 ? m - m0 : 32);
    const int M = int(m), M0 = int(m0), N = int(n), K = int(k);
    hipError_t e;
#define QL_SMALL(MT, NTB)                                                                    \
  launch_small_pass<MT, NTB, kFuse>(a_codes, a_scales, a_ts, blob, L, M, M0, N, K, y, y_dtype, \
                                    s, partial, npartial, ts)
    if (rows <= 16)
      e = wide ? QL_SMALL(1, 2) : QL_SMALL(1, 1);
    else
      e = wide ? QL_SMALL(2, 2) : QL_SMALL(2, 1);
#undef QL_SMALL
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int WN, int WM, bool kFuse = false>
hipError_t launch_tile(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                       const uint8_t* blob, const BlobLayout& L, int64_t m, int64_t n,
                       int64_t k, void* y, int y_dtype, hipStream_t s,
                       const uint32_t* partial = nullptr, int npartial = 0,
                       float* ts = nullptr) {
  constexpr int BN = 32 * WN, BM = 32 * WM;
  const int tiles = static_cast<int>(((m + BM - 1) / BM) * ((n + BN - 1) / BN));
  if (y_dtype == 1)
    w4a4_kernel<WN, WM, true, kFuse><<<tiles, kThreads, 0, s>>>(
        a_codes, a_scales, a_ts, blob, L.codes_off, L.aux_off, int(m), int(n), int(k), y,
        partial, npartial, ts);
  else
    w4a4_kernel<WN, WM, false, kFuse><<<tiles, kThreads, 0, s>>>(
        a_codes, a_scales, a_ts, blob, L.codes_off, L.aux_off, int(m), int(n), int(k), y,
        partial, npartial, ts);
  return hipGetLastError();
}

}  // namespace

namespace {

// The block-cooperative 256x256 kernel holds one block per CU (its LDS double
// buffer is 160 KiB).  It runs every problem of more than half a round of
// 256x256 tiles (more than CUs / 2 tiles) with m > 128; a problem of at most half a round
// runs on it only when the caller's workspace lets its tiles be split along k
// over the CUs, and otherwise takes the 128x128 per-wave kernel, which
// spreads 4x more blocks.  Measured on Qwen3-8B-like and 27B-class shapes at
// M = 512-3072: 129-255 tiles on the cooperative kernel run 1.21-1.45x the
// per-wave kernel's speed; the split of a small problem 1.00-2.18x (most on
// long k).  The kernel addresses activation and weight codes with 31-bit
// buffer offsets.
bool coop_fits(int64_t m, int64_t n, int64_t k) {
  const int64_t lim = (int64_t(1) << 31) - (int64_t(1) << 20);
  const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
  return m * (k / 2) <= lim && n * (k / 2) <= lim && big_tiles < (int64_t(1) << 30);
}

// At m <= 128 half of each 256-row tile would be idle MFMA work: the
// per-wave kernel's 128-row tiles measured 1.24-1.54x faster there (n =
// 40960-151936, k = 4096, bit-identical outputs); at m = 160-256 the
// cooperative kernel stays ahead (the per-wave kernel ran 0.71-0.83x).
bool use_coop(int64_t m, int64_t n, int64_t k) {
  const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
  const int cus = device_cu_count();
  return m > 128 && (cus > 0 ? big_tiles * 2 > cus : big_tiles >= 256) && coop_fits(m, n, k);
}

// A problem of at most half a round is k-split only where that beats the
// per-wave kernel: not at m <= 128 (half of each 256-row tile would be idle
// MFMA work) unless k is long.  Measured over the Qwen3-8B-like and 27B-class
// shapes at m = 128-2048: the split ran 0.80-0.99x at m = 128 with k <= 5120,
// 1.47-1.58x there with k >= 12288, and 0.93-1.99x (mostly > 1) at m >= 256.
// Batches the small-batch kernel takes are never split: it ran 2.9-3.7x the
// per-wave kernel on down 4096 x 12288 at M = 16-32, the split at most 1.6x.
bool split_pays(int64_t m, int64_t n, int64_t k) {
  if (m <= kSmallMaxM) return false;
  const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
  const int cus = device_cu_count();
  if (cus > 0 && big_tiles * 2 <= cus) return m > 128 || k >= 8192;
  return m > 128;   // larger problems at m <= 128 take the per-wave kernel
}

size_t split_bytes(int64_t m, int64_t n, int64_t k) {
  if (!coop_fits(m, n, k) || !split_pays(m, n, k)) return 0;
  return coop_split_bytes(coop_split_plan(m, n, k));
}

}  // namespace

size_t gemm_w4a4_ws_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  return split_bytes(m, n, k);
}

hipError_t launch_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                            const void* w_packed, int64_t m, int64_t n, int64_t k, void* y,
                            int y_dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  const BlobLayout L = blob_layout(0, n, k);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  const size_t need = split_bytes(m, n, k);
  const bool split = need > 0 && ws != nullptr && ws_bytes >= need;
  if (split || use_coop(m, n, k))
    return launch_gemm_w4a4_coop(a_codes, a_scales, a_ts, w_packed, m, n, k, y, y_dtype,
                                 static_cast<float*>(ws), split, s);
  if (m <= kSmallMaxM)
    return launch_small_all(a_codes, a_scales, a_ts, blob, L, m, n, k, y, y_dtype, s);
  // With fewer 128x128 tiles than CUs, 64x64 tiles (4x the blocks) fill the
  // chip better despite twice the dequantization per product: 1.07-1.87x at
  // M = 64-512 on the Qwen3-8B-like shapes (outputs bit-identical: every
  // output's k order is the same).
  const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
  const int cus = device_cu_count();
  if (cus > 0 && t128 < cus)
    return launch_tile<2, 2>(a_codes, a_scales, a_ts, blob, L, m, n, k, y, y_dtype, s);
  return launch_tile<4, 4>(a_codes, a_scales, a_ts, blob, L, m, n, k, y, y_dtype, s);
}

// Quantize folded into the GEMM: the amax pass (unless the scale is static),
// then the small-batch kernel (m <= 32) or the per-wave kernel quantizing the
// activation as they load it, with the kernel and tile size launch_gemm_w4a4
// gives that batch without a workspace (so results match it bit for bit).
hipError_t launch_quantize_gemm_w4a4(const void* x_bf16, int64_t m, int64_t k, float* ts,
                                     bool static_scale, uint32_t* partial, const void* w_packed,
                                     int64_t n, void* y, int y_dtype, hipStream_t s) {
  const BlobLayout L = blob_layout(0, n, k);
  const uint8_t* blob = static_cast<const uint8_t*>(w_packed);
  int npart = 0;
  if (!static_scale) {
    hipError_t e = launch_amax_bf16(x_bf16, m, k, partial, &npart, s);
    if (e != hipSuccess) return e;
  }
  const uint8_t* xb = static_cast<const uint8_t*>(x_bf16);
  if (m <= kSmallMaxM)
    return launch_small_all<true>(xb, nullptr, nullptr, blob, L, m, n, k, y, y_dtype, s, partial,
                                  npart, ts);
  const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
  const int cus = device_cu_count();
  if (cus > 0 && t128 < cus)
    return launch_tile<2, 2, true>(xb, nullptr, nullptr, blob, L, m, n, k, y, y_dtype, s, partial,
                                   npart, ts);
  return launch_tile<4, 4, true>(xb, nullptr, nullptr, blob, L, m, n, k, y, y_dtype, s, partial,
                                 npart, ts);
}

}  // namespace qlin
