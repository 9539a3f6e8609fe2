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
// Two kernels share this arithmetic.  Problems with at least 256 tiles of
// 256 x 256 go to the block-cooperative kernel (gemm_w4a4_coop.hip), which
// dequantizes each code once per block into fp16 LDS tiles.  Smaller problems
// use the per-wave kernel below, whose 4x smaller tiles keep every CU busy.
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
#include "qlin_internal.hpp"

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
template <int WN, int WM, bool kBF16Out>
__global__ __launch_bounds__(kThreads) void w4a4_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ blob, int64_t wc_off,
    int64_t ws_off, int M, int N, int K, void* __restrict__ y) {
  if (!blob_matches(blob, 0, N, K)) return;
  constexpr int BN = 32 * WN, BM = 32 * WM;
  constexpr int WU = BN * 4 / kThreads;   // 16-byte W code units per thread per stage
  constexpr int XU = BM * 4 / kThreads;   // 16-byte X code units per thread per stage
  constexpr int SU = (BN + BM + kThreads - 1) / kThreads;  // 8-byte scale rows per thread
  __shared__ __attribute__((aligned(16))) uint8_t wc_s[2][BN * RS];
  __shared__ __attribute__((aligned(16))) uint8_t xc_s[2][BM * RS];
  __shared__ __attribute__((aligned(16))) uint8_t sc_s[2][(BN + BM) * 8];

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

  uint4 pw[WU], px[XU];
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
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = i * kThreads + tid;
      const int m = m0 + (u >> 2);
      px[i] = m < M ? *reinterpret_cast<const uint4*>(xcodes + int64_t(m) * (K / 2) + ks * 64 +
                                                      (u & 3) * 16)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int r = i * kThreads + tid;   // 0 .. BN+BM-1; W rows first
      if (r >= BN + BM) {
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
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = i * kThreads + tid;
      *reinterpret_cast<uint4*>(&xc_s[buf][(u >> 2) * RS + (u & 3) * 16]) = px[i];
    }
#pragma unroll
    for (int i = 0; i < SU; ++i)
      if (i * kThreads + tid < BN + BM)
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

  // epilogue: scale by s_tA * s_tW and store 4 consecutive n per lane
  const float st = a_ts[0] * reinterpret_cast<const BlobHeader*>(blob)->tensor_scale;
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    const int n = n0 + wn * (BN / 2) + i * 16 + 4 * q;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int m = m0 + wm * (BM / 2) + j * 16 + r;
      if (m >= M) continue;
      const floatx4 v = acc[i][j] * st;
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

template <int WN, int WM>
hipError_t launch_tile(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                       const uint8_t* blob, const BlobLayout& L, int64_t m, int64_t n,
                       int64_t k, void* y, int y_dtype, hipStream_t s) {
  constexpr int BN = 32 * WN, BM = 32 * WM;
  const int tiles = static_cast<int>(((m + BM - 1) / BM) * ((n + BN - 1) / BN));
  if (y_dtype == 1)
    w4a4_kernel<WN, WM, true><<<tiles, kThreads, 0, s>>>(a_codes, a_scales, a_ts, blob,
                                                          L.codes_off, L.aux_off, int(m), int(n),
                                                          int(k), y);
  else
    w4a4_kernel<WN, WM, false><<<tiles, kThreads, 0, s>>>(a_codes, a_scales, a_ts, blob,
                                                           L.codes_off, L.aux_off, int(m), int(n),
                                                           int(k), y);
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
bool split_pays(int64_t m, int64_t n, int64_t k) {
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

}  // namespace qlin
