// Offline weight repack into the gfx950 operand order read by the GEMMs.
//
// The MARLIN article (abeam.tech, section "重みレイアウトの工夫" / "オフライン
// で並べ替えておく") reorders quantized weights and their group scales once,
// offline, so the kernel reads them with regular, wide accesses.  The same
// idea is applied here to the three formats, with layouts chosen for the
// 64-lane wavefront and the 16x16x32 MFMA of gfx950.  Values are only moved,
// never changed.  Every region starts 256-byte aligned after a 256-byte
// header (magic, version, format, n, k, NVFP4 tensor scale).
//
// Notation: nt = n/16 row tile, ks = k/128 column step, l = lane (0..63),
// r = l % 16 (row inside the tile), q = l / 16 (lane group).
//
// NVFP4 (W4A4 prefill):
//   codes  [nt][ks][16 rows][64 B]  the canonical bytes of 16 rows x 128 k
//   scales [nt][ks][16 rows][8 B]   the 8 E4M3 group scales of those k
// INT4 group-128 (W4A16 decode):
//   codes  [nt][ks][64 lanes][16 B] lane l, dword s (0..3) holds row r and
//          k = 128 ks + 32 s + 8 q + t, t = 0..7, with nibble t = 2j at bits
//          4j and t = 2j+1 at bits 16+4j (so OR-ing 0x4300 into each 16-bit
//          half yields the bf16 value 128 + u of two neighbours at once)
//   scales [nt][ks][16 rows] bf16
// 2:4 sparse INT4 group-128 (Sparse-MARLIN reading, W4A16 decode on the
// gfx950 2:4 sparse MFMA v_smfmac_f32_16x16x64_bf16):
//   codes  [nt][ks][64 lanes][12 B]: dwords 0 and 1 are the kept codes,
//          dword s (0, 1) covering k = 128 ks + 64 s + 16 (2 (q % 2) + h) +
//          8 (q / 2) + 4 b + p for quads g = 2 h + b (h, b in {0, 1}) and
//          p = 0..3; element 2g holds the code at the lower kept position p0
//          of quad g, element 2g+1 the one at p1, with element e at bits
//          4 (e/2) (e even) or 16 + 4 (e/2) (e odd).  Dword 2 holds the kept
//          positions: p of element e of half s at bits 16 s + 2 e (the sparse
//          MFMA's index operand).  One 12-byte load per lane and group.
//   scales [nt][ks][16 rows] bf16
//   Kept per quad: the two codes of largest |q| (ties to the lower column),
//   i.e. every nonzero code when the codes come from the 2:4 quantizer.
// LUT2 (2-bit codebook decode):
//   codes  [nt][ks][64 lanes][8 B]  dword d holds sub-steps s = 2d, 2d+1;
//          index of (s, t) at bit 8 (t % 4) + 2 (2 (s % 2) + t / 4), so that
//          (dword >> 2j) & 0x03030303 yields four indices, one per byte
//   book   [n][8 B]  low bytes of the 4 bf16 centroids, then their high bytes
#include "qlin_internal.hpp"

namespace qlin {
namespace {

__global__ void header_kernel(void* packed, int fmt, int64_t n, int64_t k,
                              const float* __restrict__ tensor_scale) {
  if (threadIdx.x == 0) {
    BlobHeader* h = static_cast<BlobHeader*>(packed);
    h->magic = kBlobMagic;
    h->version = kBlobVersion;
    h->fmt = fmt;
    h->reserved = 0;
    h->n = n;
    h->k = k;
    h->tensor_scale = tensor_scale ? *tensor_scale : 0.0f;
  }
}

// NVFP4 codes: one thread per 16-byte unit of the blob.
__global__ void repack_nvfp4_codes(const uint8_t* __restrict__ codes, int64_t n, int64_t k,
                                   uint8_t* __restrict__ out) {
  const int64_t units = n * k / 32;
  const int64_t KT = k / 128;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * blockDim.x) {
    const int64_t tile = u / 64, within = u % 64;
    const int64_t nt = tile / KT, ks = tile % KT;
    const int64_t r = within / 4, b16 = within % 4;
    const uint4* src = reinterpret_cast<const uint4*>(codes + (nt * 16 + r) * (k / 2) + ks * 64 +
                                                      b16 * 16);
    reinterpret_cast<uint4*>(out)[u] = *src;
  }
}

// NVFP4 scales: one thread per 8-byte (row, step) unit; read bytewise since
// the canonical scale array is only byte-aligned in general.
__global__ void repack_nvfp4_scales(const uint8_t* __restrict__ scales, int64_t n, int64_t k,
                                    uint8_t* __restrict__ out) {
  const int64_t units = n * k / 128;
  const int64_t KT = k / 128;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * blockDim.x) {
    const int64_t tile = u / 16, r = u % 16;
    const int64_t nt = tile / KT, ks = tile % KT;
    const uint8_t* src = scales + (nt * 16 + r) * (k / 16) + ks * 8;
#pragma unroll
    for (int b = 0; b < 8; ++b) out[u * 8 + b] = src[b];
  }
}

// INT4 codes: one thread per output dword (lane l, sub-step s).
__global__ void repack_int4_codes(const uint8_t* __restrict__ codes, int64_t n, int64_t k,
                                  uint32_t* __restrict__ out) {
  const int64_t units = n * k / 8;
  const int64_t KT = k / 128;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * blockDim.x) {
    const int64_t s = u % 4, l = (u / 4) % 64, tile = u / 256;
    const int64_t nt = tile / KT, ks = tile % KT;
    const int64_t row = nt * 16 + (l % 16);
    const int64_t k0 = ks * 128 + 32 * s + 8 * (l / 16);
    const uint8_t* src = codes + row * (k / 2) + k0 / 2;
    uint32_t v = uint32_t(src[0]) | (uint32_t(src[1]) << 8) | (uint32_t(src[2]) << 16) |
                 (uint32_t(src[3]) << 24);  // nibble t at bits 4t
    uint32_t o = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o |= ((v >> (8 * j)) & 0xFu) << (4 * j);             // t = 2j
      o |= ((v >> (8 * j + 4)) & 0xFu) << (16 + 4 * j);    // t = 2j + 1
    }
    out[u] = o;
  }
}

__global__ void repack_int4_scales(const uint16_t* __restrict__ scales, int64_t n, int64_t k,
                                   uint16_t* __restrict__ out) {
  const int64_t units = n * (k / 128);
  const int64_t KT = k / 128;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = u % 16, tile = u / 16;
    const int64_t nt = tile / KT, ks = tile % KT;
    out[u] = scales[(nt * 16 + r) * KT + ks];
  }
}

// LUT2 indices: one thread per output dword (lane l, dword d).
__global__ void repack_lut2_codes(const uint8_t* __restrict__ idx, int64_t n, int64_t k,
                                  uint32_t* __restrict__ out) {
  const int64_t units = n * k / 16;
  const int64_t KT = k / 128;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * blockDim.x) {
    const int64_t d = u % 2, l = (u / 2) % 64, tile = u / 128;
    const int64_t nt = tile / KT, ks = tile % KT;
    const int64_t row = nt * 16 + (l % 16);
    uint32_t o = 0;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int64_t s = 2 * d + sl;
      const int64_t k0 = ks * 128 + 32 * s + 8 * (l / 16);
      const uint8_t* src = idx + row * (k / 4) + k0 / 4;
      const uint32_t v = uint32_t(src[0]) | (uint32_t(src[1]) << 8);  // index t at bits 2t
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t ix = (v >> (2 * t)) & 3u;
        o |= ix << (8 * (t % 4) + 2 * (2 * sl + t / 4));
      }
    }
    out[u] = o;
  }
}

__global__ void repack_lut2_book(const uint16_t* __restrict__ cent, int64_t n,
                                 uint32_t* __restrict__ out) {
  for (int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; r < n;
       r += int64_t(gridDim.x) * blockDim.x) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c = cent[r * 4 + j];
      lo |= (c & 0xFFu) << (8 * j);
      hi |= (c >> 8) << (8 * j);
    }
    out[2 * r] = lo;
    out[2 * r + 1] = hi;
  }
}

// 2:4 INT4: one thread per (lane, 128-k step) writes its 8 code bytes and
// its 4 position bytes.
__global__ void repack_sp24(const uint8_t* __restrict__ codes, int64_t n, int64_t k,
                            uint32_t* __restrict__ out) {
  const int64_t units = n * k / 32;
  const int64_t KT = k / 128;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += int64_t(gridDim.x) * blockDim.x) {
    const int64_t l = u % 64, tile = u / 64;
    const int64_t nt = tile / KT, ks = tile % KT;
    const int64_t row = nt * 16 + (l % 16), qa = l / 16;
    uint32_t cw[2] = {0u, 0u}, meta = 0u;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t kb = ks * 128 + 64 * s + 16 * (2 * (qa & 1) + (g >> 1)) + 8 * (qa >> 1) +
                           4 * (g & 1);
        const uint8_t* src = codes + row * (k / 2) + kb / 2;
        const uint32_t uq[4] = {uint32_t(src[0] & 15u), uint32_t(src[0] >> 4),
                                uint32_t(src[1] & 15u), uint32_t(src[1] >> 4)};
        int pos[2] = {0, 1}, nk = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ac = int(uq[c]) - 8 < 0 ? 8 - int(uq[c]) : int(uq[c]) - 8;
          int beaten = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ae = int(uq[e]) - 8 < 0 ? 8 - int(uq[e]) : int(uq[e]) - 8;
            beaten += (ae > ac || (ae == ac && e < c)) ? 1 : 0;
          }
          if (beaten < 2 && nk < 2) pos[nk++] = c;
        }
        cw[s] |= (uq[pos[0]] << (4 * g)) | (uq[pos[1]] << (16 + 4 * g));
        meta |= (uint32_t(pos[0]) << (16 * s + 4 * g)) | (uint32_t(pos[1]) << (16 * s + 4 * g + 2));
      }
    out[3 * u] = cw[0];
    out[3 * u + 1] = cw[1];
    out[3 * u + 2] = meta;
  }
}

int grid_for(int64_t units) {
  int64_t b = (units + 255) / 256;
  if (b > 65536) b = 65536;
  return b < 1 ? 1 : static_cast<int>(b);
}

}  // namespace

hipError_t launch_repack(int fmt, int64_t n, int64_t k, const uint8_t* codes, const void* aux,
                         const float* tensor_scale, void* packed, hipStream_t s) {
  const BlobLayout L = blob_layout(fmt, n, k);
  uint8_t* base = static_cast<uint8_t*>(packed);
  header_kernel<<<1, 64, 0, s>>>(packed, fmt, n, k, fmt == 0 ? tensor_scale : nullptr);
  if (fmt == 0) {
    repack_nvfp4_codes<<<grid_for(n * k / 32), 256, 0, s>>>(codes, n, k, base + L.codes_off);
    repack_nvfp4_scales<<<grid_for(n * k / 128), 256, 0, s>>>(
        static_cast<const uint8_t*>(aux), n, k, base + L.aux_off);
  } else if (fmt == 1 || fmt == 3) {
    if (fmt == 1)
      repack_int4_codes<<<grid_for(n * k / 8), 256, 0, s>>>(
          codes, n, k, reinterpret_cast<uint32_t*>(base + L.codes_off));
    else
      repack_sp24<<<grid_for(n * k / 32), 256, 0, s>>>(
          codes, n, k, reinterpret_cast<uint32_t*>(base + L.codes_off));
    repack_int4_scales<<<grid_for(n * (k / 128)), 256, 0, s>>>(
        static_cast<const uint16_t*>(aux), n, k, reinterpret_cast<uint16_t*>(base + L.aux_off));
  } else {
    repack_lut2_codes<<<grid_for(n * k / 16), 256, 0, s>>>(
        codes, n, k, reinterpret_cast<uint32_t*>(base + L.codes_off));
    repack_lut2_book<<<grid_for(n), 256, 0, s>>>(static_cast<const uint16_t*>(aux), n,
                                                 reinterpret_cast<uint32_t*>(base + L.aux_off));
  }
  return hipGetLastError();
}

}  // namespace qlin
