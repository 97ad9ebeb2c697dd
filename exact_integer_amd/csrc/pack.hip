// Weight repack: canonical [n][k] codes and [n][k/32] scales into MFMA tiles.
//
// A row group is 32 rows; a block is 32 columns.  Tile (rg, b) is 1 KB in the
// lane order of the gfx950 32x32x32 int8 MFMA operand: lane l holds row
// rg*32 + l%32 and columns b*32 + 16*(l/32) .. +15, 16 contiguous bytes.  The
// same tile feeds the GEMV (one 16-byte load per lane) and the MFMA B operand
// (one 16-byte load per lane, no shuffles).  Scales follow as
// [n_pad/32][nb][32] int32, then the row offsets [n_pad] int64 (4-bit images;
// zero in Q8 images).  Rows beyond n are zero (zero codes, zero scales),
// so padded rows contribute nothing and are never written back.
#include "ei_internal.h"

namespace ei {

// One thread per (row group, block, lane): 16 code bytes.
__global__ void pack_q8_codes_kernel(const int8_t* __restrict__ codes, int64_t n, int64_t k, int64_t nb,
                                     int64_t n_pad, int8_t* __restrict__ tiles) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (n_pad / kTile) * nb * 64;
  if (gid >= total) return;
  int lane = (int)(gid % 64);
  int64_t tile = gid / 64;              // rg * nb + b
  int64_t b = tile % nb, rg = tile / nb;
  int64_t row = rg * kTile + lane % 32;
  int64_t col = b * 32 + 16 * (lane / 32);
  v4i v = {0, 0, 0, 0};
  if (row < n) {
    const int8_t* src = codes + row * k + col;   // 16-byte aligned when codes is and k % 32 == 0
    v = *reinterpret_cast<const v4i*>(src);
  }
  *reinterpret_cast<v4i*>(tiles + gid * 16) = v;
}

// One thread per (row group, block, row-in-group): one scale; also the max |S|.
__global__ void pack_q8_scales_kernel(const int32_t* __restrict__ scales, int64_t n, int64_t nb, int64_t n_pad,
                                      int32_t* __restrict__ out, uint32_t* __restrict__ smax) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (n_pad / kTile) * nb * 32;
  if (gid >= total) return;
  int r = (int)(gid % 32);
  int64_t tile = gid / 32;
  int64_t b = tile % nb, rg = tile / nb;
  int64_t row = rg * kTile + r;
  int32_t s = row < n ? scales[row * nb + b] : 0;
  out[gid] = s;
  uint32_t mag = s < 0 ? (uint32_t)0 - (uint32_t)s : (uint32_t)s;
  // integer max is order-independent
  atomicMax(smax, mag);
}

// 4-bit codes: nibble j of row i is (nib[i][j/2] >> 4*(j&1)) & 15, two's
// complement; the block's mantissa m (low nibble of the scale byte) is folded
// in, giving m*q in [-120, 105].
__global__ void pack_q4_codes_kernel(const uint8_t* __restrict__ nib, const uint8_t* __restrict__ sme, int64_t n,
                                     int64_t k, int64_t nb, int64_t n_pad, int8_t* __restrict__ tiles) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (n_pad / kTile) * nb * 64;
  if (gid >= total) return;
  int lane = (int)(gid % 64);
  int64_t tile = gid / 64;
  int64_t b = tile % nb, rg = tile / nb;
  int64_t row = rg * kTile + lane % 32;
  int64_t col = b * 32 + 16 * (lane / 32);
  int8_t out[16];
  if (row < n) {
    int m = sme[row * nb + b] & 15;
    const uint8_t* src = nib + row * (k / 2) + col / 2;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      int byte = src[p];
      int lo = byte & 15, hi = byte >> 4;
      lo = lo >= 8 ? lo - 16 : lo;
      hi = hi >= 8 ? hi - 16 : hi;
      out[2 * p] = (int8_t)(m * lo);
      out[2 * p + 1] = (int8_t)(m * hi);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = 0;
  }
  v4i v;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    v[w] = (int)((uint32_t)(uint8_t)out[4 * w] | ((uint32_t)(uint8_t)out[4 * w + 1] << 8) |
                 ((uint32_t)(uint8_t)out[4 * w + 2] << 16) | ((uint32_t)(uint8_t)out[4 * w + 3] << 24));
  *reinterpret_cast<v4i*>(tiles + gid * 16) = v;
}

// The scale of a 4-bit block is m * 2^e; m went into the codes, 2^e stays.
__global__ void pack_q4_scales_kernel(const uint8_t* __restrict__ sme, int64_t n, int64_t nb, int64_t n_pad,
                                      int32_t* __restrict__ out, uint32_t* __restrict__ smax) {
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (n_pad / kTile) * nb * 32;
  if (gid >= total) return;
  int r = (int)(gid % 32);
  int64_t tile = gid / 32;
  int64_t b = tile % nb, rg = tile / nb;
  int64_t row = rg * kTile + r;
  int32_t s = row < n ? (int32_t)(1u << (sme[row * nb + b] >> 4)) : 0;
  out[gid] = s;
  atomicMax(smax, (uint32_t)s);
}

// Row offsets of a 4-bit image, one thread per row: R_i = 128 * sum_j m 2^e q
// (the row's weight sum times kQ4Offset; |R_i| < 2^47 for k <= 262,144).
// The two-limb form adds R_i back after splitting x - 128.  Rows >= n get 0.
__global__ void pack_q4_row_offsets_kernel(const uint8_t* __restrict__ nib, const uint8_t* __restrict__ sme,
                                           int64_t n, int64_t k, int64_t nb, int64_t n_pad,
                                           int64_t* __restrict__ roff) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n_pad) return;
  int64_t sum = 0;
  if (row < n) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* src = nib + row * (k / 2) + b * 16;
      int g = 0;   // sum of the block's 32 codes, |g| <= 256
      for (int p = 0; p < 16; ++p) {
        const int lo = src[p] & 15, hi = src[p] >> 4;
        g += (lo >= 8 ? lo - 16 : lo) + (hi >= 8 ? hi - 16 : hi);
      }
      const int sc = sme[row * nb + b];
      sum += (int64_t)((sc & 15) * g) << (sc >> 4);
    }
  }
  roff[row] = kQ4Offset * sum;
}

// Q8 images carry the row-offset area too (one layout for both formats): zeros.
__global__ void zero_i64_kernel(int64_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void pack_header_kernel(PackedHeader* h, int32_t format, int64_t n, int64_t k, int64_t n_pad, int64_t nb) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  h->magic = kMagic;
  h->format = format;
  h->n = n;
  h->k = k;
  h->n_pad = n_pad;
  h->nb = nb;
  h->smax = 0;
  h->pad0 = 0;
  h->codes_off = kHeaderBytes;
  h->scales_off = kHeaderBytes + n_pad * k;
  h->roff_off = (int64_t)row_offsets_at(n_pad, k);
}

static hipError_t launch_pack(int format, const void* codes, const void* scales, int64_t n, int64_t k,
                              void* packed, hipStream_t s) {
  const int64_t nb = k / 32, n_pad = round_up(n, kTile);
  PackedHeader* h = static_cast<PackedHeader*>(packed);
  int8_t* tiles = static_cast<int8_t*>(packed) + kHeaderBytes;
  int32_t* sc = reinterpret_cast<int32_t*>(tiles + n_pad * k);
  int64_t* roff = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(packed) + row_offsets_at(n_pad, k));
  const unsigned g3 = (unsigned)((n_pad + 255) / 256);
  hipLaunchKernelGGL(pack_header_kernel, dim3(1), dim3(64), 0, s, h, format, n, k, n_pad, nb);
  const int64_t ncode = (n_pad / kTile) * nb * 64, nsc = (n_pad / kTile) * nb * 32;
  const unsigned g1 = (unsigned)((ncode + 255) / 256), g2 = (unsigned)((nsc + 255) / 256);
  if (format == EI_FORMAT_Q8) {
    hipLaunchKernelGGL(pack_q8_codes_kernel, dim3(g1), dim3(256), 0, s, static_cast<const int8_t*>(codes), n, k,
                       nb, n_pad, tiles);
    hipLaunchKernelGGL(pack_q8_scales_kernel, dim3(g2), dim3(256), 0, s, static_cast<const int32_t*>(scales), n, nb,
                       n_pad, sc, &h->smax);
    hipLaunchKernelGGL(zero_i64_kernel, dim3(g3), dim3(256), 0, s, roff, n_pad);
  } else {
    hipLaunchKernelGGL(pack_q4_codes_kernel, dim3(g1), dim3(256), 0, s, static_cast<const uint8_t*>(codes),
                       static_cast<const uint8_t*>(scales), n, k, nb, n_pad, tiles);
    hipLaunchKernelGGL(pack_q4_scales_kernel, dim3(g2), dim3(256), 0, s, static_cast<const uint8_t*>(scales), n, nb,
                       n_pad, sc, &h->smax);
    hipLaunchKernelGGL(pack_q4_row_offsets_kernel, dim3(g3), dim3(256), 0, s, static_cast<const uint8_t*>(codes),
                       static_cast<const uint8_t*>(scales), n, k, nb, n_pad, roff);
  }
  return hipGetLastError();
}

hipError_t launch_pack_q8(const int8_t* codes, const int32_t* scales, int64_t n, int64_t k, void* packed,
                          hipStream_t s) {
  return launch_pack(EI_FORMAT_Q8, codes, scales, n, k, packed, s);
}

hipError_t launch_pack_q4(const uint8_t* nib, const uint8_t* sme, int64_t n, int64_t k, void* packed,
                          hipStream_t s) {
  return launch_pack(EI_FORMAT_Q4, nib, sme, n, k, packed, s);
}

}  // namespace ei
