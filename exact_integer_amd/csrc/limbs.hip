// Activation limb split (the quantiser in front of the int8 contraction).
//
// An integer activation x is written as balanced base-256 digits
// d_l in [-128, 127], x = sum_{l<L} 256^l d_l.  The digit set is a complete
// residue system mod 256, so the digits are unique: d_0 = ((x + 128) mod 256)
// - 128, then x <- (x - d_0) / 256 (exact), and so on.  After L digits the
// remainder must be zero, otherwise x is outside the L-limb range and the
// device status gets EI_DEV_LIMB_RANGE.  With the digits, the contraction
// sum_j q_j x_j becomes L int8 x int8 contractions whose int32 block sums
// are exact (|sum over 32| <= 32 * 128 * 128 < 2^19).
#include "ei_internal.h"

namespace ei {

// L <= 4: one thread per 4 consecutive values, digits packed with limb_words.
template <int L>
__global__ void limb_split4_kernel(const int64_t* __restrict__ x, int8_t* __restrict__ d, int64_t n,
                                   int32_t* status) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 >= n) return;
  int64_t v[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) v[p] = i0 + p < n ? x[i0 + p] : 0;
  uint32_t w[L];
  if (!limb_words<L>(v, w)) flag(status, EI_DEV_LIMB_RANGE);
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (i0 + p < n) d[(int64_t)l * n + i0 + p] = (int8_t)(uint8_t)(w[l] >> (8 * p));
}

// Any L in 1..8, one value per thread.
__global__ void limb_split_flat_kernel(const int64_t* __restrict__ x, int8_t* __restrict__ d, int64_t n, int limbs,
                                       int32_t* status) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t r = (uint64_t)x[i];
  for (int l = 0; l < limbs; ++l) {
    int dl = (int)((r + 128u) & 255u) - 128;
    d[(int64_t)l * n + i] = (int8_t)dl;
    r = (uint64_t)(((int64_t)(r - (uint64_t)(int64_t)dl)) >> 8);
  }
  if (r != 0) flag(status, EI_DEV_LIMB_RANGE);
}

// One thread per (token group tg, block b, tile lane): lane = t % 32 + 32 h
// takes the 16 activations of token 32 tg + t % 32, half h of block b, into
// 16 bytes of each of the L limb tiles (l, tg, b).  Consecutive threads write
// consecutive 16-byte pieces of a tile; each reads one 128-byte (int64) or
// 64-byte (int32) run of x.
// x_off is subtracted from every activation first (the two-limb 4-bit form).
template <int L, typename XT>
__global__ void limb_tiles_kernel(const XT* __restrict__ x, int64_t t, int64_t k, int8_t* __restrict__ tiles,
                                  int64_t t_pad, int32_t* status, int64_t x_off) {
  const int64_t nb = k / 32;
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= t_pad * nb * 2) return;
  const int lane = (int)(gid & 63);
  const int h = lane >> 5;
  const int64_t b = (gid >> 6) % nb;
  const int64_t tg = (gid >> 6) / nb;
  const int64_t tok = tg * kTile + (lane & 31);
  uint32_t words[L][4];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int w = 0; w < 4; ++w) words[l][w] = 0;
  bool ok = true;
  if (sizeof(XT) != 4) x_off = 0;   // the offset is for int32 (4-bit form) activations only
  if (tok < t) {
    const XT* src = x + tok * k + b * 32 + 16 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t v[4] = {(int64_t)src[4 * q] - x_off, (int64_t)src[4 * q + 1] - x_off,
                            (int64_t)src[4 * q + 2] - x_off, (int64_t)src[4 * q + 3] - x_off};
      uint32_t w[L];
      ok &= limb_words<L>(v, w);
#pragma unroll
      for (int l = 0; l < L; ++l) words[l][q] = w[l];
    }
  }
  if (!ok) flag(status, EI_DEV_LIMB_RANGE);
  const int64_t tgs = t_pad / kTile;
#pragma unroll
  for (int l = 0; l < L; ++l) {
    v4i v = {(int)words[l][0], (int)words[l][1], (int)words[l][2], (int)words[l][3]};
    int8_t* dst = tiles + ((((int64_t)l * tgs + tg) * nb + b) * 64 + lane) * 16;
    *reinterpret_cast<v4i*>(dst) = v;
  }
}

hipError_t launch_limb_split_flat(const int64_t* x, int8_t* d, int64_t n, int limbs, int32_t* status,
                                  hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 g4((unsigned)(((n + 3) / 4 + 255) / 256)), b(256);
  switch (limbs) {
    case 1: hipLaunchKernelGGL(limb_split4_kernel<1>, g4, b, 0, s, x, d, n, status); break;
    case 2: hipLaunchKernelGGL(limb_split4_kernel<2>, g4, b, 0, s, x, d, n, status); break;
    case 3: hipLaunchKernelGGL(limb_split4_kernel<3>, g4, b, 0, s, x, d, n, status); break;
    case 4: hipLaunchKernelGGL(limb_split4_kernel<4>, g4, b, 0, s, x, d, n, status); break;
    default:
      hipLaunchKernelGGL(limb_split_flat_kernel, dim3((unsigned)((n + 255) / 256)), b, 0, s, x, d, n, limbs, status);
  }
  return hipGetLastError();
}

template <typename XT>
static void launch_tiles_t(const XT* x, int64_t t, int64_t k, int limbs, int8_t* tiles, int64_t t_pad,
                           int32_t* status, hipStream_t s, int64_t x_off) {
  const int64_t threads = t_pad * (k / 32) * 2;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  switch (limbs) {
    case 1:
      hipLaunchKernelGGL((limb_tiles_kernel<1, XT>), grid, block, 0, s, x, t, k, tiles, t_pad, status, x_off);
      break;
    case 2:
      hipLaunchKernelGGL((limb_tiles_kernel<2, XT>), grid, block, 0, s, x, t, k, tiles, t_pad, status, x_off);
      break;
    case 3:
      hipLaunchKernelGGL((limb_tiles_kernel<3, XT>), grid, block, 0, s, x, t, k, tiles, t_pad, status, x_off);
      break;
    default:
      hipLaunchKernelGGL((limb_tiles_kernel<4, XT>), grid, block, 0, s, x, t, k, tiles, t_pad, status, x_off);
      break;
  }
}

hipError_t launch_limb_tiles(const void* x, int x_is_i32, int64_t t, int64_t k, int limbs, int8_t* tiles,
                             int64_t t_pad, int32_t* status, hipStream_t s, int64_t x_off) {
  if (x_is_i32)
    launch_tiles_t(static_cast<const int32_t*>(x), t, k, limbs, tiles, t_pad, status, s, x_off);
  else
    launch_tiles_t(static_cast<const int64_t*>(x), t, k, limbs, tiles, t_pad, status, s, x_off);
  return hipGetLastError();
}

}  // namespace ei
