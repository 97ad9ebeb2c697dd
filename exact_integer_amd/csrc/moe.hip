// Expert grouping for the routed projection ("Deterministic, Reproducible
// Inference in Exact Integer Arithmetic ...", 3.2 "Mixture-of-Experts": the
// selected experts of a token are exact-integer MLPs; top-k ties are broken by
// index).
//
// A pair p = r * topk + k is activation row r sent to expert route[p].  The
// pairs are sorted stably by expert (key = expert * 2^14 + p, all keys
// distinct, so the order is unique), cut into token tiles of at most 32 pairs
// of one expert, and the tiles' activation limbs are gathered into the MFMA
// operand layout.  The grouped GEMM then runs one token tile per workgroup
// column and writes each result to its pair's own output row, so the output
// is in pair order and independent of the grouping.
#include "ei_internal.h"

namespace ei {

constexpr int kMoeSortThreads = 1024;
constexpr int64_t kMoeMaxPairs = 1 << 14;   // pair index field of the sort key

// One workgroup: bitonic sort of the keys in LDS, then segment offsets and the
// token-tile table.  Keys of pairs with an expert outside [0, E) become
// E * 2^14 + p (they sort last and join no tile) and set EI_DEV_ROUTE.
__global__ __launch_bounds__(kMoeSortThreads) void moe_sort_kernel(const int32_t* __restrict__ route, int64_t pairs,
                                                                  int64_t experts, int32_t* __restrict__ sorted_pair,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ tile_expert,
                                                                  int32_t* __restrict__ tile_row0,
                                                                  int32_t* __restrict__ tile_rows,
                                                                  int32_t* __restrict__ ntiles, int32_t* status) {
  extern __shared__ uint32_t keys[];   // n2 = next power of two >= pairs
  const int tid = threadIdx.x;
  int n2 = 1;
  while (n2 < pairs) n2 <<= 1;
  bool bad = false;
  for (int i = tid; i < n2; i += kMoeSortThreads) {
    if (i < pairs) {
      int64_t e = route[i];
      if (e < 0 || e >= experts) {
        bad = true;
        e = experts;
      }
      keys[i] = (uint32_t)(e << 14) | (uint32_t)i;
    } else {
      keys[i] = 0xFFFFFFFFu;
    }
  }
  if (bad) flag(status, EI_DEV_ROUTE);
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2; i += kMoeSortThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint32_t a = keys[i], b = keys[j];
          if ((a > b) == up) {
            keys[i] = b;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // sorted pairs; offsets[e] = first sorted position whose expert is >= e
  for (int i = tid; i <= pairs; i += kMoeSortThreads) {
    const int64_t ei = i < pairs ? (int64_t)(keys[i] >> 14) : experts;
    const int64_t ep = i > 0 ? (int64_t)(keys[i - 1] >> 14) : -1;
    if (i < pairs) sorted_pair[i] = (int32_t)(keys[i] & 0x3FFFu);
    const int64_t hi = ei < experts ? ei : experts;
    for (int64_t e = ep + 1; e <= hi; ++e) offsets[e] = i;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t j = 0;
    for (int64_t e = 0; e < experts; ++e) {
      const int32_t beg = offsets[e], cnt = offsets[e + 1] - beg;
      for (int32_t s = 0; s < cnt; s += kTile, ++j) {
        tile_expert[j] = (int32_t)e;
        tile_row0[j] = beg + s;
        tile_rows[j] = cnt - s < kTile ? cnt - s : kTile;
      }
    }
    *ntiles = j;
  }
}

// Limb tiles of the grouped activations: thread (tile j, block b, lane) takes
// the 16 activations of half lane / 32 of block b of the row of the pair at
// sorted position tile_row0[j] + lane % 32 (zeros past the tile's pairs).
template <int L>
__global__ void grouped_limb_tiles_kernel(const int64_t* __restrict__ x, int64_t k, int topk,
                                          const int32_t* __restrict__ sorted_pair,
                                          const int32_t* __restrict__ tile_row0,
                                          const int32_t* __restrict__ tile_rows, const int32_t* __restrict__ ntiles,
                                          int64_t tiles_max, int8_t* __restrict__ tiles, int32_t* status) {
  const int64_t nb = k / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= tiles_max * nb * 64) return;
  const int lane = (int)(gid & 63), h = lane >> 5;
  const int64_t b = (gid >> 6) % nb, j = (gid >> 6) / nb;
  if (j >= *ntiles) return;
  uint32_t words[L][4];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int w = 0; w < 4; ++w) words[l][w] = 0;
  bool ok = true;
  if ((lane & 31) < tile_rows[j]) {
    const int64_t r = sorted_pair[tile_row0[j] + (lane & 31)] / topk;
    const int64_t* src = x + r * k + b * 32 + 16 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t v[4] = {src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]};
      uint32_t w[L];
      ok &= limb_words<L>(v, w);
#pragma unroll
      for (int l = 0; l < L; ++l) words[l][q] = w[l];
    }
  }
  if (!ok) flag(status, EI_DEV_LIMB_RANGE);
#pragma unroll
  for (int l = 0; l < L; ++l) {
    v4i v = {(int)words[l][0], (int)words[l][1], (int)words[l][2], (int)words[l][3]};
    *reinterpret_cast<v4i*>(tiles + ((((int64_t)l * tiles_max + j) * nb + b) * 64 + lane) * 16) = v;
  }
}

hipError_t launch_moe_sort(const int32_t* route, int64_t pairs, int64_t experts, int32_t* sorted_pair,
                           int32_t* offsets, int32_t* tile_expert, int32_t* tile_row0, int32_t* tile_rows,
                           int32_t* ntiles, int32_t* status, hipStream_t s) {
  int64_t n2 = 1;
  while (n2 < pairs) n2 <<= 1;
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(kMoeSortThreads), (size_t)n2 * 4, s, route, pairs, experts,
                     sorted_pair, offsets, tile_expert, tile_row0, tile_rows, ntiles, status);
  return hipGetLastError();
}

hipError_t launch_grouped_limb_tiles(const int64_t* x, int64_t k, int topk, const int32_t* sorted_pair,
                                     const int32_t* tile_row0, const int32_t* tile_rows, const int32_t* ntiles,
                                     int64_t tiles_max, int8_t* tiles, int32_t* status, hipStream_t s) {
  const int64_t threads = tiles_max * (k / 32) * 64;
  hipLaunchKernelGGL(grouped_limb_tiles_kernel<3>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, k,
                     topk, sorted_pair, tile_row0, tile_rows, ntiles, tiles_max, tiles, status);
  return hipGetLastError();
}

}  // namespace ei
