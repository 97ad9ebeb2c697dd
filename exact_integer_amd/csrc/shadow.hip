// FP32 shadow of the Q8 projection: the negative control of the schedule gate
// ("Vendor-Invariant Integer Inference for MindChain: Handshake v0", claim C3
// and Construction / Schedule gate: the same GEMM computed in float under the
// five schedules is expected to give several bit patterns, where the integer
// profile gives one digest).
//
// Operands are w = fl32(S q 2^-24) and x = fl32(X 2^-16); products and sums
// are single float32 roundings taken one at a time (contraction into fused
// multiply-adds is switched off for this file) in the schedule's order:
//   canonical       columns ascending over all of K;
//   reversed        columns descending;
//   tiled_shuffled  128-column K tiles in a seeded permutation (splitmix64,
//                   Fisher-Yates), ascending within a tile, one running sum;
//   split_k         8 partial sums over contiguous block ranges, then
//                   0 + p7 + p6 + ... + p0;
//   tree_walk       per-block sums, then a pairwise tree (pairs (0,1), (2,3),
//                   ...; an odd last term passes up).
// One thread per output element; the tree is formed with a binary-counter
// stack, which pairs the terms exactly as the level-by-level tree does.
#include "ei_internal.h"

// every product and sum below is its own float32 rounding: no contraction
// into fused multiply-adds anywhere in this file
#pragma clang fp contract(off)

namespace ei {

__device__ inline float shadow_w(const int8_t* q, const int32_t* s, int64_t k, int64_t i, int64_t j) {
  return (float)((double)((int64_t)s[i * (k / 32) + j / 32] * (int64_t)q[i * k + j]) * (1.0 / 16777216.0));
}
__device__ inline float shadow_x(const int64_t* x, int64_t k, int64_t t, int64_t j) {
  return (float)((double)x[t * k + j] * (1.0 / 65536.0));
}

__global__ __launch_bounds__(256) void shadow_kernel(const int8_t* __restrict__ q, const int32_t* __restrict__ s,
                                                     const int64_t* __restrict__ x, float* __restrict__ y, int64_t n,
                                                     int64_t k, int64_t t, int schedule, uint64_t seed) {
  extern __shared__ int32_t ktile[];   // tiled_shuffled: permutation of the 128-column tiles
  const int64_t nkt = (k + 127) / 128, nb = k / 32;
  if (schedule == EI_SCHED_TILED_SHUFFLED) {
    if (threadIdx.x == 0) {
      for (int64_t v = 0; v < nkt; ++v) ktile[v] = (int32_t)v;
      uint64_t st = seed;
      for (int64_t i = nkt - 1; i > 0; --i) {   // splitmix64 (Steele, Lea, Flood 2014) + Fisher-Yates
        uint64_t z = (st += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        const int64_t j = (int64_t)(z % (uint64_t)(i + 1));
        const int32_t tmp = ktile[i];
        ktile[i] = ktile[j];
        ktile[j] = tmp;
      }
    }
    __syncthreads();
  }
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= t * n) return;
  const int64_t tok = e / n, i = e % n;
  float a = 0.0f;
  auto term = [&](int64_t j) { return shadow_w(q, s, k, i, j) * shadow_x(x, k, tok, j); };
  if (schedule == EI_SCHED_REVERSED) {
    for (int64_t j = k - 1; j >= 0; --j) a = a + term(j);
  } else if (schedule == EI_SCHED_TILED_SHUFFLED) {
    for (int64_t v = 0; v < nkt; ++v)
      for (int64_t j = (int64_t)ktile[v] * 128; j < (int64_t)ktile[v] * 128 + 128 && j < k; ++j) a = a + term(j);
  } else if (schedule == EI_SCHED_SPLIT_K) {
    float part[8];
    for (int p = 0; p < 8; ++p) {
      part[p] = 0.0f;
      for (int64_t j = (p * nb / 8) * 32; j < ((p + 1) * nb / 8) * 32; ++j) part[p] = part[p] + term(j);
    }
    for (int p = 7; p >= 0; --p) a = a + part[p];
  } else if (schedule == EI_SCHED_TREE) {
    float stack[40];
    int level[40], depth = 0;
    for (int64_t b = 0; b < nb; ++b) {
      float c = 0.0f;
      for (int64_t j = b * 32; j < b * 32 + 32; ++j) c = c + term(j);
      int lv = 0;
      while (depth > 0 && level[depth - 1] == lv) {   // merge equal-size neighbours: (left + right)
        c = stack[depth - 1] + c;
        --depth;
        ++lv;
      }
      stack[depth] = c;
      level[depth] = lv;
      ++depth;
    }
    a = depth > 0 ? stack[depth - 1] : 0.0f;        // remaining groups: right to left
    for (int d = depth - 2; d >= 0; --d) a = stack[d] + a;
  } else {
    for (int64_t j = 0; j < k; ++j) a = a + term(j);
  }
  y[e] = a;
}

hipError_t launch_shadow(const int8_t* q, const int32_t* s, const int64_t* x, float* y, int64_t n, int64_t k,
                         int64_t t, int schedule, uint64_t seed, hipStream_t st) {
  const int64_t total = t * n, nkt = (k + 127) / 128;
  const size_t lds = schedule == EI_SCHED_TILED_SHUFFLED ? (size_t)nkt * 4 : 0;
  hipLaunchKernelGGL(shadow_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), lds, st, q, s, x, y, n, k, t,
                     schedule, seed);
  return hipGetLastError();
}

}  // namespace ei
