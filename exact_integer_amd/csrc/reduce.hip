// Partial-sum combination for the split-K and tree schedules, and the seeded
// permutation used by the shuffled schedule ("Vendor-Invariant Integer
// Inference for MindChain: Handshake v0", Construction / Schedule gate: the
// same GEMM under canonical, reversed, tiled_shuffled, split_k and tree_walk
// schedules must give one digest).
#include "ei_internal.h"

namespace ei {

// y[t][i] from per-limb partials part[p][l][t][i]; each partial sum is exact
// in int64.  With resid,
// y = resid + (that result), checked to fit int64; with row_off (exact
// outputs), row_off[i] is added to the exact sum.
__global__ void combine_partials_kernel(const int64_t* __restrict__ part, int nparts, int64_t* __restrict__ y,
                                        int64_t t, int64_t n, int limbs, int out_mode,
                                        const int64_t* __restrict__ resid, int32_t* status,
                                        const int64_t* __restrict__ row_off) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= t * n) return;
  const int64_t tn = t * n;
  int64_t sum[kMaxLimbs] = {};
  // eight partials' loads in flight at a time (the order of the int64 sums
  // is immaterial: each is exact)
  for (int p0 = 0; p0 < nparts; p0 += 8) {
#pragma unroll
    for (int l = 0; l < kMaxLimbs; ++l) {
      if (l >= limbs) break;
      int64_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p0 + j < nparts ? part[((int64_t)(p0 + j) * limbs + l) * tn + e] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) sum[l] += v[j];
    }
  }
  int64_t out;
  bool ok = true;
  if (limbs <= 3 && out_mode == OUT_ROUND_Q24) {
    out = round_q24_3(sum[0], limbs > 1 ? sum[1] : 0, limbs > 2 ? sum[2] : 0);
  } else {
    __int128 v = row_off ? (__int128)row_off[e % n] : 0;
#pragma unroll
    for (int l = 0; l < kMaxLimbs; ++l)
      if (l < limbs) v += (__int128)sum[l] << (8 * l);
    ok = finish_output(v, out_mode, &out);
  }
  if (resid) ok = fit_i64((__int128)resid[e] + out, &out) && ok;
  if (!ok) flag(status, EI_DEV_OUT_RANGE);
  y[e] = out;
}

// y[t][i] from (h, r) partials part[p][2][t][i] (acc = 2^24 sum h + sum r;
// the r are below 3 * 2^24 each), plus resid when given.
__global__ void combine_hr_kernel(const int64_t* __restrict__ part, int nparts, int64_t* __restrict__ y, int64_t t,
                                  int64_t n, int out_mode, const int64_t* __restrict__ resid, int32_t* status,
                                  const int64_t* __restrict__ row_off) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= t * n) return;
  const int64_t tn = t * n;
  int64_t h = 0, r = 0;
  for (int p0 = 0; p0 < nparts; p0 += 8) {   // eight partials' loads in flight
    int64_t vh[8], vr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = p0 + j < nparts;
      vh[j] = in ? part[(int64_t)(p0 + j) * 2 * tn + e] : 0;
      vr[j] = in ? part[((int64_t)(p0 + j) * 2 + 1) * tn + e] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h += vh[j];
      r += vr[j];
    }
  }
  int64_t out;
  bool ok;
  if (row_off)   // exact outputs: acc = 2^24 h + r + row_off[i]
    ok = fit_i64((__int128)h * ((__int128)1 << 24) + r + row_off[e % n], &out);
  else
    ok = finish_hr(h, r, out_mode, &out);
  if (resid) ok = fit_i64((__int128)resid[e] + out, &out) && ok;
  if (!ok) flag(status, EI_DEV_OUT_RANGE);
  y[e] = out;
}

// combine_hr_kernel whose outputs also go out as 3-limb activation tiles for
// the next projection ([3][t_pad/32][n/32][64 lanes][16 B]; n a multiple of
// 32): the residual stream's next input, split where it is formed.  One
// output per thread; its three digits are single-byte stores.
__global__ void combine_hr_tiles_kernel(const int64_t* __restrict__ part, int nparts, int64_t* __restrict__ y,
                                        int64_t t, int64_t n, const int64_t* __restrict__ resid,
                                        int8_t* __restrict__ tiles, int64_t t_pad, int32_t* status) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= t * n) return;
  const int64_t tn = t * n, tok = e / n, c = e % n;
  int64_t h = 0, r = 0;
  for (int p0 = 0; p0 < nparts; p0 += 8) {   // eight partials' loads in flight
    int64_t vh[8], vr[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = p0 + q < nparts;
      vh[q] = in ? part[(int64_t)(p0 + q) * 2 * tn + e] : 0;
      vr[q] = in ? part[((int64_t)(p0 + q) * 2 + 1) * tn + e] : 0;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      h += vh[q];
      r += vr[q];
    }
  }
  int64_t out;
  bool ok = finish_hr(h, r, OUT_ROUND_Q24, &out);
  if (resid) ok = fit_i64((__int128)resid[e] + out, &out) && ok;
  if (!ok) flag(status, EI_DEV_OUT_RANGE);
  y[e] = out;
  // balanced digits: the bytes of out + 0x808080, each less 0x80
  const uint64_t u = (uint64_t)out + 0x808080u;
  if (u >> 24) flag(status, EI_DEV_LIMB_RANGE);
  const int64_t nb = n / 32, tg = tok / 32, tgs = t_pad / 32;
  const int64_t lane16 = (tok % 32) + 32 * ((c % 32) / 16);
#pragma unroll
  for (int l = 0; l < 3; ++l)
    tiles[(((l * tgs + tg) * nb + c / 32) * 64 + lane16) * 16 + (c % 16)] = (int8_t)(((u >> (8 * l)) & 0xFF) ^ 0x80);
}

// y += resid, checked to fit int64.
__global__ void add_residual_kernel(int64_t* __restrict__ y, const int64_t* __restrict__ resid, int64_t n,
                                    int32_t* status) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  int64_t out;
  if (!fit_i64((__int128)y[e] + resid[e], &out)) flag(status, EI_DEV_OUT_RANGE);
  y[e] = out;
}

// Pairwise tree over the per-block terms terms[b][l][t][i]: pairs (0,1),
// (2,3), ... at every level, an odd last term passes up unchanged.  Each
// thread owns one (t, i) and reduces its L columns in place.
__global__ void tree_terms_kernel(int64_t* __restrict__ terms, int64_t nb, int64_t* __restrict__ y, int64_t t,
                                  int64_t n, int limbs, int out_mode, int32_t* status,
                                  const int64_t* __restrict__ row_off) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= t * n) return;
  const int64_t stride = (int64_t)limbs * t * n;   // between consecutive blocks
  __int128 v = 0;
  for (int l = 0; l < limbs; ++l) {
    int64_t* col = terms + (int64_t)l * t * n + e;
    int64_t cnt = nb;
    while (cnt > 1) {
      int64_t m = 0;
      for (; 2 * m + 1 < cnt; ++m) col[m * stride] = col[2 * m * stride] + col[(2 * m + 1) * stride];
      if (cnt & 1) { col[m * stride] = col[(cnt - 1) * stride]; ++m; }
      cnt = m;
    }
    v += (__int128)(nb > 0 ? col[0] : 0) << (8 * l);
  }
  if (row_off) v += row_off[e % n];
  int64_t out;
  if (!finish_output(v, out_mode, &out)) flag(status, EI_DEV_OUT_RANGE);
  y[e] = out;
}

// splitmix64 (Steele, Lea and Flood, 2014) followed by a Fisher-Yates shuffle:
// perm is a seeded permutation of 0 .. n-1.  One thread; n is a tile or block
// count.
__global__ void make_perm_kernel(int32_t* perm, int64_t n, uint64_t seed) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  for (int64_t i = 0; i < n; ++i) perm[i] = (int32_t)i;
  uint64_t st = seed;
  for (int64_t i = n - 1; i > 0; --i) {
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    const int64_t j = (int64_t)(z % (uint64_t)(i + 1));
    const int32_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
}

hipError_t launch_combine_partials(const int64_t* part, int nparts, int64_t* y, int64_t t, int64_t n, int limbs,
                                   int out_mode, const int64_t* resid, int32_t* status, hipStream_t s,
                                   const int64_t* row_off) {
  const int64_t total = t * n;
  hipLaunchKernelGGL(combine_partials_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nparts, y,
                     t, n, limbs, out_mode, resid, status, row_off);
  return hipGetLastError();
}

hipError_t launch_combine_hr(const int64_t* part, int nparts, int64_t* y, int64_t t, int64_t n, int out_mode,
                             const int64_t* resid, int32_t* status, hipStream_t s, const int64_t* row_off) {
  const int64_t total = t * n;
  hipLaunchKernelGGL(combine_hr_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nparts, y, t, n,
                     out_mode, resid, status, row_off);
  return hipGetLastError();
}

hipError_t launch_combine_hr_tiles(const int64_t* part, int nparts, int64_t* y, int64_t t, int64_t n,
                                   const int64_t* resid, int8_t* tiles, int64_t t_pad, int32_t* status,
                                   hipStream_t s) {
  const int64_t total = t * n;
  hipLaunchKernelGGL(combine_hr_tiles_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nparts, y,
                     t, n, resid, tiles, t_pad, status);
  return hipGetLastError();
}

hipError_t launch_add_residual(int64_t* y, const int64_t* resid, int64_t n, int32_t* status, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_residual_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, resid, n, status);
  return hipGetLastError();
}

hipError_t launch_tree_terms(int64_t* terms, int64_t nb, int64_t* y, int64_t t, int64_t n, int limbs, int out_mode,
                             int32_t* status, hipStream_t s, const int64_t* row_off) {
  const int64_t total = t * n;
  hipLaunchKernelGGL(tree_terms_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, terms, nb, y, t, n,
                     limbs, out_mode, status, row_off);
  return hipGetLastError();
}

hipError_t launch_make_perm(int32_t* perm, int64_t n, uint64_t seed, hipStream_t s) {
  hipLaunchKernelGGL(make_perm_kernel, dim3(1), dim3(64), 0, s, perm, n, seed);
  return hipGetLastError();
}

}  // namespace ei
