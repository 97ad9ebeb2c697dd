// Skinny projections: T from 5 to 64 tokens (one or two 32-token tiles).
//
// Too few tokens for the tiled prefill kernel to fill the chip with its
// 128-row workgroups, too many for the GEMV's per-token registers.  The job
// is to stream the weights once, so the K blocks are split: each workgroup
// takes one 32-row tile, one token tile and a range of blocks, its W waves
// split that range again, and the waves' per-limb sums meet in LDS.  When the
// row tiles alone are too few to occupy the chip, the block range is also split
// across workgroups, which then write per-limb int64 partials
// part[p][l][t][i] for the partial combiner (any grouping of the exact block
// terms gives the same sum).
//
// Per block a wave loads one code tile, one scale per row and L activation
// limb tiles (16 bytes per lane each), runs L v_mfma_i32_32x32x32_i8 (exact
// int32 block sums P_l for 32 rows x 32 tokens) and adds S * P_l into 16 int64
// accumulators per limb.  Loads run two batches of D blocks ahead of the
// MFMAs; past the end of a wave's range they are clamped to its last block
// (in bounds, a cache hit) and their scale is taken as zero.
#include "ei_internal.h"

namespace ei {

template <int L, int D>
struct SkinnyBatch {
  v4i q[D];
  int32_t s[D];
  v4i d[D][L];
};

// G = 1: one projection; y = result, or resid + result, or per-limb partials.
// G = 2: the gate (codes, scales) and up (codes2, scales2) projections of an
// FFN layer, W waves each, meet in the epilogue: y = h, the SiLU-gated
// product of the two rounded results (one workgroup split only).
template <int L, int W, int D, int G>
__global__ __launch_bounds__(64 * W * G) void gemm_skinny_kernel(GemmArgs a) {
  __shared__ int64_t red[G][(W - 1) * 16 * 64];
  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = wave_all / W, wave = wave_all % W;   // matrix, wave within it
  const int64_t rg = blockIdx.x, part = blockIdx.y, ks = gridDim.y, tg = blockIdx.z;
  const int64_t tgs = a.t_pad / kTile;
  const int64_t g0 = part * a.nb / ks, g1 = (part + 1) * a.nb / ks;
  const int64_t w0 = g0 + wave * (g1 - g0) / W, w1 = g0 + (wave + 1) * (g1 - g0) / W;
  const int8_t* codes = G == 2 && m == 1 ? a.codes2 : a.codes;
  const int32_t* scales = G == 2 && m == 1 ? a.scales2 : a.scales;
  const v4i* cbase = reinterpret_cast<const v4i*>(codes) + rg * a.nb * 64 + lane;
  const int32_t* sbase = scales + rg * a.nb * 32 + (lane & 31);
  const v4i* lbase = reinterpret_cast<const v4i*>(a.limb_tiles) + tg * a.nb * 64 + lane;
  const int64_t lstride = tgs * a.nb * 64;   // between limbs

  int64_t acc[L][16];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[l][r] = 0;

  if (w1 > w0) {
    const v16i zero = {};
    auto load = [&](SkinnyBatch<L, D>& bt, int64_t pos0) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t b = pos0 + u < w1 ? pos0 + u : w1 - 1;
        bt.q[u] = cbase[b * 64];
        bt.s[u] = sbase[b * 32];
#pragma unroll
        for (int l = 0; l < L; ++l) bt.d[u][l] = lbase[l * lstride + b * 64];
      }
    };
    auto compute = [&](const SkinnyBatch<L, D>& bt, int64_t pos0) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t S = pos0 + u < w1 ? (int64_t)bt.s[u] : 0;
#pragma unroll
        for (int l = 0; l < L; ++l) {
          const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(bt.d[u][l], bt.q[u], zero, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[l][r] += S * (int64_t)P[r];
        }
      }
    };
    SkinnyBatch<L, D> A, B;
    load(A, w0);
    for (int64_t pos = w0; pos < w1; pos += 2 * D) {
      load(B, pos + D);
      compute(A, pos);
      load(A, pos + 2 * D);
      compute(B, pos + D);
    }
  }

  // waves 1 .. W-1 of each matrix hand their sums to its wave 0, one limb at
  // a time
#pragma unroll
  for (int l = 0; l < L; ++l) {
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[m][((wave - 1) * 16 + r) * 64 + lane] = acc[l][r];
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < W; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[l][r] += red[m][((w - 1) * 16 + r) * 64 + lane];
    }
    __syncthreads();
  }

  // D[m = token][n = row]: row lane % 32, token 8(r/4) + 4(lane/32) + r%4
  const int64_t row = rg * kTile + (lane & 31);
  auto rounded = [&](int r, int64_t* out) {
    __int128 v = 0;
#pragma unroll
    for (int l = 0; l < L; ++l) v += (__int128)acc[l][r] << (8 * l);
    return finish_output(v, a.out_mode, out);
  };
  if constexpr (G == 2) {
    // the up projection's wave 0 leaves its rounded results in LDS for the
    // gate's (the same lanes hold the same outputs)
    bool ok = true;
    if (m == 1 && wave == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t u;
        ok = rounded(r, &u) && ok;
        red[0][r * 64 + lane] = u;
      }
    }
    __syncthreads();
    if (m == 1 || wave != 0) {
      if (m == 1 && wave == 0 && !ok && row < a.n) flag(a.status, EI_DEV_OUT_RANGE);
      return;
    }
    if (row >= a.n) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t tok = tg * kTile + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (tok >= a.t) continue;
      int64_t g, h;
      bool good = rounded(r, &g);
      good = silu_gate(g, red[0][r * 64 + lane], a.lut, &h) && good;
      if (!good) flag(a.status, EI_DEV_OUT_RANGE);
      a.y[tok * a.n + row] = h;
    }
    return;
  }
  if (wave != 0) return;
  if (row >= a.n) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t tok = tg * kTile + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (tok >= a.t) continue;
    if (a.out_mode == OUT_PARTIAL) {
#pragma unroll
      for (int l = 0; l < L; ++l) a.part[((part * L + l) * a.t + tok) * a.n + row] = acc[l][r];
    } else {
      int64_t out;
      bool ok = rounded(r, &out);
      if (a.resid) ok = fit_i64((__int128)a.resid[tok * a.n + row] + out, &out) && ok;
      if (!ok) flag(a.status, EI_DEV_OUT_RANGE);
      a.y[tok * a.n + row] = out;
    }
  }
}

constexpr int kSkinnyWaves = 4, kSkinnyDepth = 2;

int skinny_splits(int64_t n_pad, int64_t t_pad, int64_t nb) {
  const int64_t wgs = (n_pad / kTile) * (t_pad / kTile);
  if (wgs >= 128) return 1;   // enough row tiles: no partials
  int64_t ks = (256 + wgs - 1) / wgs;
  const int64_t cap = nb / (kSkinnyWaves * 2 * kSkinnyDepth);   // >= two batches per wave
  if (ks > cap) ks = cap;
  if (ks > 64) ks = 64;
  return ks < 1 ? 1 : (int)ks;
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int limbs, int splits, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_pad / kTile), (unsigned)splits, (unsigned)(a.t_pad / kTile));
  const dim3 block(64 * kSkinnyWaves);
  switch (limbs) {
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, kSkinnyWaves, kSkinnyDepth, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, kSkinnyWaves, kSkinnyDepth, 1>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kSkinnyDepth, 1>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_skinny_kernel<4, kSkinnyWaves, kSkinnyDepth, 1>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_skinny_gateup(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_pad / kTile), 1, (unsigned)(a.t_pad / kTile));
  hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kSkinnyDepth, 2>), grid, dim3(64 * kSkinnyWaves * 2), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace ei
