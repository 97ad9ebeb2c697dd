// Exact block-scaled projection kernels.
//
// Both kernels compute, for every (token t, row i), the per-limb sums
//     A_l[t][i] = sum_b S[i][b] * P_l[t][i][b],
//     P_l[t][i][b] = sum_{j in b} q[i][j] * d_l[t][j]          (int32, exact)
// where d_l are the balanced base-256 limbs of x.  Each product S * P_l is
// at most 2^31 * 2^19 = 2^50 in magnitude, so A_l (and any partial sum over a
// subset of blocks) is exact in int64 for up to 2^13 blocks.  The limbs are
// combined once per output in int128, acc = sum_l 2^(8l) A_l, and rounded.
// Because every step is exact integer arithmetic, the visiting order of the
// blocks (ascending, descending, permuted, split into ranges, summed in a
// tree) cannot change a bit of the result.
#include "ei_internal.h"

namespace ei {

// ===================================================================== MFMA
// T > 4.  A = activation limb tile (M = 32 tokens), B = code tile (N = 32
// rows), both 1 KB tiles loaded with one 16-byte load per lane, K = 32 = one
// block per v_mfma_i32_32x32x32_i8.  The output tile D[m = token][n = row] puts
// one row and 16 tokens in every lane (token 8(r/4) + 4(l/32) + r%4 in
// register r, row l%32), so one scale per lane per block serves all 16
// int64 multiply-adds.  Each wave owns one 32x32 output tile; a workgroup of 4
// waves covers 64 rows x 64 tokens.
template <int L, bool TERMS>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ngx = (a.n_pad / kTile + 1) / 2;
  int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  if (a.tperm) tile = a.tperm[tile];
  const int64_t rg = 2 * (tile % ngx) + (wave & 1);
  const int64_t tg = 2 * (tile / ngx) + (wave >> 1);
  const int64_t rgs = a.n_pad / kTile, tgs = a.t_pad / kTile;
  if (rg >= rgs || tg >= tgs) return;
  const int64_t nblk = a.b1 - a.b0;
  // per-wave bases; block b adds b*64 tiles-lanes (codes, limbs) or b*32 (scales)
  const v4i* cbase = reinterpret_cast<const v4i*>(a.codes) + rg * a.nb * 64 + lane;
  const int32_t* sbase = a.scales + rg * a.nb * 32 + (lane & 31);
  const v4i* lbase = reinterpret_cast<const v4i*>(a.limb_tiles) + tg * a.nb * 64 + lane;
  const int64_t lstride = tgs * a.nb * 64;   // between limbs
  const int64_t row = rg * kTile + (lane & 31);

  int64_t acc[L][16];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[l][r] = 0;
  const v16i zero = {};

  for (int64_t pos = 0; pos < nblk; ++pos) {
    const int64_t b = block_at(a, pos);
    const v4i q = cbase[b * 64];
    const int32_t S = sbase[b * 32];
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const v4i d = lbase[l * lstride + b * 64];
      const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(d, q, zero, 0, 0, 0);
      if (TERMS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t tok = tg * kTile + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (tok < a.t && row < a.n) a.part[((b * L + l) * a.t + tok) * a.n + row] = (int64_t)S * (int64_t)D[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[l][r] += (int64_t)S * (int64_t)D[r];
      }
    }
  }
  if (TERMS || row >= a.n) return;

#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t tok = tg * kTile + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (tok >= a.t) continue;
    if (a.out_mode == OUT_PARTIAL) {
#pragma unroll
      for (int l = 0; l < L; ++l) a.part[(((int64_t)a.part_index * L + l) * a.t + tok) * a.n + row] = acc[l][r];
    } else {
      __int128 v = a.row_off ? (__int128)a.row_off[row] : 0;   // the two-limb 4-bit form's R_i
#pragma unroll
      for (int l = 0; l < L; ++l) v += (__int128)acc[l][r] << (8 * l);
      int64_t out;
      if (!finish_output(v, a.out_mode, &out)) flag(a.status, EI_DEV_OUT_RANGE);
      a.y[tok * a.n + row] = out;
    }
  }
}

// ================================================================ launchers
template <int L>
static void mfma_l(const GemmArgs& a, dim3 grid, hipStream_t s) {
  if (a.out_mode == OUT_TERMS)
    hipLaunchKernelGGL((gemm_mfma_kernel<L, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<L, false>), grid, dim3(256), 0, s, a);
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int limbs, hipStream_t s) {
  const unsigned gx = (unsigned)((a.n_pad / kTile + 1) / 2), gy = (unsigned)((a.t_pad / kTile + 1) / 2);
  const dim3 grid(gx, gy);
  switch (limbs) {
    case 1: mfma_l<1>(a, grid, s); break;
    case 2: mfma_l<2>(a, grid, s); break;
    case 3: mfma_l<3>(a, grid, s); break;
    default: mfma_l<4>(a, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace ei
