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

__device__ inline int64_t block_at(const GemmArgs& a, int64_t pos) {
  // pos-th block visited in [b0, b1)
  if (a.order == ORDER_DESC) return a.b1 - 1 - pos;
  if (a.order == ORDER_PERM) return a.kperm[a.b0 + pos];
  return a.b0 + pos;
}

// ===================================================================== GEMV
// T <= 4 tokens.  One workgroup (8 waves) per row group of 32 rows.  Lane l of
// every wave owns row l%32 and the half-block 16*(l/32) .. +15 of each block
// it visits; wave w visits the positions w, w+8, ... of each K chunk.  The
// activation limbs of a chunk (<= 128 blocks) are split once into LDS and
// read back as 16-byte broadcasts.  Per visited block a lane issues one
// 16-byte code load, one scale load, 4*T*L dot4 and T*L int64 multiply-adds.
constexpr int kGemvWaves = 8;
constexpr int kGemvChunk = 128;   // blocks staged per chunk
constexpr int kGemvBatch = 8;     // blocks whose loads a wave issues together

template <int L, int T, typename XT>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];   // 4096 * L * T bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rg = a.tperm ? a.tperm[blockIdx.x] : blockIdx.x;
  const int h = lane >> 5;
  const int64_t nblk = a.b1 - a.b0;
  const XT* x = static_cast<const XT*>(a.x);
  const v4i* codes = reinterpret_cast<const v4i*>(a.codes);

  int64_t acc[T][L];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int l = 0; l < L; ++l) acc[t][l] = 0;

  bool range_ok = true;
  for (int64_t c0 = 0; c0 < nblk; c0 += kGemvChunk) {
    const int cb = (int)(nblk - c0 < kGemvChunk ? nblk - c0 : kGemvChunk);
    // ---- stage: slot s holds limbs of block block_at(c0 + s): [s][l][t][32 bytes]
    for (int e = tid; e < cb * T * 8; e += kGemvWaves * 64) {
      const int g = e & 7, t = (e >> 3) % T, s = (e >> 3) / T;
      const int64_t b = block_at(a, c0 + s);
      const XT* src = x + (int64_t)t * a.k + b * 32 + 4 * g;
      uint32_t w[L];
#pragma unroll
      for (int l = 0; l < L; ++l) w[l] = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint64_t r = (uint64_t)(int64_t)src[p];
#pragma unroll
        for (int l = 0; l < L; ++l) {
          int dl = (int)((r + 128u) & 255u) - 128;
          w[l] |= ((uint32_t)(uint8_t)(int8_t)dl) << (8 * p);
          r = (uint64_t)(((int64_t)(r - (uint64_t)(int64_t)dl)) >> 8);
        }
        range_ok &= (r == 0);
      }
#pragma unroll
      for (int l = 0; l < L; ++l)
        reinterpret_cast<uint32_t*>(lds)[(((s * L + l) * T + t) * 32 + 4 * g) >> 2] = w[l];
    }
    __syncthreads();
    // ---- contract: kGemvBatch blocks per wave per step, their loads issued together
    for (int s0 = wave; s0 < cb; s0 += kGemvWaves * kGemvBatch) {
      v4i q[kGemvBatch];
      int32_t S[kGemvBatch];
      int64_t bb[kGemvBatch];
#pragma unroll
      for (int u = 0; u < kGemvBatch; ++u) {
        const int s = s0 + u * kGemvWaves;
        bb[u] = s < cb ? block_at(a, c0 + s) : -1;
        if (bb[u] >= 0) {
          q[u] = codes[(rg * a.nb + bb[u]) * 64 + lane];
          S[u] = a.scales[(rg * a.nb + bb[u]) * 32 + (lane & 31)];
        }
      }
#pragma unroll
      for (int u = 0; u < kGemvBatch; ++u) {
        if (bb[u] < 0) continue;
        const int s = s0 + u * kGemvWaves;
        const int64_t b = bb[u];
        int32_t P[T][L];
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int l = 0; l < L; ++l) {
            const v4i d = *reinterpret_cast<const v4i*>(lds + ((s * L + l) * T + t) * 32 + 16 * h);
            int p = 0;
            p = __builtin_amdgcn_sdot4(q[u][0], d[0], p, false);
            p = __builtin_amdgcn_sdot4(q[u][1], d[1], p, false);
            p = __builtin_amdgcn_sdot4(q[u][2], d[2], p, false);
            p = __builtin_amdgcn_sdot4(q[u][3], d[3], p, false);
            P[t][l] = p;
          }
        if (a.out_mode == OUT_TERMS) {
          // the per-block term S * P over the whole block: add the other half
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int l = 0; l < L; ++l) {
              const int32_t other = __shfl_xor(P[t][l], 32);
              const int64_t row = rg * kTile + (lane & 31);
              if (h == 0 && row < a.n)
                a.part[((b * L + l) * a.t + t) * a.n + row] = (int64_t)S[u] * (int64_t)(P[t][l] + other);
            }
        } else {
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int l = 0; l < L; ++l) acc[t][l] += (int64_t)S[u] * (int64_t)P[t][l];
        }
      }
    }
    __syncthreads();
  }
  if (!range_ok) flag(a.status, EI_DEV_LIMB_RANGE);
  if (a.out_mode == OUT_TERMS) return;

  // ---- reduce the 8 waves x 2 halves of every (row, t, l)
  int64_t* red = reinterpret_cast<int64_t*>(lds);   // [wave][lane][t][l]
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int l = 0; l < L; ++l) red[((wave * 64 + lane) * T + t) * L + l] = acc[t][l];
  __syncthreads();
  if (tid < 32 * T) {
    const int r = tid & 31, t = tid >> 5;
    const int64_t row = rg * kTile + r;
    if (row < a.n) {
      int64_t sum[L];
#pragma unroll
      for (int l = 0; l < L; ++l) sum[l] = 0;
      for (int w = 0; w < kGemvWaves; ++w)
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int l = 0; l < L; ++l) sum[l] += red[((w * 64 + hh * 32 + r) * T + t) * L + l];
      if (a.out_mode == OUT_PARTIAL) {
#pragma unroll
        for (int l = 0; l < L; ++l) a.part[(((int64_t)a.part_index * L + l) * a.t + t) * a.n + row] = sum[l];
      } else {
        __int128 v = 0;
#pragma unroll
        for (int l = 0; l < L; ++l) v += (__int128)sum[l] << (8 * l);
        int64_t out;
        if (!finish_output(v, a.out_mode, &out)) flag(a.status, EI_DEV_OUT_RANGE);
        a.y[(int64_t)t * a.n + row] = out;
      }
    }
  }
}

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
      __int128 v = 0;
#pragma unroll
      for (int l = 0; l < L; ++l) v += (__int128)acc[l][r] << (8 * l);
      int64_t out;
      if (!finish_output(v, a.out_mode, &out)) flag(a.status, EI_DEV_OUT_RANGE);
      a.y[tok * a.n + row] = out;
    }
  }
}

// ================================================================ launchers
template <int L, int T>
static void gemv_t(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_pad / kTile)), block(kGemvWaves * 64);
  const size_t lds = 4096u * L * T;
  if (a.x_is_i32)
    hipLaunchKernelGGL((gemv_kernel<L, T, int32_t>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<L, T, int64_t>), grid, block, lds, s, a);
}

template <int L>
static void gemv_l(const GemmArgs& a, hipStream_t s) {
  switch (a.t) {
    case 1: gemv_t<L, 1>(a, s); break;
    case 2: gemv_t<L, 2>(a, s); break;
    case 3: gemv_t<L, 3>(a, s); break;
    default: gemv_t<L, 4>(a, s); break;
  }
}

hipError_t launch_gemv(const GemmArgs& a, int limbs, hipStream_t s) {
  switch (limbs) {
    case 1: gemv_l<1>(a, s); break;
    case 2: gemv_l<2>(a, s); break;
    case 3: gemv_l<3>(a, s); break;
    default: gemv_l<4>(a, s); break;
  }
  return hipGetLastError();
}

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
