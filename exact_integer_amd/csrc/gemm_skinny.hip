// Skinny projections: T from 5 to 64 tokens (one or two 32-token tiles).
//
// Too few tokens for the tiled prefill kernel to fill the chip with its
// 128-row workgroups, too many for the GEMV's per-token registers.  The job
// is to stream the weights once, so the K blocks are split: each workgroup
// takes one 32-row tile, one token tile and a range of blocks, its W waves
// split that range again, and the waves' per-limb sums meet in LDS.  When the
// row tiles alone are too few to occupy the chip, the block range is also split
// across workgroups, which then write partials for a combiner (any grouping
// of the exact block terms gives the same sum).  For up to three limbs every
// wave reduces its per-limb sums to the additive pair (h, r) with
// acc = 2^24 h + r before they meet, and the four waves share the epilogue.
//
// Per block a wave loads one code tile, one scale per row and L activation
// limb tiles (16 bytes per lane each), runs L v_mfma_i32_32x32x32_i8 (exact
// int32 block sums P_l for 32 rows x 32 tokens) and adds S * P_l into 16 int64
// accumulators per limb.  Loads run two batches of D blocks ahead of the
// MFMAs; past the end of a wave's range they are clamped to its last block
// (in bounds, a cache hit) and their scale is taken as zero.  The code tiles
// and scales, read by one token tile's workgroups only, are loaded with the
// non-temporal policy (447.5-447.9 us against 449.3-449.8 us for the 24-layer
// FFN chain at T = 30).
#include "ei_internal.h"

namespace ei {

template <int L, int D>
struct SkinnyBatch {
  v4i q[D];
  int32_t s[D];
  v4i d[D][L];
};

// G = 1: one projection; y = result, or resid + result, or partials (the
// (h, r) pairs of split_hr for up to three limbs, per-limb sums for four).
// G = 2: the gate (codes, scales) and up (codes2, scales2) projections of an
// FFN layer, W waves each, meet in the epilogue: h, the SiLU-gated product of
// the two rounded results, goes out as the down projection's activation limb
// tiles (limb_out; one workgroup split only, n a multiple of 32).
// NARROW (three limbs only): two int64 chains per output, S (P_0 + 2^8 P_1)
// and (2^16 S) P_2, whose sum is the exact total (see narrow_scales).
// STAGE > 0 (the fused gate/up pass with narrow scales, one split, at most
// STAGE blocks per wave): the token tile's limb tiles for the whole K are
// staged in LDS once (the gate waves copy them, one barrier), and every wave
// issues the loads of all its code tiles and scales at once, so each wave
// waits for memory once instead of once per batch.
template <int L, int W, int D, int G, bool NARROW, int STAGE = 0>
__global__ __launch_bounds__(64 * W * G) void gemm_skinny_kernel(GemmArgs a) {
  static_assert(!NARROW || L == 3, "the narrow form takes three limbs");
  static_assert(STAGE == 0 || (G == 2 && NARROW), "staged limbs: the fused narrow gate/up pass");
  constexpr int NACC = NARROW ? 2 : L;
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

  int64_t acc[NACC][16];
#pragma unroll
  for (int l = 0; l < NACC; ++l)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[l][r] = 0;

  if constexpr (STAGE > 0) {
    extern __shared__ __align__(16) uint8_t stage[];   // limb tile (b, l) at (3 b + l) KB
    const v16i zero = {};
    {   // the gate and up waves of one block range copy its limb tiles, half each
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.limb_tiles, (uint32_t)(3 * tgs * a.nb * 1024));
      const int64_t mid = w0 + (w1 - w0 + 1) / 2;
      for (int64_t b = m == 0 ? w0 : mid; b < (m == 0 ? mid : w1); ++b)
#pragma unroll
        for (int l = 0; l < 3; ++l)
          copy16_to_lds(rl, stage + (3 * b + l) * 1024, lane * 16, (uint32_t)(((l * tgs + tg) * a.nb + b) * 1024));
    }
    // then every wave's code tiles and scales, positions past w1 repeating its last block
    v4i q[STAGE];
    int32_t sc[STAGE];
    const int64_t bl = w1 > w0 ? w1 - 1 : 0;   // a wave without blocks loads block 0 (unused)
#pragma unroll
    for (int u = 0; u < STAGE; ++u) {
      const int64_t b = w0 + u < w1 ? w0 + u : bl;
      q[u] = __builtin_nontemporal_load(cbase + b * 64);
      sc[u] = __builtin_nontemporal_load(sbase + b * 32);
    }
    // the copies were issued first: waiting until at most the 2 STAGE code
    // and scale loads are outstanding leaves only those in flight
    barrier_after_vmcnt<2 * STAGE>();
#pragma unroll
    for (int u = 0; u < STAGE; ++u) {
      if (w0 + u >= w1) break;
      const int64_t b = w0 + u;
      const v4i d0 = *reinterpret_cast<const v4i*>(stage + (3 * b + 0) * 1024 + lane * 16);
      const v4i d1 = *reinterpret_cast<const v4i*>(stage + (3 * b + 1) * 1024 + lane * 16);
      const v4i d2 = *reinterpret_cast<const v4i*>(stage + (3 * b + 2) * 1024 + lane * 16);
      v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(d1, q[u], zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = (int)((uint32_t)c[r] << 8);
      const v16i P01 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d0, q[u], c, 0, 0, 0);   // P_0 + 2^8 P_1
      const v16i P2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(d2, q[u], zero, 0, 0, 0);
      const int32_t S16 = (int32_t)((uint32_t)sc[u] << 16);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[0][r] += (int64_t)sc[u] * P01[r];
        acc[NACC - 1][r] += (int64_t)S16 * P2[r];
      }
    }
  } else if (w1 > w0) {
    const v16i zero = {};
    auto load = [&](SkinnyBatch<L, D>& bt, int64_t pos0) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t b = pos0 + u < w1 ? pos0 + u : w1 - 1;
        bt.q[u] = __builtin_nontemporal_load(cbase + b * 64);
        bt.s[u] = __builtin_nontemporal_load(sbase + b * 32);
#pragma unroll
        for (int l = 0; l < L; ++l) bt.d[u][l] = lbase[l * lstride + b * 64];
      }
    };
    auto compute = [&](const SkinnyBatch<L, D>& bt, int64_t pos0) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int32_t S = pos0 + u < w1 ? bt.s[u] : 0;
        if constexpr (NARROW) {
          v16i P[3];
#pragma unroll
          for (int l = 0; l < 3; ++l) P[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bt.d[u][l], bt.q[u], zero, 0, 0, 0);
          const int32_t S16 = (int32_t)((uint32_t)S << 16);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int32_t p01 = (int32_t)(((uint32_t)P[1][r] << 8) + (uint32_t)P[0][r]);
            acc[0][r] += (int64_t)S * p01;
            acc[NACC - 1][r] += (int64_t)S16 * P[2][r];
          }
        } else {
#pragma unroll
          for (int l = 0; l < L; ++l) {
            const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(bt.d[u][l], bt.q[u], zero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[l][r] += (int64_t)S * P[r];
          }
        }
      }
    };
    SkinnyBatch<L, D> A, B;
    if constexpr (G == 1) {
      // two batches in flight, a consumed batch refilled at once; no load
      // sits under a branch (the compiler's own waits would otherwise assume
      // the fewest requests after a load and wait for nearly all of them), so
      // past the range the refills re-read the last block (cache hits).
      // Scheduling barriers keep every load where it is written: the
      // scheduler would otherwise sink a batch's loads to its first use.
      load(A, w0);
      __builtin_amdgcn_sched_barrier(0);
      load(B, w0 + D);
      __builtin_amdgcn_sched_barrier(0);
      for (int64_t pos = w0;; pos += 2 * D) {
        compute(A, pos);
        if (pos + D >= w1) break;
        __builtin_amdgcn_sched_barrier(0);
        load(A, pos + 2 * D);
        __builtin_amdgcn_sched_barrier(0);
        compute(B, pos + D);
        __builtin_amdgcn_sched_barrier(0);
        load(B, pos + 3 * D);   // before the exit test: no path back to the top skips it
        __builtin_amdgcn_sched_barrier(0);
        if (pos + 2 * D >= w1) break;
      }
    } else {
      // the gate/up pair at 256 VGPRs: batches loaded only inside the range
      // (the form above spills here)
      load(A, w0);
      for (int64_t pos = w0;; pos += 2 * D) {
        const bool more_b = pos + D < w1;
        if (more_b) load(B, pos + D);
        compute(A, pos);
        if (!more_b) break;
        const bool more_a = pos + 2 * D < w1;
        if (more_a) load(A, pos + 2 * D);
        compute(B, pos + D);
        if (!more_a) break;
      }
    }
  }

  // D[m = token][n = row]: row lane % 32, token 8(r/4) + 4(lane/32) + r%4
  const int64_t row = rg * kTile + (lane & 31);
  auto token = [&](int r) { return tg * kTile + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };

  if constexpr (G == 2 && NARROW) {
    // Narrow scales: a wave's two chains sum exactly in int64, and so does any
    // sum of them over waves (every partial total is a sum over a subset of
    // blocks, below 2^62.01).  The gate and up waves put their totals in LDS
    // side by side, one barrier, then each of the 8 waves finishes 2 of the
    // 16 outputs of its lanes for both matrices: rounding, the SiLU-gated
    // product, and the 32 x 32 tile of h in LDS (the staged limb area, free
    // once every wave is past the barrier); one more barrier and one wave
    // writes the tile as the down projection's limb tiles.
    static_assert(W == 4, "8 waves, 2 outputs each");
    __shared__ int64_t xs[2][W][16][64];
    extern __shared__ __align__(16) uint8_t dyn[];
    int64_t(*ht)[33] = reinterpret_cast<int64_t(*)[33]>(dyn);   // [token][row], padded rows
#pragma unroll
    for (int r = 0; r < 16; ++r) xs[m][wave][r][lane] = acc[0][r] + acc[NACC - 1][r];
    __syncthreads();
    bool good = true;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 2 * wave_all + j;
      int64_t g = 0, u = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        g += xs[0][w][r][lane];
        u += xs[1][w][r][lane];
      }
      g = (g + ((int64_t)1 << 23)) >> 24;   // floor((acc + 2^23) / 2^24): no overflow below 2^62.01
      u = (u + ((int64_t)1 << 23)) >> 24;
      int64_t h = 0;
      if (token(r) < a.t && row < a.n) good = silu_gate(g, u, a.lut, &h) && good;
      ht[8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = h;
    }
    if (!good) flag(a.status, EI_DEV_OUT_RANGE);
    __syncthreads();
    if (wave_all == 0) {
      // lane: token lane % 32, rows 16 (lane / 32) .. + 15 of the tile
      const int64_t* src = &ht[lane & 31][16 * (lane >> 5)];
      uint32_t words[3][4];
      bool ok = true;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t v[4] = {src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]};
        uint32_t w[3];
        ok = limb_words<3>(v, w) && ok;
#pragma unroll
        for (int l = 0; l < 3; ++l) words[l][q] = w[l];
      }
      if (!ok) flag(a.status, EI_DEV_LIMB_RANGE);
      const int64_t nb_out = a.n_pad / kTile;
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        const v4i v = {(int)words[l][0], (int)words[l][1], (int)words[l][2], (int)words[l][3]};
        reinterpret_cast<v4i*>(a.limb_out)[((l * tgs + tg) * nb_out + rg) * 64 + lane] = v;
      }
    }
    return;
  } else if constexpr (L <= 3) {
    // Every wave turns its sums into the additive pair (h, r) of
    // acc = 2^24 h + r, the pairs meet in LDS, and wave w finishes the four
    // outputs 4w .. 4w + 3 of its lanes (all waves share the epilogue).
    static_assert(W == 4, "one quarter of the 16 outputs per wave");
    __shared__ int64_t xh[W][16][64];
    __shared__ int32_t xr[W][16][64];
    __shared__ int64_t xu[W][4][64];   // G = 2: the up projection's results
    int64_t hs[4], rs[4];
    auto exchange = [&](bool mine) {   // every thread calls it: two barriers
      if (mine) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t h, rr;
          if constexpr (NARROW)   // the exact total, |.| < 2^62.01
            split_hr(acc[0][r] + acc[NACC - 1][r], 0, 0, &h, &rr);
          else
            split_hr(acc[0][r], L > 1 ? acc[L > 1 ? 1 : 0][r] : 0, L > 2 ? acc[L > 2 ? 2 : 0][r] : 0, &h, &rr);
          xh[wave][r][lane] = h;
          xr[wave][r][lane] = (int32_t)rr;   // < 3 * 2^24
        }
      }
      __syncthreads();
      if (mine) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hs[j] = 0;
          rs[j] = 0;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            hs[j] += xh[w][4 * wave + j][lane];
            rs[j] += xr[w][4 * wave + j][lane];
          }
        }
      }
      __syncthreads();
    };
    if constexpr (G == 2) {
      // up first; its results wait in LDS for the gate's waves
      exchange(m == 1);
      if (m == 1) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int64_t u;
          ok = finish_hr(hs[j], rs[j], a.out_mode, &u) && ok;
          xu[wave][j][lane] = u;
        }
        if (!ok && row < a.n) flag(a.status, EI_DEV_OUT_RANGE);
      }
      exchange(m == 0);   // its first barrier also publishes xu
      // h is only the down projection's input: the gate's waves put the
      // 32 x 32 tile of h in LDS (zero past t), and one wave splits it into
      // the down projection's limb tiles (block rg of its K, token tile tg)
      int64_t(*ht)[33] = reinterpret_cast<int64_t(*)[33]>(&xh[0][0][0]);   // [token][row], padded rows
      if (m == 0) {
        bool good = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * wave + j;
          const int64_t tok = token(r);
          int64_t h = 0;
          if (tok < a.t && row < a.n) {
            int64_t g;
            good = finish_hr(hs[j], rs[j], a.out_mode, &g) && good;
            good = silu_gate(g, xu[wave][j][lane], a.lut, &h) && good;
          }
          ht[8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = h;
        }
        if (!good) flag(a.status, EI_DEV_OUT_RANGE);
      }
      __syncthreads();
      if (m == 0 && wave == 0) {
        // lane: token lane % 32, rows 16 (lane / 32) .. + 15 of the tile
        const int64_t* src = &ht[lane & 31][16 * (lane >> 5)];
        uint32_t words[3][4];
        bool ok = true;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t v[4] = {src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]};
          uint32_t w[3];
          ok = limb_words<3>(v, w) && ok;
#pragma unroll
          for (int l = 0; l < 3; ++l) words[l][q] = w[l];
        }
        if (!ok) flag(a.status, EI_DEV_LIMB_RANGE);
        const int64_t nb_out = a.n_pad / kTile;
#pragma unroll
        for (int l = 0; l < 3; ++l) {
          const v4i v = {(int)words[l][0], (int)words[l][1], (int)words[l][2], (int)words[l][3]};
          reinterpret_cast<v4i*>(a.limb_out)[((l * tgs + tg) * nb_out + rg) * 64 + lane] = v;
        }
      }
      return;
    } else {
      exchange(true);
      if (row >= a.n) return;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t tok = token(4 * wave + j);
        if (tok >= a.t) continue;
        if (a.out_mode == OUT_PARTIAL) {   // the (h, r) pair: part[p][2][t][n]
          a.part[((part * 2 + 0) * a.t + tok) * a.n + row] = hs[j];
          a.part[((part * 2 + 1) * a.t + tok) * a.n + row] = rs[j];
        } else {
          int64_t out;
          bool ok = a.row_off   // exact outputs of the two-limb 4-bit form: + R_i
                        ? fit_i64((__int128)hs[j] * ((__int128)1 << 24) + rs[j] + a.row_off[row], &out)
                        : finish_hr(hs[j], rs[j], a.out_mode, &out);
          if (a.resid) ok = fit_i64((__int128)a.resid[tok * a.n + row] + out, &out) && ok;
          if (!ok) flag(a.status, EI_DEV_OUT_RANGE);
          a.y[tok * a.n + row] = out;
        }
      }
      return;
    }
  } else {
    // four limbs: waves 1 .. W-1 hand their per-limb sums to wave 0, one limb
    // at a time; wave 0 writes per-limb partials or the final result
    static_assert(G == 1, "the fused gate/up pass takes three limbs");
    __shared__ int64_t red[(W - 1) * 16 * 64];
#pragma unroll
    for (int l = 0; l < L; ++l) {
      if (wave > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave - 1) * 16 + r) * 64 + lane] = acc[l][r];
      }
      __syncthreads();
      if (wave == 0) {
        for (int w = 1; w < W; ++w)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[l][r] += red[((w - 1) * 16 + r) * 64 + lane];
      }
      __syncthreads();
    }
    if (wave != 0 || row >= a.n) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t tok = token(r);
      if (tok >= a.t) continue;
      if (a.out_mode == OUT_PARTIAL) {
#pragma unroll
        for (int l = 0; l < L; ++l) a.part[((part * L + l) * a.t + tok) * a.n + row] = acc[l][r];
      } else {
        __int128 v = a.row_off ? (__int128)a.row_off[row] : 0;
#pragma unroll
        for (int l = 0; l < L; ++l) v += (__int128)acc[l][r] << (8 * l);
        int64_t out;
        bool ok = finish_output(v, a.out_mode, &out);
        if (a.resid) ok = fit_i64((__int128)a.resid[tok * a.n + row] + out, &out) && ok;
        if (!ok) flag(a.status, EI_DEV_OUT_RANGE);
        a.y[tok * a.n + row] = out;
      }
    }
  }
}

constexpr int kSkinnyWaves = 4, kSkinnyDepth = 2;

// Workgroup K splits: about 140 workgroups in all when the row tiles alone are
// fewer than 128.  (On the 896 x 4864, T = 30 projection, 6 splits measured
// 8.5 us with the partial combiner, 9 splits 9.1 us, one split 11.9 us; in the
// 24-layer FFN chain 3, 4, 5, 6 and 8 splits measured 481, 453, 450, 455 and
// 459 us.)
int skinny_splits(int64_t n_pad, int64_t t_pad, int64_t nb) {
  const int64_t wgs = (n_pad / kTile) * (t_pad / kTile);
  if (wgs >= 128) return 1;   // enough row tiles: no partials
  int64_t ks = (140 + wgs - 1) / wgs;
  const int64_t cap = nb / (kSkinnyWaves * 2 * kSkinnyDepth);   // >= two batches per wave
  if (ks > cap) ks = cap;
  if (ks > 64) ks = 64;
  return ks < 1 ? 1 : (int)ks;
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int limbs, int splits, bool narrow, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_pad / kTile), (unsigned)splits, (unsigned)(a.t_pad / kTile));
  const dim3 block(64 * kSkinnyWaves);
  switch (limbs) {
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, kSkinnyWaves, kSkinnyDepth, 1, false>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, kSkinnyWaves, kSkinnyDepth, 1, false>), grid, block, 0, s, a); break;
    case 3:
      if (narrow)
        hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kSkinnyDepth, 1, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kSkinnyDepth, 1, false>), grid, block, 0, s, a);
      break;
    default: hipLaunchKernelGGL((gemm_skinny_kernel<4, kSkinnyWaves, kSkinnyDepth, 1, false>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// The fused gate/up pass runs one workgroup split, so a wave owns a quarter
// of all the blocks (7 at K = 896).  With narrow scales and K <= 1024 the
// staged form holds the whole K's limb tiles in LDS and all of a wave's code
// tiles in flight at once (11.7 -> 10.8 us per Qwen layer); otherwise the
// narrow form keeps three blocks per batch (four spill registers) and the
// per-limb form two.
constexpr int kGateUpDepth = 3;
constexpr int kGateUpStage = 8;   // blocks per wave with the limb tiles staged in LDS (K <= 1024)

hipError_t launch_gemm_skinny_gateup(const GemmArgs& a, bool narrow, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_pad / kTile), 1, (unsigned)(a.t_pad / kTile));
  // narrow forms: dynamic LDS for the staged limb tiles, then the 32 x 33 int64 tile of h
  const size_t h_tile = (size_t)kTile * 33 * 8;
  const size_t staged = (size_t)a.nb * 3 * 1024;
  if (narrow && a.nb <= kSkinnyWaves * kGateUpStage)
    hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kGateUpDepth, 2, true, kGateUpStage>), grid,
                       dim3(64 * kSkinnyWaves * 2), staged > h_tile ? staged : h_tile, s, a);
  else if (narrow)
    hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kGateUpDepth, 2, true>), grid, dim3(64 * kSkinnyWaves * 2),
                       h_tile, s, a);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<3, kSkinnyWaves, kSkinnyDepth, 2, false>), grid, dim3(64 * kSkinnyWaves * 2),
                       0, s, a);
  return hipGetLastError();
}

}  // namespace ei

namespace ei {

// ================================================================ finishing down projection, 16 x 16 tiles
// The down projection of an FFN layer at up to 32 tokens, without a split of
// K across workgroups, so that no combiner launch follows it.  A 32-row tile
// gives too few workgroups (28 for 896 rows) to pull the weights, so this
// kernel works on 16-row x 16-token tiles with v_mfma_i32_16x16x32_i8 (lane
// l holds A[l % 16][8 (l / 16) .. +7] of the 16 x 32 limb operand,
// B[8 (l / 16) .. +7][l % 16] of the 32 x 16 code operand and D[4 (l / 16) +
// i][l % 16] of the result): 56 x 2 workgroups for 896 rows and 30 tokens.
// The operands are read straight from the 1 KB tiles of the 32 x 32 layout
// (an 8-byte piece of a lane's 16 bytes there).  The W waves of a workgroup
// split the K blocks; each wave requests all of its blocks at once (past its
// range the loads point outside the buffers and read nothing), accumulates
// the narrow form's two chains, and the waves' int64 totals meet in LDS.  One
// thread per output then forms y = resid + floor((acc + 2^23) / 2^24) and, if
// asked, y's balanced base-256 digits as the next layer's limb tiles (tile
// (l, token / 32, row / 32), lane (token % 32) + 32 ((row % 32) / 16), byte
// row % 16) -- the work of the split-K combiner.  Narrow scales only.
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
constexpr int kF16Waves = 16;
constexpr int kF16MaxBlocks = 10;   // blocks per wave at most (K <= 16 x 10 x 32 = 5,120)

// MB: blocks per wave at most (the launch takes the smallest instance that
// holds ceil(nb / W)); every slot is computed, past cnt with scale 0, so the
// loop has no branch for the compiler to wait around
template <int MB>
__global__ __launch_bounds__(64 * kF16Waves) void skinny16_finish_kernel(GemmArgs a) {
  constexpr int W = kF16Waves;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rt = blockIdx.x, th = blockIdx.y;   // 16-row tile, 16-token half
  const int64_t rg = rt >> 1, rh = rt & 1;           // its 32-row group and half
  const int64_t nb = a.nb, tgs = a.t_pad / kTile;
  const int64_t w0 = wave * nb / W, cnt = (wave + 1) * nb / W - w0;   // cnt <= MB (checked on the host)
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + rg * nb * 1024, (uint32_t)(nb * 1024));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + rg * nb * 32, (uint32_t)(nb * 128));
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.limb_tiles, (uint32_t)(3 * tgs * nb * 1024));
  const int vo_end = (int)(3 * tgs * nb * 1024);   // at or past the end of all three ranges
  const int q = lane >> 4;
  // token 16 th + lane % 16 of the 32-token tile th / 2, k piece q
  const int64_t tg = th >> 1;
  const int vo_limb = (int)(((16 * (th & 1) + (lane & 15)) + 32 * (q >> 1)) * 16 + 8 * (q & 1));
  const int vo_code = (int)(((16 * rh + (lane & 15)) + 32 * (q >> 1)) * 16 + 8 * (q & 1));
  const int vo_scale = (int)((16 * rh + (lane & 15)) * 4);

  // the residual of this thread's output (threads 0-255, one output each),
  // requested first so that the epilogue does not wait for it
  const int tl = (threadIdx.x >> 4) & 15, rl16 = threadIdx.x & 15;   // token tl of the half, row rl16 of the tile
  const int64_t tok = 16 * th + tl, row = 16 * rt + rl16;
  const bool mine = threadIdx.x < 256 && tok < a.t && row < a.n;
  const int64_t resid = mine ? a.resid[tok * a.n + row] : 0;
  int64_t code[MB], d[MB][3];
  int32_t S[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const bool live = u < cnt;
    const int b = live ? (int)(w0 + u) : 0;
    // default cache policy: both token halves' workgroups read these pieces
    // (24-layer chain 0.389 ms against 0.432 ms with non-temporal loads)
    const v2u c2 = __builtin_amdgcn_raw_buffer_load_b64(rc, live ? vo_code : vo_end, b * 1024, 0);
    code[u] = (int64_t)(((uint64_t)c2[1] << 32) | c2[0]);
    S[u] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, live ? vo_scale : vo_end, b * 128, 0);
#pragma unroll
    for (int l = 0; l < 3; ++l) {
      const v2u d2 = __builtin_amdgcn_raw_buffer_load_b64(rl, live ? vo_limb : vo_end,
                                                           (int)(((l * tgs + tg) * nb + b) * 1024), 0);
      d[u][l] = (int64_t)(((uint64_t)d2[1] << 32) | d2[0]);
    }
    __builtin_amdgcn_sched_barrier(0);   // requests in block order: block u is waited for alone
  }
  int64_t acc0[4] = {0, 0, 0, 0}, acc1[4] = {0, 0, 0, 0};
  const v4i zero = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int32_t Su = u < cnt ? S[u] : 0;
    v4i c = __builtin_amdgcn_mfma_i32_16x16x32_i8(d[u][1], code[u], zero, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = (int)((uint32_t)c[i] << 8);
    const v4i P01 = __builtin_amdgcn_mfma_i32_16x16x32_i8(d[u][0], code[u], c, 0, 0, 0);   // P_0 + 2^8 P_1
    const v4i P2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(d[u][2], code[u], zero, 0, 0, 0);
    const int32_t S16 = (int32_t)((uint32_t)Su << 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc0[i] += (int64_t)Su * P01[i];
      acc1[i] += (int64_t)S16 * P2[i];
    }
  }

  // the waves' totals (each a sum over a subset of blocks: |.| < 2^62.01)
  __shared__ int64_t red[W][4][64];
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc0[i] + acc1[i];
  __syncthreads();
  if (!mine) return;
  const int src_lane = rl16 + 16 * (tl >> 2), src_i = tl & 3;
  int64_t v = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) v += red[w][src_i][src_lane];
  const int64_t e = tok * a.n + row;
  int64_t out;
  bool ok = fit_i64((__int128)resid + ((v + ((int64_t)1 << 23)) >> 24), &out);   // |v| < 2^62.01: no overflow
  a.y[e] = out;
  if (a.limb_out) {
    // balanced digits: the bytes of out + 0x808080, each less 0x80
    const uint64_t u = (uint64_t)out + 0x808080u;
    if (u >> 24) flag(a.status, EI_DEV_LIMB_RANGE);
    const int64_t nbo = a.n / 32, lane16 = (tok % 32) + 32 * ((row % 32) / 16);
#pragma unroll
    for (int l = 0; l < 3; ++l)
      a.limb_out[((((int64_t)l * tgs + tg) * nbo + row / 32) * 64 + lane16) * 16 + (row % 16)] =
          (int8_t)(((u >> (8 * l)) & 0xFF) ^ 0x80);
  }
  if (!ok) flag(a.status, EI_DEV_OUT_RANGE);
}

bool skinny16_finish_fits(int64_t n, int64_t nb, int64_t t) {
  return n % 32 == 0 && t <= 2 * kTile && nb <= (int64_t)kF16Waves * kF16MaxBlocks && nb >= kF16Waves;
}

hipError_t launch_skinny16_finish(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n / 16), (unsigned)((a.t + 15) / 16)), block(64 * kF16Waves);
  const int64_t per = (a.nb + kF16Waves - 1) / kF16Waves;   // blocks of the busiest wave
  if (per <= 4)
    hipLaunchKernelGGL(skinny16_finish_kernel<4>, grid, block, 0, s, a);
  else if (per <= 6)
    hipLaunchKernelGGL(skinny16_finish_kernel<6>, grid, block, 0, s, a);
  else if (per <= 8)
    hipLaunchKernelGGL(skinny16_finish_kernel<8>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(skinny16_finish_kernel<kF16MaxBlocks>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ei
