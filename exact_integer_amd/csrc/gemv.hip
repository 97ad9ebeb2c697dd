// Exact block-scaled projection for a few tokens (T <= 4): the HBM-bound GEMV.
//
// For every (token t, row i) it computes the per-limb sums
//     A_l[t][i] = sum_b S[i][b] * P_l[t][i][b],
//     P_l[t][i][b] = sum_{j in b} q[i][j] * d_l[t][j]          (int32, exact)
// with d_l the balanced base-256 limbs of x, then acc = sum_l 2^(8l) A_l in
// int128 and the output rounding.  Each term S * P_l is below 2^31 * 2^19 =
// 2^50 in magnitude, so every partial sum over up to 2^13 blocks is exact in
// int64 and the visiting order of the blocks cannot change a bit.
//
// Work split.  One workgroup of W waves owns one row group (32 rows).  Wave w
// owns a contiguous range of the block positions; lane l holds row l%32 and
// the half-block 16*(l/32) .. +15 of every block it visits, i.e. one 16-byte
// piece of the 1 KB code tile, so every code load of a wave is one fully
// coalesced 1 KB request.  A wave alternates two register batches of D
// blocks of codes and scales: the loads of one batch are in flight while the
// other is consumed.  No load sits under a branch: where a batch runs past
// the wave's blocks its loads point past the end of the buffer and read
// nothing, so the compiler's waits count exactly the requests in flight (with
// the refills under a branch it waited for all of them before every other
// batch: 13.4 against 12.6 us per launch at 14336 x 4096, T = 1, rocprofv3
// medians).
//
// Activations.  Each wave splits the activations of its own block range into
// limbs and parks them in a private slice of LDS ([slot][limb][token][32 B]),
// read back as 16-byte broadcasts (all 32 lanes of a half-wave read the same
// address).  No workgroup barrier separates staging from use: a wave's LDS
// operations complete in order.  Large K is staged in chunks of `a.chunk`
// blocks per wave.  When the first chunk's activations fit two items of four
// per lane (T = 1 up to 16 blocks per wave) they are requested before the
// code tiles, so that their split runs while the code tiles are in flight
// (loads complete in issue order: issued after the codes, they would be
// waited for behind them).
//
// Scales.  In the ascending order a wave's blocks are contiguous, so the
// scales of a chunk (128 B per block) arrive in at most four 1 KB wave loads
// and wait in LDS next to the limbs (the first chunk's are requested before
// the code tiles); the other orders load 128 B per block.
//
// Codes and scales are loaded non-temporal: each byte is read once.
//
// Per block a lane issues one 16-byte code load, L*T 16-byte LDS reads and
// one 4-byte scale read, 4*L*T dot4 and L*T int64 multiply-adds.  The two
// halves of every row are added with a cross-lane swap, the W waves through
// LDS.
#include "ei_internal.h"

namespace ei {

constexpr int kGemvLdsPerWave = 8192;   // bytes of limb staging per wave (upper bound)
constexpr int kGemvScaleLoads = 4;       // 1 KB scale loads per chunk: at most 32 blocks per chunk
// Cache policy of the code and scale loads: non-temporal (nt).  Every weight
// byte is read once per launch, so the lines need not stay in the caches; on
// the 14336 x 4096 matrix at T = 1 this measured 14.3-14.4 us per launch
// against 15.4 us (12 launches in a graph, two interleaved rounds), with the
// codes alone 14.8 us.  The activations, which every workgroup reads, keep the
// default policy.
constexpr int kStream = 2;

template <typename XT>
constexpr bool kIsI32 = sizeof(XT) == 4;   // int32 (4-bit form) activations

// Block visited at position pos: the plain ascending order unless the launch
// is one of the schedule variants (kGeneric).
template <bool kGeneric>
__device__ inline int64_t visit(const GemmArgs& a, int64_t pos) {
  return kGeneric ? block_at(a, pos) : a.b0 + pos;
}

// Limbs of the wave's visits c0 .. c0 + cb - 1 (visit m is block position
// p0 + m) into the wave's LDS slice, slot m - c0.
template <int L, int T, typename XT, bool kGeneric>
__device__ inline bool stage_limbs(const GemmArgs& a, int64_t p0, int64_t c0, int cb, uint8_t* my, int lane) {
  // item e: 4 consecutive activations (group g of 8) of token t at slot s
  const XT* x = static_cast<const XT*>(a.x);
  bool ok = true;
  for (int e = lane; e < cb * T * 8; e += 64) {
    const int g = e & 7, t = (e >> 3) % T, s = (e >> 3) / T;
    const int64_t b = visit<kGeneric>(a, p0 + c0 + s);
    const XT* src = x + (int64_t)t * a.k + b * 32 + 4 * g;
    const int64_t xo = kIsI32<XT> ? a.x_off : 0;   // the two-limb 4-bit form splits x - x_off
    const int64_t v[4] = {(int64_t)src[0] - xo, (int64_t)src[1] - xo, (int64_t)src[2] - xo, (int64_t)src[3] - xo};
    uint32_t w[L];
    ok &= limb_words<L>(v, w);
#pragma unroll
    for (int l = 0; l < L; ++l)
      *reinterpret_cast<uint32_t*>(my + ((s * L + l) * T + t) * 32 + 4 * g) = w[l];
  }
  return ok;
}

// The projection of row group rg of the matrix in `a` by one workgroup of W
// waves.  kGeneric: any block order (descending, permuted) and the
// per-block-term output of the tree schedule; otherwise ascending blocks only.
template <int L, int T, typename XT, int W, int D, bool kGeneric>
__device__ inline void gemv_rows(const GemmArgs& a, int64_t rg, uint8_t* lds) {
  constexpr int kSlot = L * T * 32;                  // LDS bytes of one block's limbs
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nblk = a.b1 - a.b0;
  const int64_t p0 = wave * nblk / W, cnt = (wave + 1) * nblk / W - p0;   // this wave's block positions
  const int chunk = a.chunk;   // a multiple of 2D
  uint8_t* my = lds + (size_t)wave * chunk * kSlot;
  // ascending order: the scales of a chunk's blocks, [slot][32] int32
  uint8_t* mysc = lds + (size_t)W * chunk * kSlot + (size_t)wave * chunk * 128;
  // this row group's code tiles (nb x 1 KB) and scales (nb x 128 B)
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + rg * a.nb * 1024, (uint32_t)(a.nb * 1024));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + rg * a.nb * 32, (uint32_t)(a.nb * 128));
  const int vo_code = lane * 16, vo_scale = (lane & 31) * 4;
  const int64_t row = rg * kTile + (lane & 31);

  int64_t acc[T][L];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int l = 0; l < L; ++l) acc[t][l] = 0;

  // Two register batches of D blocks alternate: while one is consumed the
  // other is in flight.  Every batch is requested, with no branch around the
  // loads (the compiler's own wait tracking would then assume the fewest
  // requests after a load and wait for nearly all of them before each use):
  // a position past the wave's last visit gets a lane offset past the end of
  // the buffer's range, so its load reads nothing (zeros), and it counts with
  // a zero scale.
  v4i qa[D], qb[D];
  int32_t Sa[D], Sb[D];
  const int vo_end = (int)(a.nb * 1024);   // at or past the end of both ranges
  auto load = [&](v4i (&q)[D], int32_t (&S)[D], int64_t m0) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const bool live = m0 + u < cnt;
      const int b = live ? (int)visit<kGeneric>(a, p0 + m0 + u) : 0;
      q[u] = __builtin_amdgcn_raw_buffer_load_b128(rc, live ? vo_code : vo_end, b * 1024, kStream);
      if constexpr (kGeneric) S[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, live ? vo_scale : vo_end, b * 128, kStream);
    }
  };
  auto consume = [&](const v4i (&q)[D], const int32_t (&S)[D], int64_t m0, int64_t c0) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int s = (int)(m0 - c0) + u;   // LDS slot; < chunk because chunk is a multiple of 2D
      int32_t P[T][L];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int l = 0; l < L; ++l) {
          const v4i d = *reinterpret_cast<const v4i*>(my + s * kSlot + (l * T + t) * 32 + 16 * h);
          int p = 0;
          p = __builtin_amdgcn_sdot4(q[u][0], d[0], p, false);
          p = __builtin_amdgcn_sdot4(q[u][1], d[1], p, false);
          p = __builtin_amdgcn_sdot4(q[u][2], d[2], p, false);
          p = __builtin_amdgcn_sdot4(q[u][3], d[3], p, false);
          P[t][l] = p;
        }
      if (kGeneric && a.out_mode == OUT_TERMS) {
        // the per-block term S * P of the whole block: add the other half
        if (m0 + u < cnt) {
          const int64_t b = visit<kGeneric>(a, p0 + m0 + u);
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int l = 0; l < L; ++l) {
              const int32_t other = __shfl_xor(P[t][l], 32);
              if (h == 0 && row < a.n)
                a.part[((b * L + l) * a.t + t) * a.n + row] = (int64_t)S[u] * (int64_t)(P[t][l] + other);
            }
        }
      } else {
        int32_t Sb;
        if constexpr (kGeneric) Sb = S[u];
        else Sb = *reinterpret_cast<const int32_t*>(mysc + (s * 32 + (lane & 31)) * 4);
        const int32_t Su = m0 + u < cnt ? Sb : 0;   // a clamped reload past the end counts zero
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int l = 0; l < L; ++l) acc[t][l] += (int64_t)Su * (int64_t)P[t][l];
      }
    }
  };

  bool ok = true;
  // the first chunk's activations are requested first (at most kXPre items
  // of 4 per lane, held in registers) so that their split can run while the
  // code tiles are in flight; then the first two batches of code tiles
  constexpr int kXPre = 2;
  const int cb0 = (int)(cnt < chunk ? cnt : chunk);
  const bool pre = cb0 * T * 8 <= 64 * kXPre;
  int64_t xv[kXPre][4];
  if (pre) {
    const XT* x = static_cast<const XT*>(a.x);
#pragma unroll
    for (int i = 0; i < kXPre; ++i) {
      const int e = lane + 64 * i;
      if (e < cb0 * T * 8) {
        const int g = e & 7, t = (e >> 3) % T, s = (e >> 3) / T;
        const XT* src = x + (int64_t)t * a.k + visit<kGeneric>(a, p0 + s) * 32 + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[i][j] = (int64_t)src[j] - (kIsI32<XT> ? a.x_off : 0);
      }
    }
  }
  // ascending order: a chunk's scales are cb x 128 contiguous bytes, fetched
  // with at most four 1 KB wave loads and parked in LDS (one 128-byte request
  // per block measured slower); the first chunk's are requested before the
  // code tiles, so that waiting for them leaves the code tiles in flight
  v4i sc[kGemvScaleLoads];
  auto load_scales = [&](int64_t c0, int cb) {
    const int nsl = kGeneric ? 0 : (cb * 128 + 1023) / 1024;
#pragma unroll
    for (int i = 0; i < kGemvScaleLoads; ++i)
      if (i < nsl)
        sc[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, (int)(a.b0 + p0 + c0) * 128 + i * 1024, kStream);
  };
  __builtin_amdgcn_sched_barrier(0);
  if (cnt > 0) {
    load_scales(0, cb0);
    __builtin_amdgcn_sched_barrier(0);
    load(qa, Sa, 0);
    load(qb, Sb, D);
  }
  for (int64_t c0 = 0; c0 < cnt; c0 += chunk) {
    const int cb = (int)(cnt - c0 < chunk ? cnt - c0 : chunk);
    const int nsl = kGeneric ? 0 : (cb * 128 + 1023) / 1024;
    if (c0 > 0) load_scales(c0, cb);
    if (pre && c0 == 0) {
#pragma unroll
      for (int i = 0; i < kXPre; ++i) {
        const int e = lane + 64 * i;
        if (e < cb * T * 8) {
          const int g = e & 7, t = (e >> 3) % T, s = (e >> 3) / T;
          uint32_t w[L];
          ok &= limb_words<L>(xv[i], w);
#pragma unroll
          for (int l = 0; l < L; ++l)
            *reinterpret_cast<uint32_t*>(my + ((s * L + l) * T + t) * 32 + 4 * g) = w[l];
        }
      }
    } else {
      ok &= stage_limbs<L, T, XT, kGeneric>(a, p0, c0, cb, my, lane);
    }
#pragma unroll
    for (int i = 0; i < kGemvScaleLoads; ++i)
      if (i < nsl && lane * 16 + i * 1024 < cb * 128) *reinterpret_cast<v4i*>(mysc + lane * 16 + i * 1024) = sc[i];
    __builtin_amdgcn_wave_barrier();
    // a consumed batch is refilled at once (past the wave's last block the
    // loads read nothing: with the non-temporal policy a re-read of its last
    // block would go back to HBM)
    for (int64_t m = c0; m < c0 + cb; m += 2 * D) {
      consume(qa, Sa, m, c0);
      load(qa, Sa, m + 2 * D);
      consume(qb, Sb, m + D, c0);
      load(qb, Sb, m + 3 * D);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (!ok) flag(a.status, EI_DEV_LIMB_RANGE);
  if (kGeneric && a.out_mode == OUT_TERMS) return;

  // ---- the two halves of every row, then the W waves
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t v = acc[t][l];
      const int lo = __shfl_xor((int)(uint32_t)v, 32), hi = __shfl_xor((int)(v >> 32), 32);
      acc[t][l] = v + (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    }
  // the waves' sums meet in an LDS area of their own, after the limbs and scales
  int64_t* red = reinterpret_cast<int64_t*>(lds + (size_t)W * chunk * (kSlot + 128));   // [W][32][T][L]
  if (lane < 32) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int l = 0; l < L; ++l) red[((wave * 32 + lane) * T + t) * L + l] = acc[t][l];
  }
  __syncthreads();
  if (tid < 32 * T) {
    const int r = tid & 31, t = tid >> 5;
    const int64_t orow = rg * kTile + r;
    if (orow < a.n) {
      int64_t sum[L];
#pragma unroll
      for (int l = 0; l < L; ++l) sum[l] = 0;
      for (int w = 0; w < W; ++w)
#pragma unroll
        for (int l = 0; l < L; ++l) sum[l] += red[((w * 32 + r) * T + t) * L + l];
      if (a.out_mode == OUT_PARTIAL) {
#pragma unroll
        for (int l = 0; l < L; ++l) a.part[(((int64_t)a.part_index * L + l) * a.t + t) * a.n + orow] = sum[l];
      } else {
        __int128 v = a.row_off ? (__int128)a.row_off[orow] : 0;   // the two-limb 4-bit form's R_i
#pragma unroll
        for (int l = 0; l < L; ++l) v += (__int128)sum[l] << (8 * l);
        int64_t out;
        if (!finish_output(v, a.out_mode, &out)) flag(a.status, EI_DEV_OUT_RANGE);
        a.y[(int64_t)t * a.n + orow] = out;
      }
    }
  }
}

template <int L, int T, typename XT, int W, int D, bool kGeneric>
__global__ __launch_bounds__(W * 64) void gemv_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  gemv_rows<L, T, XT, W, D, kGeneric>(a, a.tperm ? a.tperm[blockIdx.x] : blockIdx.x, lds);
}

// Several matrices of the same k against the same activations in one launch:
// workgroup g takes row group g - rg0[m] of matrix m, rg0[m] <= g < rg0[m + 1].
template <int L, int T, int W, int D>
__global__ __launch_bounds__(W * 64) void gemv_multi_kernel(GemmArgs a, GemvMulti mm) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int64_t g = blockIdx.x;
  int m = 0;
  while (m + 1 < mm.count && g >= mm.rg0[m + 1]) ++m;
  GemmArgs b = a;
  b.codes = mm.codes[m];
  b.scales = mm.scales[m];
  b.y = mm.y[m];
  b.n = mm.n[m];
  b.n_pad = mm.n_pad[m];
  gemv_rows<L, T, int64_t, W, D, false>(b, g - mm.rg0[m], lds);
}

// ================================================================ launchers
// Launch shape: W waves per row group, D blocks in flight per wave.
template <int L, int T, int W, int D>
static hipError_t gemv_launch(GemmArgs a, hipStream_t s) {
  constexpr int kSlot = L * T * 32;
  const int64_t nblk = a.b1 - a.b0;
  const int64_t per_wave = ((nblk + W - 1) / W + 2 * D - 1) / (2 * D) * (2 * D);   // up to a multiple of 2D
  int64_t chunk = kGemvLdsPerWave / kSlot / (2 * D) * (2 * D);                      // down to a multiple of 2D
  constexpr int kMaxScaleChunk = kGemvScaleLoads * 1024 / 128 / (2 * D) * (2 * D);
  static_assert(kMaxScaleChunk >= 2 * D, "scale staging holds at least two batches");
  if (chunk > kMaxScaleChunk) chunk = kMaxScaleChunk;
  if (chunk < 2 * D) chunk = 2 * D;
  if (chunk > per_wave) chunk = per_wave;
  a.chunk = (int)chunk;
  const size_t red = (size_t)W * 32 * T * L * 8;
  const size_t lds = (size_t)W * chunk * (kSlot + 128) + red;   // limbs, scales, then the waves' sums
  const dim3 grid((unsigned)(a.n_pad / kTile)), block(W * 64);
  const bool generic = a.order != ORDER_ASC || a.out_mode == OUT_TERMS;
  if (a.x_is_i32) {
    if (generic)
      hipLaunchKernelGGL((gemv_kernel<L, T, int32_t, W, D, true>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((gemv_kernel<L, T, int32_t, W, D, false>), grid, block, lds, s, a);
  } else {
    if (generic)
      hipLaunchKernelGGL((gemv_kernel<L, T, int64_t, W, D, true>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((gemv_kernel<L, T, int64_t, W, D, false>), grid, block, lds, s, a);
  }
  return hipGetLastError();
}

constexpr int kGemvWaves = 8;
constexpr int kGemvDepth = 2;

template <int L, int T, int W, int D>
static hipError_t gemv_multi_launch(GemmArgs a, const GemvMulti& mm, hipStream_t s) {
  constexpr int kSlot = L * T * 32;
  const int64_t nblk = a.b1 - a.b0;
  const int64_t per_wave = ((nblk + W - 1) / W + 2 * D - 1) / (2 * D) * (2 * D);
  int64_t chunk = kGemvLdsPerWave / kSlot / (2 * D) * (2 * D);
  constexpr int kMaxScaleChunk = kGemvScaleLoads * 1024 / 128 / (2 * D) * (2 * D);
  if (chunk > kMaxScaleChunk) chunk = kMaxScaleChunk;
  if (chunk < 2 * D) chunk = 2 * D;
  if (chunk > per_wave) chunk = per_wave;
  a.chunk = (int)chunk;
  const size_t red = (size_t)W * 32 * T * L * 8;
  const size_t lds = (size_t)W * chunk * (kSlot + 128) + red;
  hipLaunchKernelGGL((gemv_multi_kernel<L, T, W, D>), dim3((unsigned)mm.rg0[mm.count]), dim3(W * 64), lds, s, a,
                     mm);
  return hipGetLastError();
}

template <int L>
static hipError_t gemv_multi_l(const GemmArgs& a, const GemvMulti& mm, hipStream_t s) {
  switch (a.t) {
    case 1: return gemv_multi_launch<L, 1, kGemvWaves, kGemvDepth>(a, mm, s);
    case 2: return gemv_multi_launch<L, 2, kGemvWaves, kGemvDepth>(a, mm, s);
    case 3: return gemv_multi_launch<L, 3, kGemvWaves, kGemvDepth>(a, mm, s);
    default: return gemv_multi_launch<L, 4, kGemvWaves, kGemvDepth>(a, mm, s);
  }
}

hipError_t launch_gemv_multi(const GemmArgs& a, const GemvMulti& mm, int limbs, hipStream_t s) {
  switch (limbs) {
    case 1: return gemv_multi_l<1>(a, mm, s);
    case 2: return gemv_multi_l<2>(a, mm, s);
    case 3: return gemv_multi_l<3>(a, mm, s);
    default: return gemv_multi_l<4>(a, mm, s);
  }
}

template <int L>
static hipError_t gemv_l(const GemmArgs& a, hipStream_t s) {
  switch (a.t) {
    case 1: return gemv_launch<L, 1, kGemvWaves, kGemvDepth>(a, s);
    case 2: return gemv_launch<L, 2, kGemvWaves, kGemvDepth>(a, s);
    case 3: return gemv_launch<L, 3, kGemvWaves, kGemvDepth>(a, s);
    default: return gemv_launch<L, 4, kGemvWaves, kGemvDepth>(a, s);
  }
}

hipError_t launch_gemv(const GemmArgs& a, int limbs, hipStream_t s) {
  switch (limbs) {
    case 1: return gemv_l<1>(a, s);
    case 2: return gemv_l<2>(a, s);
    case 3: return gemv_l<3>(a, s);
    default: return gemv_l<4>(a, s);
  }
}

}  // namespace ei
