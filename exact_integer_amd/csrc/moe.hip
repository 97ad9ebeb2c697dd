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
constexpr int kMoePer = (int)(kMoeMaxPairs / kMoeSortThreads);   // keys per thread, at most

// Exclusive scans over the workgroup in thread order: a sum of packed
// counters (four 16-bit fields; no field may exceed 65535 in total) and a
// maximum.  wave_tot: LDS scratch of one word per wave.  Two barriers each.
__device__ inline uint64_t block_exclusive_sum(uint64_t v, uint64_t* total, uint64_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint64_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kMoeSortThreads / 64; ++w) {
    base += w < wave ? wave_tot[w] : 0;
    tot += wave_tot[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__device__ inline int64_t block_exclusive_max(int64_t v, uint64_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(inc, d, 64);
    if (lane >= d && u > inc) inc = u;
  }
  int64_t ex = __shfl_up(inc, 1, 64);
  if (lane == 0) ex = -1;
  if (lane == 63) wave_tot[wave] = (uint64_t)inc;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMoeSortThreads / 64; ++w)
    if (w < wave && (int64_t)wave_tot[w] > ex) ex = (int64_t)wave_tot[w];
  __syncthreads();
  return ex;
}

// One workgroup: a stable LSD radix sort of the keys expert * 2^14 + p (two
// bits of the expert field per pass), then segment offsets and the token-tile
// table.  The input is in pair order, so the result is ordered by expert and,
// within an expert, by pair index.  Keys of pairs with an expert outside
// [0, E) become E * 2^14 + p (they sort last and join no tile) and set
// EI_DEV_ROUTE.
//
// Each thread holds a contiguous run of `per` keys in registers; a pass
// counts the run's digits, scans the counts over the workgroup and writes
// every key to its place in its digit's region (a stable 4-way split).
__global__ __launch_bounds__(kMoeSortThreads) void moe_sort_kernel(const int32_t* __restrict__ route, int64_t pairs,
                                                                  int64_t experts, int32_t* __restrict__ sorted_pair,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ tile_expert,
                                                                  int32_t* __restrict__ tile_row0,
                                                                  int32_t* __restrict__ tile_rows,
                                                                  int32_t* __restrict__ ntiles, int32_t* status) {
  extern __shared__ uint32_t keys[];   // per * 1024 keys; positions >= pairs hold all-ones sentinels
  __shared__ uint64_t wave_tot[kMoeSortThreads / 64];
  const int tid = threadIdx.x;
  const int per = (int)((pairs + kMoeSortThreads - 1) / kMoeSortThreads);
  const int r0 = tid * per;
  uint32_t k[kMoePer];
  bool bad = false;
#pragma unroll
  for (int u = 0; u < kMoePer; ++u) {
    k[u] = 0xFFFFFFFFu;
    const int i = r0 + u;
    if (u < per && i < pairs) {
      int64_t e = route[i];
      if (e < 0 || e >= experts) {
        bad = true;
        e = experts;
      }
      k[u] = (uint32_t)(e << 14) | (uint32_t)i;
    }
  }
  if (bad) flag(status, EI_DEV_ROUTE);
  int bits = 0;
  while (((int64_t)1 << bits) <= experts) ++bits;   // expert fields 0 .. E
  for (int bit = 0; bit < bits; bit += 2) {
    const int sh = 14 + bit;
    uint64_t c = 0;
#pragma unroll
    for (int u = 0; u < kMoePer; ++u)
      if (u < per) c += (uint64_t)1 << (16 * ((k[u] >> sh) & 3u));
    uint64_t tot;
    const uint64_t pre = block_exclusive_sum(c, &tot, wave_tot);
    const int t0 = (int)(tot & 0xFFFF), t1 = (int)((tot >> 16) & 0xFFFF), t2 = (int)((tot >> 32) & 0xFFFF);
    int p0 = (int)(pre & 0xFFFF);
    int p1 = t0 + (int)((pre >> 16) & 0xFFFF);
    int p2 = t0 + t1 + (int)((pre >> 32) & 0xFFFF);
    int p3 = t0 + t1 + t2 + (int)(pre >> 48);
#pragma unroll
    for (int u = 0; u < kMoePer; ++u) {
      if (u < per) {
        const uint32_t d = (k[u] >> sh) & 3u;
        const int dst = d == 0 ? p0 : d == 1 ? p1 : d == 2 ? p2 : p3;
        keys[dst] = k[u];
        p0 += d == 0;
        p1 += d == 1;
        p2 += d == 2;
        p3 += d == 3;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMoePer; ++u)
      if (u < per) k[u] = keys[r0 + u];
    // the next pass rewrites keys only after its scan's barriers
  }
  // sorted pairs; offsets[e] = first sorted position whose expert is >= e
  for (int i = tid; i <= pairs; i += kMoeSortThreads) {
    const int64_t ei = i < pairs ? (int64_t)(keys[i] >> 14) : experts;
    const int64_t ep = i > 0 ? (int64_t)(keys[i - 1] >> 14) : -1;
    if (i < pairs) sorted_pair[i] = (int32_t)(keys[i] & 0x3FFFu);
    const int64_t hi = ei < experts ? ei : experts;
    for (int64_t e = ep + 1; e <= hi; ++e) offsets[e] = i;
  }
  __syncthreads();   // the offsets are visible to the workgroup
  // Token tiles: expert e's segment [offsets[e], offsets[e+1]) is cut into
  // ceil(count / 32) tiles; tiles are numbered by a scan of the per-expert
  // tile counts (experts in order, 1024 at a time), so they come out in
  // sorted order.
  uint64_t total = 0;
  for (int64_t e0 = 0; e0 < experts; e0 += kMoeSortThreads) {
    const int64_t e = e0 + tid;
    const int64_t beg = e < experts ? offsets[e] : 0;
    const int64_t cnt = e < experts ? offsets[e + 1] - beg : 0;
    const int64_t nt = (cnt + kTile - 1) / kTile;
    uint64_t chunk;
    const int64_t j0 = (int64_t)(total + block_exclusive_sum((uint64_t)nt, &chunk, wave_tot));
    for (int64_t s = 0; s < nt; ++s) {
      const int64_t left = cnt - s * kTile;
      tile_expert[j0 + s] = (int32_t)e;
      tile_row0[j0 + s] = (int32_t)(beg + s * kTile);
      tile_rows[j0 + s] = (int32_t)(left < kTile ? left : kTile);
    }
    total += chunk;
  }
  if (tid == 0) *ntiles = (int32_t)total;
}

// The same grouping for up to kMoeFastExperts experts by a stable counting
// sort.  The pairs are cut into 16 contiguous wave ranges.  A wave ranks its
// keys 64 at a time: lanes with the same bucket (expert, or E for an id
// outside [0, E)) find each other with one ballot per bucket bit, a key's rank
// is the wave's running count of its bucket plus the matching lanes before it,
// and the first lane of each bucket adds the group's size to that count.  A
// scan over the waves per bucket and one over the buckets then place every key:
// position = bucket start + keys of the bucket in earlier waves + rank in its
// wave, which is the order (bucket, pair index).  Five barriers in all, against
// two scans per two-bit pass of the radix sort.
constexpr int kMoeFastExperts = 255;      // buckets 0 .. E fit 8 bits
constexpr int kMoeWaves = kMoeSortThreads / 64;

__global__ __launch_bounds__(kMoeSortThreads) void moe_count_sort_kernel(
    const int32_t* __restrict__ route, int64_t pairs, int64_t experts, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_row0,
    int32_t* __restrict__ tile_rows, int32_t* __restrict__ ntiles, int32_t* status) {
  __shared__ uint16_t rank_of[kMoeMaxPairs];    // rank of pair i among its bucket's keys in its wave range
  __shared__ uint8_t bucket_of[kMoeMaxPairs];
  __shared__ uint16_t cnt[kMoeWaves][256];      // keys per (wave, bucket); then the exclusive base over waves
  __shared__ uint64_t seg[256];                 // (keys, tiles) of bucket b, then their exclusive prefix
  __shared__ uint64_t wave_tot[kMoeWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int nb = (int)experts + 1;               // buckets
  const int per = (int)((pairs + kMoeWaves - 1) / kMoeWaves);   // keys per wave range
  for (int b = lane; b < 256; b += 64) cnt[wave][b] = 0;
  // every key's bucket, all route loads in flight at once
  bool bad = false;
  for (int i = tid; i < pairs; i += kMoeSortThreads) {
    const int32_t e = route[i];
    const int b = (e >= 0 && e < experts) ? e : (int)experts;
    bad |= b == (int)experts;
    bucket_of[i] = (uint8_t)b;
  }
  if (bad) flag(status, EI_DEV_ROUTE);
  __syncthreads();
  const int i0 = wave * per, i1 = (int)(i0 + per < pairs ? i0 + per : pairs);
  const uint64_t lt = ((uint64_t)1 << lane) - 1;
  for (int base = i0; base < i1; base += 64) {
    const int i = base + lane;
    const bool valid = i < i1;
    const int b = valid ? bucket_of[i] : 0;
    uint64_t match = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t ones = __ballot(valid && ((b >> bit) & 1));
      match &= ((b >> bit) & 1) ? ones : ~ones;
    }
    if (valid) {
      const int prior = cnt[wave][b];
      rank_of[i] = (uint16_t)(prior + __popcll(match & lt));
      if ((match & lt) == 0) cnt[wave][b] = (uint16_t)(prior + __popcll(match));   // the bucket's first lane
    }
  }
  __syncthreads();
  // per bucket: exclusive base over the waves, the bucket's total and tile count
  uint64_t v = 0;
  if (tid < 256) {
    int run = 0;
    for (int w = 0; w < kMoeWaves; ++w) {
      const int c = cnt[w][tid];
      cnt[w][tid] = (uint16_t)run;
      run += c;
    }
    const int tiles = tid < experts ? (run + kTile - 1) / kTile : 0;
    v = (uint64_t)run | ((uint64_t)tiles << 32);
  }
  // exclusive scan of (keys, tiles) over the buckets: threads 0 .. 255 are waves 0 .. 3
  uint64_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (tid < 256) {
    uint64_t pre = inc - v;
    for (int w = 0; w < wave; ++w) pre += wave_tot[w];
    seg[tid] = pre;
    if (tid <= experts) offsets[tid] = (int32_t)(pre & 0xFFFFFFFFu);
    if (tid < experts) {
      const int start = (int)(pre & 0xFFFFFFFFu), keys = (int)(v & 0xFFFFFFFFu);
      const int t0 = (int)(pre >> 32), nt = (int)(v >> 32);
      for (int s2 = 0; s2 < nt; ++s2) {
        const int left = keys - s2 * kTile;
        tile_expert[t0 + s2] = tid;
        tile_row0[t0 + s2] = start + s2 * kTile;
        tile_rows[t0 + s2] = left < kTile ? left : kTile;
      }
    }
    if (tid == 0) *ntiles = (int32_t)((wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3]) >> 32);
  }
  __syncthreads();
  for (int i = tid; i < pairs; i += kMoeSortThreads) {
    const int b = bucket_of[i];
    const int w = i / per;
    sorted_pair[(int)(seg[b] & 0xFFFFFFFFu) + cnt[w][b] + rank_of[i]] = i;
  }
  (void)nb;
}

// Limb tiles of the grouped activations.  A workgroup takes one token tile j
// and kGatherBlocks consecutive 32-wide blocks of K.  It reads the tile's 32
// activation rows over those blocks, each a contiguous run of 2 KB (a wave
// takes one row per pass, 32 B per lane, so every load is coalesced), splits
// them into limb bytes in LDS, and then writes each (limb, block) tile in the
// MFMA lane order (lane: row lane % 32, columns 16 (lane / 32) .. + 15 of the
// block) as one contiguous 1 KB store.  Rows past the tile's pairs are zero.
// (Gathering straight into the lane order, one lane per row, spread every load
// over 64 rows: 17 us against 13 us on the OLMoE route, rocprofv3 medians.)
constexpr int kGatherBlocks = 8;
constexpr int kGatherCols = 32 * kGatherBlocks;   // activations per row and workgroup
constexpr int kGatherPitch = kGatherCols + 16;    // LDS row pitch in bytes: the lane-order reads of 32 rows spread over the banks

template <int L>
__global__ __launch_bounds__(256) void grouped_limb_tiles_kernel(const int64_t* __restrict__ x, int64_t k, int topk,
                                                                 const int32_t* __restrict__ sorted_pair,
                                                                 const int32_t* __restrict__ tile_row0,
                                                                 const int32_t* __restrict__ tile_rows,
                                                                 const int32_t* __restrict__ ntiles, int64_t tiles_max,
                                                                 int8_t* __restrict__ tiles, int32_t* status) {
  __shared__ __align__(16) uint8_t digits[L][kTile][kGatherPitch];
  __shared__ int64_t token[kTile];
  const int64_t nb = k / 32, chunks = (nb + kGatherBlocks - 1) / kGatherBlocks;
  const int64_t j = blockIdx.x / chunks, c = blockIdx.x % chunks;
  if (j >= *ntiles) return;   // the whole workgroup, before any barrier
  const int tid = threadIdx.x;
  if (tid < kTile) {
    const int rows = tile_rows[j];
    token[tid] = tid < rows ? sorted_pair[tile_row0[j] + tid] / topk : -1;
  }
  __syncthreads();
  const int64_t col0 = c * kGatherCols;
  const int cols = (int)(k - col0 < kGatherCols ? k - col0 : kGatherCols);   // a multiple of 32
  const int cq = (tid & 63) * 4;   // this lane's 4 activations of the row
  // every pass's loads are issued before any is used (a load under a branch
  // would wait once per pass); a row past the tile's pairs reads x[0 .. 3]
  // and is written as zeros
  int64_t v[kTile / 4][4];
#pragma unroll
  for (int p = 0; p < kTile / 4; ++p) {
    const int64_t r = token[4 * p + (tid >> 6)];
    const int64_t* src = x + (r >= 0 && cq < cols ? r * k + col0 + cq : 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[p][e] = src[e];
  }
  bool ok = true;
#pragma unroll
  for (int p = 0; p < kTile / 4; ++p) {
    const int row = 4 * p + (tid >> 6);
    uint32_t w[L];
    const bool live = token[row] >= 0 && cq < cols;
    ok = (limb_words<L>(v[p], w) || !live) && ok;
#pragma unroll
    for (int l = 0; l < L; ++l) *reinterpret_cast<uint32_t*>(&digits[l][row][cq]) = live ? w[l] : 0u;
  }
  if (!ok) flag(status, EI_DEV_LIMB_RANGE);
  __syncthreads();
  const int lane = tid & 63, nblk = cols / 32;
  for (int t = tid >> 6; t < L * nblk; t += 4) {
    const int l = t / nblk, bl = t % nblk;
    const v4i v = *reinterpret_cast<const v4i*>(&digits[l][lane & 31][bl * 32 + 16 * (lane >> 5)]);
    const int64_t b = c * kGatherBlocks + bl;
    reinterpret_cast<v4i*>(tiles)[(((int64_t)l * tiles_max + j) * nb + b) * 64 + lane] = v;
  }
}

hipError_t launch_moe_sort(const int32_t* route, int64_t pairs, int64_t experts, int32_t* sorted_pair,
                           int32_t* offsets, int32_t* tile_expert, int32_t* tile_row0, int32_t* tile_rows,
                           int32_t* ntiles, int32_t* status, hipStream_t s) {
  if (experts <= kMoeFastExperts && pairs <= kMoeMaxPairs) {
    hipLaunchKernelGGL(moe_count_sort_kernel, dim3(1), dim3(kMoeSortThreads), 0, s, route, pairs, experts,
                       sorted_pair, offsets, tile_expert, tile_row0, tile_rows, ntiles, status);
    return hipGetLastError();
  }
  const int64_t per = (pairs + kMoeSortThreads - 1) / kMoeSortThreads;
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(kMoeSortThreads), (size_t)(per * kMoeSortThreads) * 4, s, route,
                     pairs, experts,
                     sorted_pair, offsets, tile_expert, tile_row0, tile_rows, ntiles, status);
  return hipGetLastError();
}

hipError_t launch_grouped_limb_tiles(const int64_t* x, int64_t k, int topk, const int32_t* sorted_pair,
                                     const int32_t* tile_row0, const int32_t* tile_rows, const int32_t* ntiles,
                                     int64_t tiles_max, int8_t* tiles, int32_t* status, hipStream_t s) {
  const int64_t chunks = (k / 32 + kGatherBlocks - 1) / kGatherBlocks;
  hipLaunchKernelGGL(grouped_limb_tiles_kernel<3>, dim3((unsigned)(tiles_max * chunks)), dim3(256), 0, s, x, k, topk,
                     sorted_pair, tile_row0, tile_rows, ntiles, tiles_max, tiles, status);
  return hipGetLastError();
}

}  // namespace ei
