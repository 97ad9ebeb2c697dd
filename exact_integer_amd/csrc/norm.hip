// Requantization and integer RMSNorm ("Deterministic, Reproducible Inference
// in Exact Integer Arithmetic ...", 3.1 arithmetic specification: a scale is
// an integer mantissa m and a shift k, applied as round(c * m / 2^k) with a
// 128-bit product and a round-half-away-from-zero shift; 3.2 Normalization:
// the sum of squares is an exact integer reduction and the per-row
// inverse-RMS an integer inverse square root folded into the scale).
//
// RMSNorm of Q16 codes X with a Q16 weight G and eps in Q32:
//   inv = floor(sqrt(2^104 d / (sum X^2 + d eps)))      (= 2^52 / rms, exact)
//   Y_i = round_half_away(X_i * G_i * inv / 2^52)
// One workgroup per row: the squares are summed in uint64 (|X| <= 2^23 and
// d <= 2^16 keep the sum below 2^63), one thread forms inv from a float64
// estimate corrected to the exact floor with 128-bit integer products, and
// the row is scaled in a second pass.
#include "ei_internal.h"

namespace ei {

constexpr int kRmsShift = 52;
constexpr int kNormThreads = 256;

// round_half_away(p / 2^k) for |p| < 2^127, 0 <= k <= 126; false if the
// result does not fit int64.
__device__ inline bool shift_half_away(__int128 p, int k, int64_t* out) {
  if (k == 0) return fit_i64(p, out);
  const unsigned __int128 a = ((unsigned __int128)(p < 0 ? -p : p) + ((unsigned __int128)1 << (k - 1))) >> k;
  return fit_i64(p < 0 ? -(__int128)a : (__int128)a, out);
}

// floor(sqrt(2^104 d / den)) for 1 <= d <= 2^16 and d <= den < 2^63, i.e.
// the largest z with z^2 den <= 2^104 d (no division: z^2 den is an integer
// and 2^104 d / den >= z^2 iff z^2 den <= 2^104 d).  The root is at most 2^52;
// a float64 estimate is within 2 of it, and near the root z^2 den stays below
// 2^121, so the two correction loops compare exact 128-bit products.
__device__ inline uint64_t rms_inverse(uint64_t ss, int64_t d, int64_t eps) {
  const uint64_t den = ss + (uint64_t)d * (uint64_t)eps;
  const unsigned __int128 lim = (unsigned __int128)(uint64_t)d << 104;
  uint64_t z = (uint64_t)(sqrt((double)d / (double)den) * 4503599627370496.0);   // 2^52
  auto above = [&](uint64_t v) { return (unsigned __int128)v * v * den > lim; };
  while (z > 0 && above(z)) --z;
  while (!above(z + 1)) ++z;
  return z;
}

// kTiles: the normalized row goes out as 3-limb activation tiles for the MFMA
// kernels ([3][t_pad/32][d/32][64 lanes][16 B]; d a multiple of 32), with
// rows t .. t_pad-1 of the last token tile written as zeros; otherwise as
// int64 y [t][d].
template <bool kTiles>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_q16_kernel(const int64_t* __restrict__ x,
                                                                  const int32_t* __restrict__ g, int64_t eps,
                                                                  int64_t* __restrict__ y, int8_t* __restrict__ tiles,
                                                                  int64_t t, int64_t t_pad, int64_t d,
                                                                  int32_t* status) {
  __shared__ uint64_t part[kNormThreads / 64];
  __shared__ uint64_t inv_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok = blockIdx.x;
  if (kTiles && tok >= t) {   // padding token of the last tile: zero limbs
    const int64_t nb = d / 32, tg = tok / kTile, tgs = t_pad / kTile;
    const int tl = (int)(tok % kTile);
    const v4i z = {0, 0, 0, 0};
    for (int64_t c = tid; c < 2 * nb; c += kNormThreads)
#pragma unroll
      for (int l = 0; l < 3; ++l)
        reinterpret_cast<v4i*>(tiles)[((l * tgs + tg) * nb + c / 2) * 64 + tl + 32 * (c & 1)] = z;
    return;
  }
  const int64_t* row = x + tok * d;
  int64_t* out = kTiles ? nullptr : y + tok * d;
  uint64_t ss = 0;
  bool ok = true;
  for (int64_t i = tid; i < d; i += kNormThreads) {
    const int64_t v = row[i];
    const bool in = v >= -((int64_t)1 << 23) && v <= ((int64_t)1 << 23);
    ok = ok && in;
    ss += in ? (uint64_t)(v * v) : 0;
  }
  if (!ok) flag(status, EI_DEV_LIMB_RANGE);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)ss, o, 64), hi = __shfl_xor((uint32_t)(ss >> 32), o, 64);
    ss += ((uint64_t)hi << 32) | lo;
  }
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    uint64_t tot = 0;
    for (int w = 0; w < kNormThreads / 64; ++w) tot += part[w];
    inv_s = rms_inverse(tot, d, eps);
  }
  __syncthreads();
  const uint64_t inv = inv_s;
  // |X G| <= 2^23 2^31, times inv <= 2^52: below 2^106
  auto scaled = [&](int64_t i, int64_t* v) {
    return shift_half_away((__int128)(row[i] * (int64_t)g[i]) * (__int128)inv, kRmsShift, v);
  };
  if constexpr (!kTiles) {
    for (int64_t i = tid; i < d; i += kNormThreads) {
      int64_t v;
      if (!scaled(i, &v)) flag(status, EI_DEV_OUT_RANGE);
      out[i] = v;
    }
  } else {
    // item i = four consecutive columns 4i .. 4i+3: word i % 4 of the 16-byte
    // piece of lane tok % 32 + 32 (half) in block i / 8, half (i / 4) % 2
    const int64_t nb = d / 32, tg = tok / kTile, tgs = t_pad / kTile;
    const int tl = (int)(tok % kTile);
    bool range_ok = true, fit = true;
    for (int64_t i = tid; i < d / 4; i += kNormThreads) {
      int64_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fit = scaled(4 * i + j, &v[j]) && fit;
      uint32_t w[3];
      range_ok = limb_words<3>(v, w) && range_ok;
      const int64_t lane16 = tl + 32 * ((i >> 2) & 1);
#pragma unroll
      for (int l = 0; l < 3; ++l)
        reinterpret_cast<uint32_t*>(tiles)[(((l * tgs + tg) * nb + (i >> 3)) * 64 + lane16) * 4 + (i & 3)] = w[l];
    }
    if (!fit) flag(status, EI_DEV_OUT_RANGE);
    if (!range_ok) flag(status, EI_DEV_LIMB_RANGE);
  }
}

// The residual stream between two pre-norm layers, in one pass per token:
// y = resid + (the down projection's split-K (h, r) partials, rounded), then
// y's RMSNorm with the next layer's weight g, written as that layer's 3-limb
// activation tiles (layout and padding rows as rmsnorm_q16_kernel<true>).
// Each thread owns groups of four consecutive columns 4i .. 4i+3 in both
// passes, so the second pass re-reads only its own stores of y.
__global__ __launch_bounds__(kNormThreads) void combine_rmsnorm_tiles_kernel(
    const int64_t* __restrict__ part, int nparts, const int64_t* __restrict__ resid, int64_t* __restrict__ y,
    const int32_t* __restrict__ g, int64_t eps, int8_t* __restrict__ tiles, int64_t t, int64_t t_pad, int64_t d,
    int32_t* status) {
  __shared__ uint64_t wsum[kNormThreads / 64];
  __shared__ uint64_t inv_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok = blockIdx.x, nb = d / 32, tg = tok / kTile, tgs = t_pad / kTile;
  const int tl = (int)(tok % kTile);
  if (tok >= t) {   // padding token of the last tile: zero limbs
    const v4i z = {0, 0, 0, 0};
    for (int64_t c = tid; c < 2 * nb; c += kNormThreads)
#pragma unroll
      for (int l = 0; l < 3; ++l)
        reinterpret_cast<v4i*>(tiles)[((l * tgs + tg) * nb + c / 2) * 64 + tl + 32 * (c & 1)] = z;
    return;
  }
  const int64_t tn = t * d;
  int64_t* yrow = y + tok * d;
  const int64_t* rrow = resid + tok * d;
  uint64_t ss = 0;
  bool fit = true, in_range = true;
  for (int64_t i = tid; i < d / 4; i += kNormThreads) {
    int64_t h[4] = {0, 0, 0, 0}, r[4] = {0, 0, 0, 0};
    for (int p0 = 0; p0 < nparts; p0 += 4) {   // four partials' loads in flight (past nparts: the last, not added)
      int64_t vh[4][4], vr[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t p = p0 + q < nparts ? p0 + q : nparts - 1;
        const int64_t* ph = part + 2 * p * tn + tok * d + 4 * i;
        const int64_t* pr = part + (2 * p + 1) * tn + tok * d + 4 * i;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vh[q][j] = ph[j];
          vr[q][j] = pr[j];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (p0 + q < nparts)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            h[j] += vh[q][j];
            r[j] += vr[q][j];
          }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t out;
      fit = finish_hr(h[j], r[j], OUT_ROUND_Q24, &out) && fit;
      fit = fit_i64((__int128)rrow[4 * i + j] + out, &out) && fit;
      yrow[4 * i + j] = out;
      const bool in = out >= -((int64_t)1 << 23) && out <= ((int64_t)1 << 23);
      in_range = in_range && in;
      ss += in ? (uint64_t)(out * out) : 0;
    }
  }
  if (!fit) flag(status, EI_DEV_OUT_RANGE);
  if (!in_range) flag(status, EI_DEV_LIMB_RANGE);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)ss, o, 64), hi = __shfl_xor((uint32_t)(ss >> 32), o, 64);
    ss += ((uint64_t)hi << 32) | lo;
  }
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    uint64_t tot = 0;
    for (int w = 0; w < kNormThreads / 64; ++w) tot += wsum[w];
    inv_s = rms_inverse(tot, d, eps);
  }
  __syncthreads();
  const uint64_t inv = inv_s;
  bool range_ok = true, sfit = true;
  for (int64_t i = tid; i < d / 4; i += kNormThreads) {
    int64_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)   // this thread's own stores of y
      sfit = shift_half_away((__int128)(yrow[4 * i + j] * (int64_t)g[4 * i + j]) * (__int128)inv, kRmsShift, &v[j]) &&
             sfit;
    uint32_t w[3];
    range_ok = limb_words<3>(v, w) && range_ok;
    const int64_t lane16 = tl + 32 * ((i >> 2) & 1);
#pragma unroll
    for (int l = 0; l < 3; ++l)
      reinterpret_cast<uint32_t*>(tiles)[(((l * tgs + tg) * nb + (i >> 3)) * 64 + lane16) * 4 + (i & 3)] = w[l];
  }
  if (!sfit) flag(status, EI_DEV_OUT_RANGE);
  if (!range_ok) flag(status, EI_DEV_LIMB_RANGE);
}

__global__ void requant_kernel(const int64_t* __restrict__ c, int64_t m, int k, int64_t* __restrict__ y, int64_t n,
                               int32_t* status) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  int64_t v;
  if (!shift_half_away((__int128)c[e] * (__int128)m, k, &v)) flag(status, EI_DEV_OUT_RANGE);
  y[e] = v;
}

hipError_t launch_rmsnorm_q16(const int64_t* x, const int32_t* g, int64_t eps, int64_t* y, int64_t t, int64_t d,
                              int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_q16_kernel<false>, dim3((unsigned)t), dim3(kNormThreads), 0, s, x, g, eps, y,
                     (int8_t*)nullptr, t, t, d, status);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_limb_tiles(const int64_t* x, const int32_t* g, int64_t eps, int8_t* tiles, int64_t t,
                                     int64_t t_pad, int64_t d, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_q16_kernel<true>, dim3((unsigned)t_pad), dim3(kNormThreads), 0, s, x, g, eps,
                     (int64_t*)nullptr, tiles, t, t_pad, d, status);
  return hipGetLastError();
}

hipError_t launch_combine_rmsnorm_tiles(const int64_t* part, int nparts, const int64_t* resid, int64_t* y,
                                        const int32_t* g, int64_t eps, int8_t* tiles, int64_t t, int64_t t_pad,
                                        int64_t d, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(combine_rmsnorm_tiles_kernel, dim3((unsigned)t_pad), dim3(kNormThreads), 0, s, part, nparts,
                     resid, y, g, eps, tiles, t, t_pad, d, status);
  return hipGetLastError();
}

hipError_t launch_requant(const int64_t* c, int64_t m, int k, int64_t* y, int64_t n, int32_t* status,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(requant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, c, m, k, y, n, status);
  return hipGetLastError();
}

}  // namespace ei
