// Wide-code exact GEMM ("Deterministic, Reproducible Inference in Exact
// Integer Arithmetic ...", 3.1: weights are integer codes of 12 balanced
// trits, |c| <= 265,720, activations int32 codes; 3.2 Matmul: the i32 x i32
// products are accumulated exactly, no rounding):
//     y[t][i] = sum_j c[i][j] * a[t][j]      (int64)
//
// On gfx950 both operands enter the int8 matrix cores as balanced base-256
// digits: c = sum_m 256^m w_m (3 digits hold -8,421,504 .. 8,355,711) and
// a = sum_l 256^l d_l (4 digits hold -2^31 .. 2,139,062,143 of int32), so
//     y = sum_{m,l} 256^(m+l) sum_j w_m[i][j] d_l[t][j].
// There is no per-block scale, so every digit product accumulates across the
// whole K inside the MFMA (int32 C = D): the 12 products of a 32x32 tile per
// 32-wide block go to 6 accumulators, one per power 256^s, s = m + l.  At most
// 3 products share one, each adding at most 32 * 128 * 128 = 2^19 per block,
// so K <= 32768 keeps every int32 accumulator exact; the 6 are combined once
// per output in int128.  No VALU work per block: the kernel is bound by the
// matrix cores and the operand traffic.
//
// Packed weights: the 256-byte header, then digit tiles
// [n_pad/32][nb][3 digits][64 lanes][16 B] in the v_mfma_i32_32x32x32_i8
// operand lane order (lane l: row l % 32, columns 16 (l / 32) .. + 15).
// Workgroup: 4 waves as 2 row tiles x 2 token tiles (64 rows x 64 tokens);
// per block the 6 weight-digit and 8 activation-digit tiles are copied to
// LDS with direct-to-LDS loads, one block ahead.  (Wave tiles of 2 x 1, 1 x 2
// and 2 x 2 MFMA tiles, which read less LDS per MFMA, measured the same time
// on the 896 x 896, 4096-row shape: LDS traffic is not what bounds it.)
#include "ei_internal.h"

namespace ei {

constexpr int kWideDigits = 3, kWideActLimbs = 4;
constexpr int kWideBlockBytes = 16 * 1024;   // 6 + 8 tiles of 1 KB, 2 KB of padding copies
constexpr int kWideNbuf = 2;                 // one block ahead: measured faster than two (44 vs 47 us)
constexpr int kWideCopiesPerWave = 4;        // 16 copies of 1 KB per block, 4 per wave

// One thread per (row tile, block, lane): 16 codes -> 3 digit words x 4.
__global__ void wide_pack_kernel(const int32_t* __restrict__ codes, int64_t n, int64_t k, int64_t n_pad,
                                 int8_t* __restrict__ tiles, uint32_t* bad) {
  const int64_t nb = k / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (n_pad / 32) * nb * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t b = (gid >> 6) % nb, rg = (gid >> 6) / nb;
  const int64_t row = rg * 32 + (lane & 31);
  uint32_t words[kWideDigits][4];
  bool ok = true;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t v[4] = {0, 0, 0, 0};
    if (row < n) {
      const int32_t* src = codes + row * k + b * 32 + 16 * (lane >> 5) + 4 * q;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = src[j];
    }
    uint32_t w[kWideDigits];
    ok = limb_words<kWideDigits>(v, w) && ok;
#pragma unroll
    for (int m = 0; m < kWideDigits; ++m) words[m][q] = w[m];
  }
  if (!ok) atomicOr(bad, 1u);
#pragma unroll
  for (int m = 0; m < kWideDigits; ++m) {
    const v4i v = {(int)words[m][0], (int)words[m][1], (int)words[m][2], (int)words[m][3]};
    reinterpret_cast<v4i*>(tiles)[((rg * nb + b) * kWideDigits + m) * 64 + lane] = v;
  }
}

__global__ __launch_bounds__(256) void wide_gemm_kernel(const int8_t* __restrict__ wtiles,
                                                        const int8_t* __restrict__ atiles, int64_t* __restrict__ y,
                                                        int64_t n, int64_t t, int64_t n_pad, int64_t t_pad,
                                                        int64_t nb, int32_t* status) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave & 1, wt = wave >> 1;
  const int64_t rgs = n_pad / 32, tgs = t_pad / 32;
  const int64_t tbs = (tgs + 1) / 2;
  const int64_t rb = blockIdx.x / tbs, tb = blockIdx.x % tbs;

  // copy j = wave + 4 i: j < 6 weight digit tile (row tile j / 3, digit j % 3),
  // j < 14 activation digit tile (token tile (j - 6) / 4, limb (j - 6) % 4),
  // else a padding copy of weight tile 0 into the block's spare 2 KB.  Row and
  // token tiles past the matrix re-read the last one (results unused).
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wtiles, (uint32_t)(n_pad * nb * 32 * kWideDigits));
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(atiles, (uint32_t)(kWideActLimbs * t_pad * nb * 32));
  uint32_t soff[kWideCopiesPerWave];
  bool is_w[kWideCopiesPerWave];
  int dst[kWideCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kWideCopiesPerWave; ++i) {
    const int j = wave + 4 * i;
    if (j < 6 || j >= 14) {
      const int jw = j < 6 ? j : 0;
      int64_t rg = 2 * rb + jw / 3;
      rg = rg < rgs ? rg : rgs - 1;
      soff[i] = (uint32_t)((rg * nb * kWideDigits + jw % 3) * 1024);
      is_w[i] = true;
      dst[i] = j < 6 ? j * 1024 : (14 + (j - 14)) * 1024;
    } else {
      const int jj = j - 6;
      int64_t tg = 2 * tb + jj / 4;
      tg = tg < tgs ? tg : tgs - 1;
      soff[i] = (uint32_t)(((int64_t)(jj % 4) * tgs + tg) * nb * 1024);
      is_w[i] = false;
      dst[i] = j * 1024;
    }
  }
  auto issue = [&](int64_t b) {
    uint8_t* blk = lds + (int)(b % kWideNbuf) * kWideBlockBytes;
#pragma unroll
    for (int i = 0; i < kWideCopiesPerWave; ++i)
      copy16_to_lds(is_w[i] ? rw : ra, blk + dst[i], lane * 16,
                    soff[i] + (uint32_t)b * (is_w[i] ? 1024u * kWideDigits : 1024u));
  };

  v16i acc[kWideDigits + kWideActLimbs - 1];
#pragma unroll
  for (int s = 0; s < kWideDigits + kWideActLimbs - 1; ++s) acc[s] = (v16i){};

  for (int64_t b = 0; b < kWideNbuf - 1 && b < nb; ++b) issue(b);
  for (int64_t b = 0; b < nb; ++b) {
    if (b + kWideNbuf - 2 < nb)
      barrier_after_vmcnt<(kWideNbuf - 2) * kWideCopiesPerWave>();
    else
      barrier_after_vmcnt<0>();
    if (b + kWideNbuf - 1 < nb) issue(b + kWideNbuf - 1);
    const uint8_t* blk = lds + (int)(b % kWideNbuf) * kWideBlockBytes;
    v4i w[kWideDigits], d[kWideActLimbs];
#pragma unroll
    for (int m = 0; m < kWideDigits; ++m)
      w[m] = *reinterpret_cast<const v4i*>(blk + (wr * kWideDigits + m) * 1024 + lane * 16);
#pragma unroll
    for (int l = 0; l < kWideActLimbs; ++l)
      d[l] = *reinterpret_cast<const v4i*>(blk + (6 + wt * kWideActLimbs + l) * 1024 + lane * 16);
#pragma unroll
    for (int m = 0; m < kWideDigits; ++m)
#pragma unroll
      for (int l = 0; l < kWideActLimbs; ++l)
        acc[m + l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(d[l], w[m], acc[m + l], 0, 0, 0);
  }

  // D[m = token][n = row]: row lane % 32, token 8(r/4) + 4(lane/32) + r%4
  const int64_t row = (2 * rb + wr) * 32 + (lane & 31);
  if (row >= n) return;
  bool ok = true;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t tok = (2 * tb + wt) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (tok >= t) continue;
    __int128 v = 0;
#pragma unroll
    for (int s = 0; s < kWideDigits + kWideActLimbs - 1; ++s) v += (__int128)acc[s][r] << (8 * s);
    int64_t out;
    ok = fit_i64(v, &out) && ok;
    __builtin_nontemporal_store(out, y + tok * n + row);   // written once, not read here
  }
  if (!ok) flag(status, EI_DEV_OUT_RANGE);
}

hipError_t launch_wide_pack(const int32_t* codes, int64_t n, int64_t k, int64_t n_pad, int8_t* tiles, uint32_t* bad,
                            hipStream_t s) {
  const int64_t threads = (n_pad / 32) * (k / 32) * 64;
  hipLaunchKernelGGL(wide_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, codes, n, k, n_pad,
                     tiles, bad);
  return hipGetLastError();
}

hipError_t launch_wide_gemm(const int8_t* wtiles, const int8_t* atiles, int64_t* y, int64_t n, int64_t t,
                            int64_t n_pad, int64_t t_pad, int64_t nb, int32_t* status, hipStream_t s) {
  const int64_t wgs = ((n_pad / 32 + 1) / 2) * ((t_pad / 32 + 1) / 2);
  hipLaunchKernelGGL(wide_gemm_kernel, dim3((unsigned)wgs), dim3(256), (size_t)kWideNbuf * kWideBlockBytes, s,
                     wtiles, atiles, y, n, t, n_pad, t_pad, nb, status);
  return hipGetLastError();
}

}  // namespace ei
