// Second derivations by table reads ("D11 integer table serving (UORLUT01)",
// "How it works": "One projection (definition)" and "Products of two runtime
// values").  They compute the same integers as the MFMA projection and the
// SiLU gate by the pages' own multiply-free route, so that two independent
// GPU implementations can be compared bit for bit.
//
// Q4 projection.  For every activation x_j a 16-entry table T_j[q] = q x_j,
// q in [-8, 7], is filled by repeated addition (in LDS, one column per
// thread), and each weight's 4-bit code selects its entry.  A thread owns four
// output rows (the pages' 4-row blocking reuses every table four times); per
// group of 32 columns it sums the table reads and applies the group scale
// m 2^e by shifts and adds (one add per set bit of the 4-bit mantissa, then a
// shift by e).  K is cut into 256-column chunks, one workgroup each, whose
// exact int128 sums a second kernel adds (integer sums: any order gives the
// same result).  Input is the export format itself: nibbles [n][k/2] (element
// 2j in the low nibble of byte j, two's complement) and one scale byte per
// group [n][k/32] (m in the low nibble, e in the high nibble).
//
// Runtime product.  a b = sum_k 16^k T_a[d_k(|b|)] (sign applied after), with
// T_a the sixteen multiples of a built by repeated addition and d_k the
// base-16 digits of |b|; used for the SiLU-gated product lut[idx] * u.
#include "ei_internal.h"

namespace ei {

constexpr int kTabCols = 256;     // columns per table chunk: one chunk per workgroup
constexpr int kTabRows = 4;       // output rows per thread (each table entry read for four rows)
constexpr int kTabThreads = 64;   // one wave: 256 rows per workgroup

// Workgroup (row block, token, K chunk): the chunk's tables, then the exact
// sums of its 4-row blocks.  With one chunk the result goes to y (checked to
// fit int64); otherwise each chunk's int128 sums go to part[chunk][t][n] for
// q4_table_combine_kernel.
__global__ __launch_bounds__(kTabThreads) void q4_table_kernel(const uint8_t* __restrict__ nib,
                                                               const uint8_t* __restrict__ sme,
                                                               const int32_t* __restrict__ x, int64_t* __restrict__ y,
                                                               __int128* __restrict__ part, int64_t n, int64_t k,
                                                               int64_t t, int32_t* status) {
  __shared__ int64_t tab[kTabCols][16];   // tab[j][q + 8] = q * x_j
  const int64_t tok = blockIdx.y, chunk = blockIdx.z, c0 = chunk * kTabCols;
  const int cols = (int)(k - c0 < kTabCols ? k - c0 : kTabCols);   // a multiple of 32
  const int64_t r0 = ((int64_t)blockIdx.x * kTabThreads + threadIdx.x) * kTabRows;
  for (int j = threadIdx.x; j < cols; j += kTabThreads) {
    const int64_t xj = x[tok * k + c0 + j];
    int64_t v = 0;
    tab[j][8] = 0;
    for (int q = 1; q <= 7; ++q) {
      v += xj;
      tab[j][8 + q] = v;
    }
    v = 0;
    for (int q = 1; q <= 8; ++q) {
      v -= xj;
      tab[j][8 - q] = v;
    }
  }
  __syncthreads();
  __int128 acc[kTabRows] = {};
  for (int g = 0; g < cols / 32; ++g) {
#pragma unroll
    for (int rr = 0; rr < kTabRows; ++rr) {
      const int64_t row = r0 + rr;
      if (row >= n) continue;
      const uint8_t* nb = nib + row * (k / 2) + (c0 + 32 * g) / 2;
      int64_t gs = 0;
      for (int jj = 0; jj < 16; ++jj) {   // byte jj: columns 2 jj (low nibble) and 2 jj + 1
        const int b = nb[jj];
        gs += tab[32 * g + 2 * jj][(b & 15) ^ 8];        // code c -> q = c - 16 [c >= 8]; index q + 8 = c ^ 8
        gs += tab[32 * g + 2 * jj + 1][(b >> 4) ^ 8];
      }
      const int sc = sme[row * (k / 32) + (c0 / 32 + g)];
      const int m = sc & 15, e = sc >> 4;
      int64_t mg = 0;
#pragma unroll
      for (int bit = 0; bit < 4; ++bit)
        if ((m >> bit) & 1) mg += gs << bit;
      acc[rr] += (__int128)mg << e;
    }
  }
  bool ok = true;
#pragma unroll
  for (int rr = 0; rr < kTabRows; ++rr) {
    const int64_t row = r0 + rr;
    if (row >= n) continue;
    if (gridDim.z > 1) {
      part[(chunk * t + tok) * n + row] = acc[rr];
    } else {
      int64_t out;
      ok = fit_i64(acc[rr], &out) && ok;
      y[tok * n + row] = out;
    }
  }
  if (!ok) flag(status, EI_DEV_OUT_RANGE);
}

// y[e] = the sum of the chunks' int128 sums, checked to fit int64.
__global__ void q4_table_combine_kernel(const __int128* __restrict__ part, int64_t chunks, int64_t* __restrict__ y,
                                        int64_t tn, int32_t* status) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= tn) return;
  __int128 v = 0;
  for (int64_t c = 0; c < chunks; ++c) v += part[c * tn + e];
  int64_t out;
  if (!fit_i64(v, &out)) flag(status, EI_DEV_OUT_RANGE);
  y[e] = out;
}

size_t q4_table_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  const int64_t chunks = (k + kTabCols - 1) / kTabCols;
  return chunks > 1 ? (size_t)chunks * (size_t)t * (size_t)n * sizeof(__int128) : 0;
}

__global__ __launch_bounds__(256) void silu_mul_radix16_kernel(const int64_t* __restrict__ g,
                                                               const int64_t* __restrict__ u,
                                                               const int32_t* __restrict__ lut,
                                                               int64_t* __restrict__ h, int64_t n, int32_t* status) {
  __shared__ int64_t tab[256][16];   // per thread: the sixteen multiples of its table value
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int64_t gv = g[e];
  int64_t idx = (gv >> 5) + ((gv & 31) >= 16 ? 1 : 0);   // floor((g + 16) / 32)
  idx = idx < -32768 ? -32768 : (idx > 32768 ? 32768 : idx);
  const int64_t a = lut[idx + 32768];
  int64_t v = 0;
  for (int d = 0; d < 16; ++d) {
    tab[threadIdx.x][d] = v;
    v += a;
  }
  const int64_t b = u[e];
  uint64_t mag = b < 0 ? (uint64_t)0 - (uint64_t)b : (uint64_t)b;
  __int128 p = 0;
  for (int dk = 0; dk < 16; ++dk, mag >>= 4) p += (__int128)tab[threadIdx.x][mag & 15] << (4 * dk);
  if (b < 0) p = -p;
  int64_t out;
  if (!fit_i64(p >> 16, &out)) flag(status, EI_DEV_OUT_RANGE);   // arithmetic shift: floor
  h[e] = out;
}

hipError_t launch_q4_table(const uint8_t* nib, const uint8_t* sme, const int32_t* x, int64_t* y, int64_t n,
                           int64_t k, int64_t t, void* workspace, int32_t* status, hipStream_t s) {
  const int64_t per = (int64_t)kTabThreads * kTabRows;
  const int64_t chunks = (k + kTabCols - 1) / kTabCols;
  __int128* part = static_cast<__int128*>(workspace);
  hipLaunchKernelGGL(q4_table_kernel, dim3((unsigned)((n + per - 1) / per), (unsigned)t, (unsigned)chunks),
                     dim3(kTabThreads), 0, s, nib, sme, x, y, part, n, k, t, status);
  if (chunks == 1) return hipGetLastError();
  const int64_t tn = t * n;
  hipLaunchKernelGGL(q4_table_combine_kernel, dim3((unsigned)((tn + 255) / 256)), dim3(256), 0, s, part, chunks, y,
                     tn, status);
  return hipGetLastError();
}

hipError_t launch_silu_mul_radix16(const int64_t* g, const int64_t* u, const int32_t* lut, int64_t* h, int64_t n,
                                   int32_t* status, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_radix16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, u, lut, h, n,
                     status);
  return hipGetLastError();
}

}  // namespace ei
