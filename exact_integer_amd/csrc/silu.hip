// SiLU table and the SiLU-gated product ("Vendor-Invariant Integer Inference
// for MindChain: Handshake v0", claims C1 and C4: a committed 65537-entry
// table, Q11 input clamped at +-16, Q16 output; inputs beyond +16 read the end
// entry, so the error there grows as x - 16).
#include "ei_internal.h"

namespace ei {

// lut[k + 32768] = round(silu(k / 2^11) * 2^16), silu(z) = z / (1 + e^-z).
// Evaluated in fp64: every exact value lies at least 5e-6 away from a
// half-integer, far above fp64's error at these magnitudes (< 2^20 * 2^-50),
// so rounding to nearest gives the exact table.
__global__ void silu_lut_kernel(int32_t* lut) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i > 65536) return;
  const double z = (double)(i - 32768) * (1.0 / 2048.0);
  const double v = z / (1.0 + exp(-z)) * 65536.0;
  lut[i] = (int32_t)rint(v);
}

// h = floor(lut[clamp(floor((g + 16) / 32), -32768, 32768) + 32768] * u / 2^16)
__global__ void silu_mul_kernel(const int64_t* __restrict__ g, const int64_t* __restrict__ u,
                                const int32_t* __restrict__ lut, int64_t* __restrict__ h, int64_t n,
                                int32_t* status) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  int64_t v;
  if (!silu_gate(g[e], u[e], lut, &v)) flag(status, EI_DEV_OUT_RANGE);
  h[e] = v;
}

hipError_t launch_silu_lut(int32_t* lut, hipStream_t s) {
  hipLaunchKernelGGL(silu_lut_kernel, dim3((65537 + 255) / 256), dim3(256), 0, s, lut);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const int64_t* g, const int64_t* u, const int32_t* lut, int64_t* h, int64_t n,
                           int32_t* status, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, u, lut, h, n, status);
  return hipGetLastError();
}

}  // namespace ei
