// Integer top-k routing ("Deterministic, Reproducible Inference in Exact
// Integer Arithmetic ...", 3.2 "Mixture-of-Experts": the router scores the
// experts in integer, the top-k selection is an integer comparison, ties go to
// the lower expert index).  Slot s of token t receives the expert of rank s in
// the order (score descending, index ascending), so the route is a function
// of the scores alone.
//
// One wave per token.  Lane l holds the scores of experts l, l + 64, ...,
// l + 64 (PER - 1).  Each of the k rounds takes every lane's best expert not
// yet chosen, reduces the 64 candidates with a butterfly of cross-lane swaps
// under the same order (which leaves the winner in every lane), and the owning
// lane marks it taken.
#include "ei_internal.h"

namespace ei {

// (score, index) ahead of (score2, index2) in the routing order; index < 0
// marks "no candidate", which is behind everything.
__device__ inline bool route_ahead(int64_t s, int32_t i, int64_t s2, int32_t i2) {
  if (i < 0) return false;
  if (i2 < 0) return true;
  return s > s2 || (s == s2 && i < i2);
}

template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const int64_t* __restrict__ scores, int64_t t, int64_t e, int k,
                                                   int32_t* __restrict__ route) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;   // one wave per token
  if (tok >= t) return;
  const int64_t* row = scores + tok * e;
  int64_t v[PER];
  uint32_t taken = 0;   // bit u: expert lane + 64 u is chosen (or does not exist)
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t ex = lane + 64 * u;
    v[u] = ex < e ? row[ex] : 0;
    if (ex >= e) taken |= 1u << u;
  }
  for (int s = 0; s < k; ++s) {
    int64_t bs = 0;
    int32_t bi = -1;
    int bu = -1;
#pragma unroll
    for (int u = 0; u < PER; ++u) {   // ascending index within the lane: a tie keeps the first
      if (!(taken & (1u << u)) && route_ahead(v[u], lane + 64 * u, bs, bi)) {
        bs = v[u];
        bi = lane + 64 * u;
        bu = u;
      }
    }
    int64_t ws = bs;
    int32_t wi = bi;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const int lo = __shfl_xor((int)(uint32_t)ws, d, 64), hi = __shfl_xor((int)(ws >> 32), d, 64);
      const int64_t os = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
      const int32_t oi = __shfl_xor(wi, d, 64);
      if (route_ahead(os, oi, ws, wi)) {
        ws = os;
        wi = oi;
      }
    }
    if (bi == wi && bu >= 0) taken |= 1u << bu;   // the owning lane
    if (lane == 0) route[tok * k + s] = wi;
  }
}

hipError_t launch_topk(const int64_t* scores, int64_t t, int64_t e, int k, int32_t* route, hipStream_t s) {
  const dim3 grid((unsigned)((t + 3) / 4)), block(256);
  if (e <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, scores, t, e, k, route);
  else if (e <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, scores, t, e, k, route);
  else if (e <= 1024)
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, scores, t, e, k, route);
  else
    hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, s, scores, t, e, k, route);
  return hipGetLastError();
}

}  // namespace ei
