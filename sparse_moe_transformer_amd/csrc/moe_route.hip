// Routing: one wavefront per token.
//
// The rule (mlxcel #845 "Routing detail"; mlxcel #763 "Architecture
// specification", MoE bullet): sigmoid scores; a per-expert bias is added for
// SELECTION only; the k chosen weights are gathered from the unbiased
// scores, renormalised to sum to one (route_norm) and multiplied by
// route_scale.
//
// The selection key s + b is formed in fp64 from the fp32 logit, so that the
// order of two keys is decided exactly the same way as by a float64
// reference fed the same logits (exactly equal logits give exactly equal
// keys; distinct keys would have to lie within ~1e-16 of each other for the
// last-ulp differences of two exp implementations to matter). Ties go to the
// lower expert index, and the k indices are emitted in selection order.
//
// Lane l holds experts l, l+64, ... (NPL per lane). Each of the k rounds takes
// the lane-local best candidate and reduces (key desc, index asc) across the
// wave with xor shuffles; the winning lane retires its candidate.
#include <float.h>
#include <limits.h>

#include "moe_common.h"
#include "moe_kernels.h"

namespace {

template <int NPL>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int route_norm, float route_scale,
                                                    int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out,
                                                    int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave leaves together
  const float* Lrow = logits + (size_t)t * E;
  double key[NPL], sc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const double s = 1.0 / (1.0 + exp(-(double)Lrow[e]));
      sc[i] = s;
      key[i] = s + (bias ? (double)bias[e] : 0.0);
    } else {
      sc[i] = 0.0;
      key[i] = -DBL_MAX;
    }
  }
  bool live[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) live[i] = (lane + 64 * i) < E;

  double gsum = 0.0, my_g = 0.0;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    double bk = -DBL_MAX, bs = 0.0;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      // candidates are visited in ascending index, so '>' keeps the lowest
      // index among equal keys
      if (live[i] && (bi == INT_MAX || key[i] > bk)) {
        bk = key[i];
        bi = e;
        bs = sc[i];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ok = __shfl_xor(bk, off);
      const int oi = __shfl_xor(bi, off);
      const double os = __shfl_xor(bs, off);
      const bool better = (oi != INT_MAX) && (bi == INT_MAX || ok > bk || (ok == bk && oi < bi));
      if (better) {
        bk = ok;
        bi = oi;
        bs = os;
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i == bi) live[i] = false;
    gsum += bs;  // same order (j = 0..k-1) in every lane
    if (lane == j) {
      my_g = bs;
      my_idx = bi;
    }
  }
  if (lane < k) {
    double w = my_g;
    if (route_norm) w = gsum != 0.0 ? w / gsum : 0.0;
    w *= (double)route_scale;
    idx_out[(size_t)t * k + lane] = my_idx;
    w_out[(size_t)t * k + lane] = (float)w;
    if (counts) atomicAdd(counts + my_idx, 1);
  }
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int route_norm, float route_scale, int32_t* idx, float* w,
                        int32_t* counts, hipStream_t st) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  const int npl = (E + 63) / 64;
#define MOE_ROUTE(N)                                                                        \
  hipLaunchKernelGGL(route_kernel<N>, grid, block, 0, st, logits, bias, T, E, k, route_norm, \
                     route_scale, idx, w, counts)
  if (npl <= 1) MOE_ROUTE(1);
  else if (npl <= 2) MOE_ROUTE(2);
  else if (npl <= 4) MOE_ROUTE(4);
  else if (npl <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}
