// The layer value of a token from the fused decode FFN's fp32 partial
// planes (one plane per 128-column slice of the intermediate width; routed
// planes indexed by routed row t*k + j, shared planes by token):
//   v[t] = sum_a shared_a[t] + sum_j w[t,j] * (sum_c routed_c[t*k+j])
// with every sum in index order (a, then j, and c inside each j), so the
// result does not depend on timing. Shared by the plain and the normalising
// combine; eight consecutive columns per call.
#pragma once

#include "moe_common.h"
#include "moe_kernels.h"

namespace {

constexpr int PARTS_KGROUP = 8;  // routed slots per group of loads

// Every load below is unconditional (slots past k and planes past the count
// re-read a valid row and are then masked by a select), so all of a group's
// loads are in flight at once; predicated loads leave the compiler waiting
// for each one before the next.
__device__ __forceinline__ void parts_value(const PartsSrc& s, const float* __restrict__ topk_w,
                                            size_t t, int c, int T, int H, int k,
                                            float (&v)[VEC8]) {
  const float* sh = s.p + (size_t)s.nr * s.rows * H;
#pragma unroll
  for (int u = 0; u < VEC8; ++u) v[u] = 0.f;
  // shared planes, two at a time, added in plane order
  for (int a0 = 0; a0 < s.ns; a0 += 2) {
    float z0[VEC8], z1[VEC8];
    const bool two = a0 + 1 < s.ns;
    Vec8<float>::load(sh + ((size_t)a0 * T + t) * H + c, z0);
    Vec8<float>::load(sh + ((size_t)(two ? a0 + 1 : a0) * T + t) * H + c, z1);
#pragma unroll
    for (int u = 0; u < VEC8; ++u) {
      v[u] += z0[u];
      v[u] = two ? v[u] + z1[u] : v[u];
    }
  }
  for (int j0 = 0; j0 < k; j0 += PARTS_KGROUP) {
    const int m = min(PARTS_KGROUP, k - j0);
    const size_t p0 = t * k + j0;  // this group's routed rows p0 .. p0 + m - 1
    float w[PARTS_KGROUP];
#pragma unroll
    for (int j = 0; j < PARTS_KGROUP; ++j) w[j] = topk_w[p0 + min(j, m - 1)];
    // y[j] = the row's planes summed in plane order, two planes per round
    float y[PARTS_KGROUP][VEC8];
    for (int c0 = 0; c0 < s.nr; c0 += 2) {
      const bool two = c0 + 1 < s.nr;
      const float* pl0 = s.p + (size_t)c0 * s.rows * H;
      const float* pl1 = s.p + (size_t)(two ? c0 + 1 : c0) * s.rows * H;
      float z0[PARTS_KGROUP][VEC8], z1[PARTS_KGROUP][VEC8];
#pragma unroll
      for (int j = 0; j < PARTS_KGROUP; ++j) {
        const size_t row = p0 + min(j, m - 1);
        Vec8<float>::load(pl0 + row * H + c, z0[j]);
        Vec8<float>::load(pl1 + row * H + c, z1[j]);
      }
#pragma unroll
      for (int j = 0; j < PARTS_KGROUP; ++j)
#pragma unroll
        for (int u = 0; u < VEC8; ++u) {
          const float a = c0 == 0 ? z0[j][u] : y[j][u] + z0[j][u];
          y[j][u] = two ? a + z1[j][u] : a;
        }
    }
#pragma unroll
    for (int j = 0; j < PARTS_KGROUP; ++j)
#pragma unroll
      for (int u = 0; u < VEC8; ++u) v[u] = j < m ? v[u] + w[j] * y[j][u] : v[u];
  }
}

}  // namespace
