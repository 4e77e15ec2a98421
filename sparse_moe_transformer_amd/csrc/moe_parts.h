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

constexpr int PARTS_KGROUP = 8;  // gathered rows in flight per plane

__device__ __forceinline__ void parts_value(const PartsSrc& s, const float* __restrict__ topk_w,
                                            size_t t, int c, int T, int H, int k,
                                            float (&v)[VEC8]) {
  const float* sh = s.p + (size_t)s.nr * s.rows * H;
#pragma unroll
  for (int u = 0; u < VEC8; ++u) v[u] = 0.f;
  if (s.ns > 0) Vec8<float>::load(sh + t * H + c, v);
  for (int a = 1; a < s.ns; ++a) {
    float z[VEC8];
    Vec8<float>::load(sh + ((size_t)a * T + t) * H + c, z);
#pragma unroll
    for (int u = 0; u < VEC8; ++u) v[u] += z[u];
  }
  for (int j0 = 0; j0 < k; j0 += PARTS_KGROUP) {
    const int m = min(PARTS_KGROUP, k - j0);
    const size_t p0 = t * k + j0;  // this group's routed rows p0 .. p0 + m - 1
    float w[PARTS_KGROUP];
#pragma unroll
    for (int j = 0; j < PARTS_KGROUP; ++j) w[j] = j < m ? topk_w[p0 + j] : 0.f;
    float y[PARTS_KGROUP][VEC8];
#pragma unroll
    for (int j = 0; j < PARTS_KGROUP; ++j)
      if (j < m) Vec8<float>::load(s.p + (p0 + j) * H + c, y[j]);
    for (int a = 1; a < s.nr; ++a) {
      const float* pl = s.p + (size_t)a * s.rows * H;
      float z[PARTS_KGROUP][VEC8];
#pragma unroll
      for (int j = 0; j < PARTS_KGROUP; ++j)
        if (j < m) Vec8<float>::load(pl + (p0 + j) * H + c, z[j]);
#pragma unroll
      for (int j = 0; j < PARTS_KGROUP; ++j)
        if (j < m) {
#pragma unroll
          for (int u = 0; u < VEC8; ++u) y[j][u] += z[j][u];
        }
    }
#pragma unroll
    for (int j = 0; j < PARTS_KGROUP; ++j)
      if (j < m) {
#pragma unroll
        for (int u = 0; u < VEC8; ++u) v[u] += w[j] * y[j][u];
      }
  }
}

}  // namespace
