// Finalise the layer output from the fp32 accumulator.
//   y_perm == NULL: out[t] = acc[t]                    (routed rows were added
//                                                      by the down projection)
//   y_perm != NULL: out[t] = acc[t] + sum_j w[t,j] * y_perm[row_pos[t*k+j]]
//                   summed in j order, so the result does not depend on timing.
// Each thread handles 8 consecutive columns of one token (H % 64 == 0). The
// k gathered rows are fetched in groups of 8 slots whose loads are all in
// flight together (unconditional loads: a predicated load makes the compiler
// wait for each before the next); the sum still runs slot by slot in j
// order.
#include "moe_common.h"
#include "moe_kernels.h"
#include "moe_parts.h"

namespace {

constexpr int CW = VEC8;   // columns per thread
constexpr int KGROUP = 8;  // gathered rows in flight per thread

template <typename T, bool GATHER>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ acc,
                                                      const T* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_pos,
                                                      const float* __restrict__ topk_w,
                                                      T* __restrict__ out, int T_, int H, int k) {
  const int per_row = H / CW;
  const size_t n = (size_t)T_ * per_row;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / per_row;
    const int c = (int)(i - t * per_row) * CW;
    float v[CW];
    Vec8<float>::load(acc + t * H + c, v);
    if (GATHER) {
      for (int j0 = 0; j0 < k; j0 += KGROUP) {
        // slots past k re-read the last slot's row and are masked by a
        // select: every load is unconditional, so all are in flight at once
        const int m = min(KGROUP, k - j0);
        int p[KGROUP];
        float w[KGROUP];
#pragma unroll
        for (int j = 0; j < KGROUP; ++j) {
          const size_t r = t * k + j0 + min(j, m - 1);
          p[j] = row_pos[r];
          w[j] = topk_w[r];
        }
        float y[KGROUP][CW];
#pragma unroll
        for (int j = 0; j < KGROUP; ++j) Vec8<T>::load(y_perm + (size_t)p[j] * H + c, y[j]);
#pragma unroll
        for (int j = 0; j < KGROUP; ++j)
#pragma unroll
          for (int u = 0; u < CW; ++u) v[u] = j < m ? v[u] + w[j] * y[j][u] : v[u];
      }
    }
    Vec8<T>::store(out + t * H + c, v);
  }
}

// The same from the fused decode FFN's partial planes.
template <typename T>
__global__ void __launch_bounds__(256) combine_parts_kernel(PartsSrc parts,
                                                            const float* __restrict__ topk_w,
                                                            T* __restrict__ out, int T_, int H,
                                                            int k) {
  const int per_row = H / CW;
  const size_t n = (size_t)T_ * per_row;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / per_row;
    const int c = (int)(i - t * per_row) * CW;
    float v[CW];
    parts_value(parts, topk_w, t, c, T_, H, k, v);
    Vec8<T>::store(out + t * H + c, v);
  }
}

}  // namespace

hipError_t launch_combine_parts(const PartsSrc& parts, const float* topk_w, void* out, int T,
                                int H, int k, int dtype, hipStream_t st) {
  const size_t n = (size_t)T * (H / CW);
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 grid((unsigned)blocks), block(256);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_parts_kernel<bf16_t>, grid, block, 0, st, parts, topk_w,
                       static_cast<bf16_t*>(out), T, H, k);
  else
    hipLaunchKernelGGL(combine_parts_kernel<float>, grid, block, 0, st, parts, topk_w,
                       static_cast<float*>(out), T, H, k);
  return hipGetLastError();
}

hipError_t launch_combine(const float* acc, const void* y_perm, const int32_t* row_pos,
                          const float* topk_w, void* out, int T, int H, int k, int dtype,
                          hipStream_t st) {
  const size_t n = (size_t)T * (H / CW);
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 grid((unsigned)blocks), block(256);
  if (dtype == MOE_BF16) {
    if (y_perm)
      hipLaunchKernelGGL((combine_kernel<bf16_t, true>), grid, block, 0, st, acc,
                         static_cast<const bf16_t*>(y_perm), row_pos, topk_w,
                         static_cast<bf16_t*>(out), T, H, k);
    else
      hipLaunchKernelGGL((combine_kernel<bf16_t, false>), grid, block, 0, st, acc,
                         (const bf16_t*)nullptr, row_pos, topk_w, static_cast<bf16_t*>(out), T,
                         H, k);
  } else {
    if (y_perm)
      hipLaunchKernelGGL((combine_kernel<float, true>), grid, block, 0, st, acc,
                         static_cast<const float*>(y_perm), row_pos, topk_w,
                         static_cast<float*>(out), T, H, k);
    else
      hipLaunchKernelGGL((combine_kernel<float, false>), grid, block, 0, st, acc,
                         (const float*)nullptr, row_pos, topk_w, static_cast<float*>(out), T, H,
                         k);
  }
  return hipGetLastError();
}
