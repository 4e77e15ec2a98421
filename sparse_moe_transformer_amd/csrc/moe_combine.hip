// Finalise the layer output from the fp32 accumulator.
//   y_perm == NULL: out[t] = acc[t]                    (routed rows were added
//                                                      by the down projection)
//   y_perm != NULL: out[t] = acc[t] + sum_j w[t,j] * y_perm[row_pos[t*k+j]]
//                   summed in j order, so the result does not depend on timing.
// Each thread handles 4 consecutive columns of one token (H % 64 == 0).
#include "moe_common.h"
#include "moe_kernels.h"

namespace {

template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
  floatx4_t u = *reinterpret_cast<const floatx4_t*>(p);
  v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float (&v)[4]) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = bf16_bits_to_f32((uint16_t)(u.x & 0xFFFF));
  v[1] = bf16_bits_to_f32((uint16_t)(u.x >> 16));
  v[2] = bf16_bits_to_f32((uint16_t)(u.y & 0xFFFF));
  v[3] = bf16_bits_to_f32((uint16_t)(u.y >> 16));
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<floatx4_t*>(p) = floatx4_t{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float (&v)[4]) {
  uint2 u;
  u.x = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
  u.y = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

template <typename T, bool GATHER>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ acc,
                                                      const T* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_pos,
                                                      const float* __restrict__ topk_w,
                                                      T* __restrict__ out, int T_, int H, int k) {
  const size_t nq = (size_t)T_ * (H / 4);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / (H / 4);
    const int c = (int)(i - t * (H / 4)) * 4;
    float v[4];
    load4<float>(acc + t * H + c, v);
    if (GATHER) {
      for (int j = 0; j < k; ++j) {
        const float w = topk_w[t * k + j];
        const int p = row_pos[t * k + j];
        float y[4];
        load4<T>(y_perm + (size_t)p * H + c, y);
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] += w * y[u];
      }
    }
    store4<T>(out + t * H + c, v);
  }
}

}  // namespace

hipError_t launch_combine(const float* acc, const void* y_perm, const int32_t* row_pos,
                          const float* topk_w, void* out, int T, int H, int k, int dtype,
                          hipStream_t st) {
  const size_t nq = (size_t)T * (H / 4);
  size_t blocks = (nq + 255) / 256;
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
