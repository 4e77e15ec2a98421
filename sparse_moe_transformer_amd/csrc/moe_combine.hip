// Finalise the layer output from the fp32 accumulator.
//   y_perm == NULL: out[t] = acc[t]                    (routed rows were added
//                                                      by the down projection)
//   y_perm != NULL: out[t] = acc[t] + sum_j w[t,j] * y_perm[row_pos[t*k+j]]
//                   summed in j order, so the result does not depend on timing.
// Each thread handles 8 consecutive columns of one token (H % 64 == 0). The
// k gathered rows are fetched in groups of 8 slots whose loads are all in
// flight together; the sum still runs slot by slot in j order.
#include "moe_common.h"
#include "moe_kernels.h"

namespace {

constexpr int CW = 8;      // columns per thread
constexpr int KGROUP = 8;  // gathered rows in flight per thread

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  typedef floatx4_t raw[2];
  static __device__ __forceinline__ void load(const float* p, float (&v)[CW]) {
    const floatx4_t a = *reinterpret_cast<const floatx4_t*>(p);
    const floatx4_t b = *reinterpret_cast<const floatx4_t*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[CW]) {
    *reinterpret_cast<floatx4_t*>(p) = floatx4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4_t*>(p + 4) = floatx4_t{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[CW]) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[CW]) {
    u32x4_t u;
    u.x = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    u.y = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    u.z = f32_to_bf16_bits(v[4]) | ((uint32_t)f32_to_bf16_bits(v[5]) << 16);
    u.w = f32_to_bf16_bits(v[6]) | ((uint32_t)f32_to_bf16_bits(v[7]) << 16);
    *reinterpret_cast<u32x4_t*>(p) = u;
  }
};

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
        const int m = min(KGROUP, k - j0);
        int p[KGROUP];
        float w[KGROUP];
#pragma unroll
        for (int j = 0; j < KGROUP; ++j) {
          p[j] = j < m ? row_pos[t * k + j0 + j] : 0;
          w[j] = j < m ? topk_w[t * k + j0 + j] : 0.f;
        }
        float y[KGROUP][CW];
#pragma unroll
        for (int j = 0; j < KGROUP; ++j)
          if (j < m) Vec8<T>::load(y_perm + (size_t)p[j] * H + c, y[j]);
#pragma unroll
        for (int j = 0; j < KGROUP; ++j)
          if (j < m) {
#pragma unroll
            for (int u = 0; u < CW; ++u) v[u] += w[j] * y[j][u];
          }
      }
    }
    Vec8<T>::store(out + t * H + c, v);
  }
}

}  // namespace

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
