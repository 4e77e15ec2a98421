// RMSNorms either side of the MoE layer (the sandwich block of AFMoE, mlxcel
// issue #845 "What the original body missed": out = h + post_mlp_norm(
// mlp(pre_mlp_norm(h)))):
//
//   rmsnorm_kernel:      y[t] = x[t] * r_t * (w + off),
//                        r_t = 1 / sqrt(sum_i x[t,i]^2 / H + eps)
//   combine_norm_kernel: v[t] = acc[t] (+ sum_j topk_w[t,j] * y_perm[row_pos[t*k+j]]
//                        in j order), or v[t] from the fused decode FFN's partial
//                        planes (moe_parts.h), then
//                        out[t] = residual[t] + v[t] * r_t * (w + off)
//
// off = 1 gives the Gemma-style scale of MiniMax-M3 (mlxcel issue #763,
// Norms bullet). One workgroup per row: each thread holds up to MAXCH
// groups of 8 columns in registers, so the row is read once. The sum of
// squares runs in a fixed order (per thread in column order, then a fixed
// butterfly across the wave, then the waves in index order), so results do
// not depend on timing. The layer output v is normalised in fp32 before any
// rounding to the storage dtype.
#include "moe_common.h"
#include "moe_kernels.h"
#include "moe_parts.h"

namespace {

constexpr int MAXCH = 4;    // 8-column groups per thread: H <= 8 * 256 * MAXCH
constexpr int KGROUP = 8;   // gathered rows in flight per thread
constexpr int MAXWAVES = 4;

// Sum over the workgroup, identical on every thread, fixed order.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int m = MOE_WAVE / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  const int wave = threadIdx.x / MOE_WAVE;
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) red[wave] = v;
  __syncthreads();
  const int nw = blockDim.x / MOE_WAVE;
  float s = red[0];
  for (int i = 1; i < nw; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ void load_w8(const float* p, float off, float (&s)[VEC8]) {
  Vec8<float>::load(p, s);
#pragma unroll
  for (int u = 0; u < VEC8; ++u) s[u] += off;
}

template <typename T, int NCH>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const T* __restrict__ x,
                                                      const float* __restrict__ w, float off,
                                                      float eps, float inv_h,
                                                      T* __restrict__ y, int H) {
  __shared__ float red[MAXWAVES];
  const size_t row = (size_t)blockIdx.x * H;
  float v[NCH][VEC8];
  float ss = 0.f;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int c = (ch * blockDim.x + threadIdx.x) * VEC8;
    if (c < H) {
      Vec8<T>::load(x + row + c, v[ch]);
#pragma unroll
      for (int u = 0; u < VEC8; ++u) ss += v[ch][u] * v[ch][u];
    }
  }
  const float r = 1.0f / sqrtf(block_sum(ss, red) * inv_h + eps);
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int c = (ch * blockDim.x + threadIdx.x) * VEC8;
    if (c < H) {
      float s[VEC8];
      load_w8(w + c, off, s);
#pragma unroll
      for (int u = 0; u < VEC8; ++u) v[ch][u] = v[ch][u] * r * s[u];
      Vec8<T>::store(y + row + c, v[ch]);
    }
  }
}

// MODE: 0 acc only, 1 acc + the gathered y_perm rows, 2 the partial planes
template <typename T, int MODE, int NCH>
__global__ void __launch_bounds__(256) combine_norm_kernel(
    const float* __restrict__ acc, const T* __restrict__ y_perm, PartsSrc parts,
    const int32_t* __restrict__ row_pos, const float* __restrict__ topk_w,
    const float* __restrict__ w, float off, float eps, float inv_h, const T* residual, T* out,
    int T_, int H, int k) {
  __shared__ float red[MAXWAVES];
  const size_t t = blockIdx.x;
  const size_t row = t * H;
  float v[NCH][VEC8];
  float ss = 0.f;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int c = (ch * blockDim.x + threadIdx.x) * VEC8;
    if (c < H) {
      if (MODE == 2) parts_value(parts, topk_w, t, c, T_, H, k, v[ch]);
      else Vec8<float>::load(acc + row + c, v[ch]);
      if (MODE == 1) {
        for (int j0 = 0; j0 < k; j0 += KGROUP) {
          // unconditional loads (slots past k re-read the last row, masked
          // by a select), so all of a group's loads are in flight at once
          const int m = min(KGROUP, k - j0);
          int p[KGROUP];
          float wj[KGROUP];
#pragma unroll
          for (int j = 0; j < KGROUP; ++j) {
            const size_t r = t * k + j0 + min(j, m - 1);
            p[j] = row_pos[r];
            wj[j] = topk_w[r];
          }
          float yv[KGROUP][VEC8];
#pragma unroll
          for (int j = 0; j < KGROUP; ++j) Vec8<T>::load(y_perm + (size_t)p[j] * H + c, yv[j]);
#pragma unroll
          for (int j = 0; j < KGROUP; ++j)
#pragma unroll
            for (int u = 0; u < VEC8; ++u) v[ch][u] = j < m ? v[ch][u] + wj[j] * yv[j][u] : v[ch][u];
        }
      }
#pragma unroll
      for (int u = 0; u < VEC8; ++u) ss += v[ch][u] * v[ch][u];
    }
  }
  const float r = 1.0f / sqrtf(block_sum(ss, red) * inv_h + eps);
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int c = (ch * blockDim.x + threadIdx.x) * VEC8;
    if (c < H) {
      float s[VEC8], h[VEC8];
      load_w8(w + c, off, s);
      // read before write: out may be the residual buffer itself
      Vec8<T>::load(residual + row + c, h);
#pragma unroll
      for (int u = 0; u < VEC8; ++u) h[u] += v[ch][u] * r * s[u];
      Vec8<T>::store(out + row + c, h);
    }
  }
}

// Threads per row and 8-column groups per thread for a row of H columns.
void row_shape(int H, int* threads, int* nch) {
  const int groups = H / VEC8;
  int nt = groups < 256 ? groups : 256;
  nt = (nt + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
  *threads = nt;
  *nch = (groups + nt - 1) / nt;
}

template <typename T, int NCH>
void rmsnorm_go(const void* x, const float* w, float off, float eps, void* y, int T_, int H,
                int nt, hipStream_t st) {
  hipLaunchKernelGGL((rmsnorm_kernel<T, NCH>), dim3(T_), dim3(nt), 0, st,
                     static_cast<const T*>(x), w, off, eps, 1.0f / (float)H, static_cast<T*>(y),
                     H);
}

// parts.p != NULL: the partial planes (acc and y_perm unused)
template <typename T, int NCH>
void combine_norm_go(const float* acc, const void* y_perm, const PartsSrc& parts,
                     const int32_t* row_pos, const float* topk_w, const float* w, float off,
                     float eps, const void* residual, void* out, int T_, int H, int k, int nt,
                     hipStream_t st) {
  const T* yp = static_cast<const T*>(y_perm);
  const T* res = static_cast<const T*>(residual);
  T* o = static_cast<T*>(out);
  const float inv_h = 1.0f / (float)H;
  if (parts.p)
    hipLaunchKernelGGL((combine_norm_kernel<T, 2, NCH>), dim3(T_), dim3(nt), 0, st, acc, yp,
                       parts, row_pos, topk_w, w, off, eps, inv_h, res, o, T_, H, k);
  else if (y_perm)
    hipLaunchKernelGGL((combine_norm_kernel<T, 1, NCH>), dim3(T_), dim3(nt), 0, st, acc, yp,
                       parts, row_pos, topk_w, w, off, eps, inv_h, res, o, T_, H, k);
  else
    hipLaunchKernelGGL((combine_norm_kernel<T, 0, NCH>), dim3(T_), dim3(nt), 0, st, acc, yp,
                       parts, row_pos, topk_w, w, off, eps, inv_h, res, o, T_, H, k);
}

template <typename T>
void rmsnorm_dispatch(int nch, const void* x, const float* w, float off, float eps, void* y,
                      int T_, int H, int nt, hipStream_t st) {
  switch (nch) {
    case 1: rmsnorm_go<T, 1>(x, w, off, eps, y, T_, H, nt, st); break;
    case 2: rmsnorm_go<T, 2>(x, w, off, eps, y, T_, H, nt, st); break;
    case 3: rmsnorm_go<T, 3>(x, w, off, eps, y, T_, H, nt, st); break;
    default: rmsnorm_go<T, 4>(x, w, off, eps, y, T_, H, nt, st); break;
  }
}

template <typename T>
void combine_norm_dispatch(int nch, const float* acc, const void* y_perm, const PartsSrc& parts,
                           const int32_t* row_pos, const float* topk_w, const float* w,
                           float off, float eps, const void* residual, void* out, int T_, int H,
                           int k, int nt, hipStream_t st) {
  switch (nch) {
    case 1: combine_norm_go<T, 1>(acc, y_perm, parts, row_pos, topk_w, w, off, eps, residual, out, T_, H, k, nt, st); break;
    case 2: combine_norm_go<T, 2>(acc, y_perm, parts, row_pos, topk_w, w, off, eps, residual, out, T_, H, k, nt, st); break;
    case 3: combine_norm_go<T, 3>(acc, y_perm, parts, row_pos, topk_w, w, off, eps, residual, out, T_, H, k, nt, st); break;
    default: combine_norm_go<T, 4>(acc, y_perm, parts, row_pos, topk_w, w, off, eps, residual, out, T_, H, k, nt, st); break;
  }
}

}  // namespace

bool norm_fits(int H) { return H % 64 == 0 && H > 0 && H <= VEC8 * 256 * MAXCH; }

hipError_t launch_rmsnorm(const void* x, const float* w, int add_one, float eps, void* y, int T,
                          int H, int dtype, hipStream_t st) {
  if (!norm_fits(H) || T <= 0) return hipErrorInvalidValue;
  int nt, nch;
  row_shape(H, &nt, &nch);
  const float off = add_one ? 1.0f : 0.0f;
  if (dtype == MOE_BF16)
    rmsnorm_dispatch<bf16_t>(nch, x, w, off, eps, y, T, H, nt, st);
  else
    rmsnorm_dispatch<float>(nch, x, w, off, eps, y, T, H, nt, st);
  return hipGetLastError();
}

static hipError_t combine_norm_any(const float* acc, const void* y_perm, const PartsSrc& parts,
                                   const int32_t* row_pos, const float* topk_w, const float* w,
                                   int add_one, float eps, const void* residual, void* out, int T,
                                   int H, int k, int dtype, hipStream_t st) {
  if (!norm_fits(H) || T <= 0) return hipErrorInvalidValue;
  int nt, nch;
  row_shape(H, &nt, &nch);
  const float off = add_one ? 1.0f : 0.0f;
  if (dtype == MOE_BF16)
    combine_norm_dispatch<bf16_t>(nch, acc, y_perm, parts, row_pos, topk_w, w, off, eps,
                                  residual, out, T, H, k, nt, st);
  else
    combine_norm_dispatch<float>(nch, acc, y_perm, parts, row_pos, topk_w, w, off, eps, residual,
                                 out, T, H, k, nt, st);
  return hipGetLastError();
}

hipError_t launch_combine_norm(const float* acc, const void* y_perm, const int32_t* row_pos,
                               const float* topk_w, const float* w, int add_one, float eps,
                               const void* residual, void* out, int T, int H, int k, int dtype,
                               hipStream_t st) {
  return combine_norm_any(acc, y_perm, PartsSrc{nullptr, 0, 0, 0}, row_pos, topk_w, w, add_one,
                          eps, residual, out, T, H, k, dtype, st);
}

hipError_t launch_combine_norm_parts(const PartsSrc& parts, const float* topk_w, const float* w,
                                     int add_one, float eps, const void* residual, void* out,
                                     int T, int H, int k, int dtype, hipStream_t st) {
  if (!parts.p) return hipErrorInvalidValue;
  return combine_norm_any(nullptr, nullptr, parts, nullptr, topk_w, w, add_one, eps, residual,
                          out, T, H, k, dtype, st);
}
