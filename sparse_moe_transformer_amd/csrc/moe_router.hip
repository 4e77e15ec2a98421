// Router GEMM: logits[T,E] = x[T,H] . W_r[E,H]^T with fp32 accumulation.
// The router is a bias-free linear layer kept at higher precision than the
// experts (mlxcel #845 "Checkpoint weight layout" and its note on per-tensor
// quantisation overrides: the router gate is stored at more bits).
//
// bf16 activations: the fp32 router weight is split on the fly into three
// bf16 terms hi + mid + lo that represent it exactly; every product of a bf16
// activation with a bf16 term is exact in fp32, so three bf16 MFMAs per tile
// give fp32-accurate logits at bf16 MFMA rate.
// fp32 activations: fp32 MFMA (16x16x4).
//
// One wave computes 32 tokens x 32 experts (2 x 2 blocks of 16x16); a
// workgroup of 4 waves covers 32 tokens x 128 experts.
#include "moe_common.h"
#include "moe_kernels.h"

namespace {

constexpr int RT_M = 32;     // tokens per workgroup
constexpr int RT_N = 128;    // experts per workgroup (32 per wave)

__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16_bits(w);
  float r1 = w - bf16_bits_to_f32(hi);
  mid = f32_to_bf16_bits(r1);
  float r2 = r1 - bf16_bits_to_f32(mid);
  lo = f32_to_bf16_bits(r2);
}

// One K-group of 32*G elements for bf16 x: lane q loads 8*G contiguous
// elements at k0 + q*8*G of its row; sub-chunk i feeds MFMA i. A and B use the
// same (lane group, slot) -> k assignment, so the dot products are exact.
template <int G>
__device__ __forceinline__ void router_group_bf16(const uint16_t* const (&xa)[2],
                                                  const float* const (&wb)[2], int k0, int q,
                                                  floatx4_t (&acc)[2][2]) {
  u32x4_t a[2][G];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < G; ++i)
      a[mb][i] = *reinterpret_cast<const u32x4_t*>(xa[mb] + k0 + q * 8 * G + i * 8);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float* p = wb[nb] + k0 + q * 8 * G + i * 8;
      floatx4_t w0 = *reinterpret_cast<const floatx4_t*>(p);
      floatx4_t w1 = *reinterpret_cast<const floatx4_t*>(p + 4);
      float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      uint16_t hi[8], mid[8], lo[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) split3(wv[v], hi[v], mid[v], lo[v]);
      u32x4_t bh, bm, bl;
      bh.x = hi[0] | ((uint32_t)hi[1] << 16); bh.y = hi[2] | ((uint32_t)hi[3] << 16);
      bh.z = hi[4] | ((uint32_t)hi[5] << 16); bh.w = hi[6] | ((uint32_t)hi[7] << 16);
      bm.x = mid[0] | ((uint32_t)mid[1] << 16); bm.y = mid[2] | ((uint32_t)mid[3] << 16);
      bm.z = mid[4] | ((uint32_t)mid[5] << 16); bm.w = mid[6] | ((uint32_t)mid[7] << 16);
      bl.x = lo[0] | ((uint32_t)lo[1] << 16); bl.y = lo[2] | ((uint32_t)lo[3] << 16);
      bl.z = lo[4] | ((uint32_t)lo[5] << 16); bl.w = lo[6] | ((uint32_t)lo[7] << 16);
      const bf16x8_t Bh = __builtin_bit_cast(bf16x8_t, bh);
      const bf16x8_t Bm = __builtin_bit_cast(bf16x8_t, bm);
      const bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, bl);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a[mb][i]);
        // smallest terms first
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl, acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bm, acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh, acc[mb][nb], 0, 0, 0);
      }
    }
  }
}

__global__ void __launch_bounds__(256) router_bf16_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          float* __restrict__ logits, int T,
                                                          int H, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int t0 = blockIdx.x * RT_M;
  const int e0 = blockIdx.y * RT_N + wave * 32;
  if (e0 >= E) return;
  const uint16_t* xa[2];
  const float* wb[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) xa[mb] = x + (size_t)min(t0 + mb * 16 + r, T - 1) * H;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) wb[nb] = wr + (size_t)min(e0 + nb * 16 + r, E - 1) * H;
  floatx4_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  int k0 = 0;
  for (; k0 + 128 <= H; k0 += 128) router_group_bf16<4>(xa, wb, k0, q, acc);
  for (; k0 < H; k0 += 32) router_group_bf16<1>(xa, wb, k0, q, acc);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + mb * 16 + q * 4 + v;
      if (t >= T) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int e = e0 + nb * 16 + r;
        if (e < E) logits[(size_t)t * E + e] = acc[mb][nb][v];
      }
    }
}

__global__ void __launch_bounds__(256) router_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ wr,
                                                         float* __restrict__ logits, int T,
                                                         int H, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int t0 = blockIdx.x * RT_M;
  const int e0 = blockIdx.y * RT_N + wave * 32;
  if (e0 >= E) return;
  const float* xa[2];
  const float* wb[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) xa[mb] = x + (size_t)min(t0 + mb * 16 + r, T - 1) * H;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) wb[nb] = wr + (size_t)min(e0 + nb * 16 + r, E - 1) * H;
  floatx4_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < H; k0 += 32) {
    float a[2][8], b[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      floatx4_t u0 = *reinterpret_cast<const floatx4_t*>(xa[mb] + k0 + q * 8);
      floatx4_t u1 = *reinterpret_cast<const floatx4_t*>(xa[mb] + k0 + q * 8 + 4);
      a[mb][0] = u0.x; a[mb][1] = u0.y; a[mb][2] = u0.z; a[mb][3] = u0.w;
      a[mb][4] = u1.x; a[mb][5] = u1.y; a[mb][6] = u1.z; a[mb][7] = u1.w;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      floatx4_t u0 = *reinterpret_cast<const floatx4_t*>(wb[nb] + k0 + q * 8);
      floatx4_t u1 = *reinterpret_cast<const floatx4_t*>(wb[nb] + k0 + q * 8 + 4);
      b[nb][0] = u0.x; b[nb][1] = u0.y; b[nb][2] = u0.z; b[nb][3] = u0.w;
      b[nb][4] = u1.x; b[nb][5] = u1.y; b[nb][6] = u1.z; b[nb][7] = u1.w;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int v = 0; v < 8; ++v)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mb][v], b[nb][v], acc[mb][nb], 0, 0, 0);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + mb * 16 + q * 4 + v;
      if (t >= T) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int e = e0 + nb * 16 + r;
        if (e < E) logits[(size_t)t * E + e] = acc[mb][nb][v];
      }
    }
}

}  // namespace

hipError_t launch_router_logits(const void* x, const float* w_router, float* logits, int T,
                                int H, int E, int dtype, hipStream_t st) {
  dim3 grid((T + RT_M - 1) / RT_M, (E + RT_N - 1) / RT_N);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(router_bf16_kernel, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), w_router, logits, T, H, E);
  else
    hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       w_router, logits, T, H, E);
  return hipGetLastError();
}
