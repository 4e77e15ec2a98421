// Router GEMM: logits[T,E] = x[T,H] . W_r[E,H]^T with fp32 accumulation.
// The router is a bias-free linear layer kept at higher precision than the
// experts (mlxcel #845 "Checkpoint weight layout" and its note on per-tensor
// quantisation overrides: the router gate is stored at more bits).
//
// bf16 activations: the fp32 router weight is first split into three bf16
// planes hi + mid + lo that represent it exactly; every product of a bf16
// activation with a bf16 plane value is exact in fp32, so three bf16 MFMAs
// per tile give fp32-accurate logits at bf16 MFMA rate. The K range is split
// into KC chunks computed by separate workgroups (enough of them to fill the
// chip at decode sizes); the chunk partials are summed in chunk order, so the
// result is the same on every run and two identical router rows give
// bitwise identical logit columns.
// fp32 activations: fp32 MFMA (16x16x4), one chunk.
#include "moe_common.h"
#include "moe_kernels.h"

typedef float floatx16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int RT_M = 32;   // tokens per workgroup
constexpr int RT_N = 128;  // experts per workgroup (32 per wave)
constexpr int RT_KG = 64;  // K elements per pipeline group

__global__ void __launch_bounds__(256) router_split_kernel(const float* __restrict__ w, size_t n,
                                                           uint16_t* __restrict__ planes) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const float v = w[i];
    const uint16_t hi = f32_to_bf16_bits(v);
    const float r1 = v - bf16_bits_to_f32(hi);
    const uint16_t mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(mid);
    planes[i] = hi;
    planes[n + i] = mid;
    planes[2 * n + i] = f32_to_bf16_bits(r2);
  }
}

// Loads of one K-group (64 elements): lane group q (= lane/32) takes the 32
// contiguous elements k0 + 32q .. +31 of its row; sub-step s of the group
// feeds elements 8s..8s+7 of that run to MFMA s. A and the three B planes use
// the same (lane group, slot) -> k assignment, so the products pair up.
struct RGroup {
  u32x4_t a[4];
  u32x4_t b[3][4];
};

__device__ __forceinline__ void rload(const uint16_t* xa, const uint16_t* const (&wb)[3], int k,
                                      RGroup& g) {
#pragma unroll
  for (int i = 0; i < 4; ++i) g.a[i] = *reinterpret_cast<const u32x4_t*>(xa + k + 8 * i);
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) g.b[p][i] = *reinterpret_cast<const u32x4_t*>(wb[p] + k + 8 * i);
}

__device__ __forceinline__ void rcompute(const RGroup& g, floatx16_t& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, g.a[i]);
    // smallest terms first
#pragma unroll
    for (int p = 2; p >= 0; --p)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, g.b[p][i]),
                                                    acc, 0, 0, 0);
  }
}

// grid (ceil(T/32), ceil(E/128), KC). Each wave: 32 tokens x 32 experts over
// K chunk blockIdx.z (kc_len elements, a multiple of 64).
__global__ void __launch_bounds__(256) router_partial_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ planes,
                                                             float* __restrict__ part, int T,
                                                             int H, int E, int kc_len) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 5, r = lane & 31;
  const int t0 = blockIdx.x * RT_M;
  const int e0 = blockIdx.y * RT_N + wave * 32;
  if (e0 >= E) return;
  const int kbeg = blockIdx.z * kc_len;
  const size_t plane = (size_t)E * H;
  const uint16_t* xa = x + (size_t)min(t0 + r, T - 1) * H + kbeg + 32 * q;
  const size_t wrow = (size_t)min(e0 + r, E - 1) * H + kbeg + 32 * q;
  const uint16_t* wb[3] = {planes + wrow, planes + plane + wrow, planes + 2 * plane + wrow};
  floatx16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int ng = kc_len / RT_KG;
  RGroup g0, g1;
  rload(xa, wb, 0, g0);
  int gi = 0;
  for (; gi + 2 <= ng; gi += 2) {
    rload(xa, wb, (gi + 1) * RT_KG, g1);
    rcompute(g0, acc);
    if (gi + 2 < ng) rload(xa, wb, (gi + 2) * RT_KG, g0);
    rcompute(g1, acc);
  }
  if (gi < ng) rcompute(g0, acc);
  float* out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + (v >> 2) * 8 + q * 4 + (v & 3);
    const int e = e0 + r;
    if (t < T && e < E) out[(size_t)t * E + e] = acc[v];
  }
}

__global__ void __launch_bounds__(256) router_reduce_kernel(const float* __restrict__ part,
                                                            int KC, size_t n,
                                                            float* __restrict__ logits) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    float s = part[i];
    for (int c = 1; c < KC; ++c) s += part[(size_t)c * n + i];
    logits[i] = s;
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

inline int grid_blocks(size_t n) {
  size_t b = (n + 255) / 256;
  return (int)(b > 4096 ? 4096 : (b ? b : 1));
}

}  // namespace

// K chunks of the bf16 router GEMM: enough workgroups to fill the chip, each
// chunk a multiple of 64 elements that divides H.
int router_kchunks(int64_t T, int E, int H, int dtype) {
  if (dtype != MOE_BF16) return 1;
  const int64_t tiles = ((T + RT_M - 1) / RT_M) * ((E + RT_N - 1) / RT_N);
  int kc = 1;
  while (tiles * kc < 512 && H % (2 * kc * RT_KG) == 0) kc *= 2;
  return kc;
}

size_t router_ws_bytes(int64_t T, int E, int H, int dtype) {
  if (dtype != MOE_BF16) return 0;
  const int kc = router_kchunks(T, E, H, dtype);
  return (size_t)3 * E * H * 2 + 256 + (kc > 1 ? (size_t)kc * T * E * 4 : 0);
}

hipError_t launch_router_logits(const void* x, const float* w_router, float* logits, int T,
                                int H, int E, int dtype, void* ws, hipStream_t st) {
  if (dtype != MOE_BF16) {
    dim3 grid((T + RT_M - 1) / RT_M, (E + RT_N - 1) / RT_N);
    hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       w_router, logits, T, H, E);
    return hipGetLastError();
  }
  const int kc = router_kchunks(T, E, H, dtype);
  const size_t n = (size_t)E * H;
  uint16_t* planes = static_cast<uint16_t*>(ws);
  float* part = kc > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                  ((3 * n * 2 + 255) & ~size_t(255)))
                       : logits;
  hipLaunchKernelGGL(router_split_kernel, dim3(grid_blocks(n)), dim3(256), 0, st, w_router, n,
                     planes);
  dim3 grid((T + RT_M - 1) / RT_M, (E + RT_N - 1) / RT_N, kc);
  hipLaunchKernelGGL(router_partial_kernel, grid, dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), planes, part, T, H, E, H / kc);
  if (kc > 1) {
    const size_t m = (size_t)T * E;
    hipLaunchKernelGGL(router_reduce_kernel, dim3(grid_blocks(m)), dim3(256), 0, st, part, kc, m,
                       logits);
  }
  return hipGetLastError();
}
