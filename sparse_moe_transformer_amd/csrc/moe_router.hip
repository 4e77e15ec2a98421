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

// ---------------------------------------------------------------------------
// Tiled bf16 router for prefill-sized batches: workgroup tile 128 tokens x 64
// experts; the three weight planes are 192 weight rows of the tile. K-steps of
// 64 elements (128 bytes per row), three LDS stages filled by direct
// global->LDS loads two steps ahead (the grouped-GEMM pipeline), so each
// plane row is read once per 128 tokens instead of once per 32. Stage rows:
// 0..127 tokens, 128 + 64p + j plane p of expert j; chunk c of row r at
// c ^ ((r >> 1) & 7). Four waves (2x2): wave (wm, wn) owns tokens 64wm..+63 x
// experts 32wn..+31, two 32x32 blocks, three MFMAs (lo, mid, hi) per block and
// sub-step. A workgroup covers K-chunk blockIdx.z; chunks are summed in order.
constexpr int RTT_M = 128, RTT_N = 64, RTT_ROWS = RTT_M + 3 * RTT_N;  // 320
constexpr int RTT_LOADS = RTT_ROWS / 32;  // 10 loads per lane per stage

__device__ __align__(128) uint32_t g_router_zero[32] = {};

__device__ __forceinline__ int rswz(int row) { return (row >> 1) & 7; }

template <int N>
__device__ __forceinline__ void r_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct RTile {
  const char* p[RTT_LOADS];  // this lane's row pointers (+ chunk offset)
  int nk;                    // real K-steps of the chunk
};

__device__ __forceinline__ void rt_issue(const RTile& t, int j, u32x4_t* st) {
  const bool real = j < t.nk;
  const int kb = j * 128;
  const char* z = reinterpret_cast<const char*>(g_router_zero) + (threadIdx.x & 7) * 16;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < RTT_LOADS; ++i)
    __builtin_amdgcn_global_load_lds(real ? t.p[i] + kb : z, st + (w * RTT_LOADS * 8 + i * 8) * 8,
                                     16, 0, 0);
}

__device__ __forceinline__ void rt_compute(const u32x4_t* st, floatx16_t (&acc)[2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 5, r = lane & 31;
  bf16x8_t fa[2][2], fb[2][3];
  auto read = [&](int s, int slot) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = wm * 64 + mb * 32 + r;
      fa[slot][mb] = __builtin_bit_cast(bf16x8_t, st[row * 8 + ((2 * s + q) ^ rswz(row))]);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int row = RTT_M + p * RTT_N + wn * 32 + r;
      fb[slot][p] = __builtin_bit_cast(bf16x8_t, st[row * 8 + ((2 * s + q) ^ rswz(row))]);
    }
  };
  read(0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) read(s + 1, (s + 1) & 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int p = 2; p >= 0; --p)  // smallest terms first
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][mb], fb[s & 1][p], acc[mb],
                                                          0, 0, 0);
  }
  // per sub-step: 6 MFMAs carry the next sub-step's 5 fragment reads and
  // 2-3 of the step's 10 global->LDS loads
  __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s < 3 && i < 5) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if ((i == 1 || i == 4) || (i == 5 && s < 2)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
}

#define RT_STEP(J, SC, SD)                   \
  {                                          \
    r_wait_vmcnt<RTT_LOADS>();               \
    __builtin_amdgcn_s_barrier();            \
    rt_issue(t, J, SD);                      \
    rt_compute(SC, acc);                     \
  }

// grid (ceil(T/128), ceil(E/64), KC); kc_steps K-steps of 64 per chunk
__global__ void __launch_bounds__(256) router_tile_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ planes,
                                                          float* __restrict__ part, int T,
                                                          int H, int E, int kc_steps) {
  __shared__ __align__(16) u32x4_t st0[RTT_ROWS * 8];
  __shared__ __align__(16) u32x4_t st1[RTT_ROWS * 8];
  __shared__ __align__(16) u32x4_t st2[RTT_ROWS * 8];
  const int t0 = blockIdx.x * RTT_M, e0 = blockIdx.y * RTT_N;
  const int k0 = blockIdx.z * kc_steps * 64;
  const size_t plane = (size_t)E * H;
  RTile t;
  t.nk = min(kc_steps, H / 64 - blockIdx.z * kc_steps);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RTT_LOADS; ++i) {
    const int row = w * RTT_LOADS * 8 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ rswz(row);
    const uint16_t* src;
    if (row < RTT_M) {
      src = x + (size_t)min(t0 + row, T - 1) * H;
    } else {
      const int pr = row - RTT_M, p = pr / RTT_N, j = pr % RTT_N;
      src = planes + p * plane + (size_t)min(e0 + j, E - 1) * H;
    }
    t.p[i] = reinterpret_cast<const char*>(src + k0 + chunk * 8);
  }
  const int nk3 = (t.nk + 2) / 3 * 3;
  floatx16_t acc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[mb][v] = 0.f;
  rt_issue(t, 0, st0);
  rt_issue(t, 1, st1);
  for (int j = 0; j < nk3; j += 3) {
    RT_STEP(j + 2, st0, st2)
    RT_STEP(j + 3, st1, st0)
    RT_STEP(j + 4, st2, st1)
  }
  r_wait_vmcnt<0>();
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1, q = lane >> 5, r = lane & 31;
  float* out = part + (size_t)blockIdx.z * T * E;
  const int e = e0 + wn * 32 + r;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tk = t0 + wm * 64 + mb * 32 + (v >> 2) * 8 + q * 4 + (v & 3);
      if (tk < T && e < E) out[(size_t)tk * E + e] = acc[mb][v];
    }
}
#undef RT_STEP

// ---------------------------------------------------------------------------
// Small batches (decode): the fp32 weights are split into hi/mid/lo bf16 in
// registers (the same exact split as the plane kernel) and three MFMAs run per
// sub-step, smallest terms first.

__device__ __forceinline__ void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16_bits(v);
  const float r1 = v - bf16_bits_to_f32(hi);
  mid = f32_to_bf16_bits(r1);
  lo = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mid));
}

// Small batches, one plane per K group: workgroup (tile of 32 tokens x 32
// experts, group g) is one wave that computes the group's 64-element partial
// and stores it to plane g. The planes are summed
// in plane order by the consumer (the routing kernel, or
// router_reduce_kernel), so every logit is the same fixed sequence of fp32
// operations on its token row and expert row (identical router rows give
// identical logit columns). Many single-wave workgroups put every group's
// loads in flight at once.
__global__ void __launch_bounds__(64) router_group_kernel(const uint16_t* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         float* __restrict__ part, int T, int H,
                                                         int E) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 5, r = lane & 31;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32, g = blockIdx.z;
  const int k = g * 64;
  const uint16_t* xa = x + (size_t)min(t0 + r, T - 1) * H + 32 * q + k;
  const float* wb = w + (size_t)min(e0 + r, E - 1) * H + 32 * q + k;
  u32x4_t a[4];
  floatx4_t b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(xa + 8 * i);
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = *reinterpret_cast<const floatx4_t*>(wb + 4 * i);
  floatx16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint16_t h[8], m[8], l[8];
    const float f[8] = {b[2 * i].x, b[2 * i].y, b[2 * i].z, b[2 * i].w,
                        b[2 * i + 1].x, b[2 * i + 1].y, b[2 * i + 1].z, b[2 * i + 1].w};
#pragma unroll
    for (int u = 0; u < 8; ++u) split3(f[u], h[u], m[u], l[u]);
    auto pack = [](const uint16_t (&v)[8]) {
      return u32x4_t{v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                     v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
    };
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a[i]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, pack(l)), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, pack(m)), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, pack(h)), acc, 0, 0, 0);
  }
  // 32x32 MFMA layout: lane l holds rows 8*(v/4) + 4*(l/32) + v%4, column l%32
  float* out = part + (size_t)g * T * E;
  const int e = e0 + r;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + (v >> 2) * 8 + q * 4 + (v & 3);
    if (t < T && e < E) out[(size_t)t * E + e] = acc[v];
  }
}

// MXFP8 router weights (E4M3 codes [E, H], E8M0 scales block-major
// [H/32, E]) -> their exact fp32 values, one element per thread: code
// (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
// subnormal) times 2^(scale - 127), formed as one exact ldexp of the
// integer significand (at least 2^-136: an fp32 value).
__global__ void __launch_bounds__(256) router_dequant_mx_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 float* __restrict__ out, int E,
                                                                 int H) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)E * H) return;
  const int e = (int)(i / H), k = (int)(i % H);
  const uint32_t c = codes[i];
  const int s = scales[(size_t)(k / 32) * E + e];
  const int ef = (c >> 3) & 15, m = c & 7;
  float v = ldexpf((float)(ef == 0 ? m : 8 + m), (ef == 0 ? -9 : ef - 10) + s - 127);
  if ((c & 0x7F) == 0x7F || s == 255) v = __builtin_nanf("");
  out[i] = (c & 0x80) ? -v : v;
}

inline int grid_blocks(size_t n) {
  size_t b = (n + 255) / 256;
  return (int)(b > 4096 ? 4096 : (b ? b : 1));
}

}  // namespace

// The bf16 router plan: the tiled kernel for batches of at least 128 tokens
// (else the per-wave kernel), and the number of K chunks: enough workgroups
// to fill the chip, each chunk a whole number of 64-element steps (at least
// three for the tiled kernel) that divides H.
static bool router_tiled(int64_t T) { return T >= RTT_M; }
static bool router_small(int64_t T, int H) { return T < RTT_M && H / 64 <= ROUTER_MAX_PLANES; }

int router_kchunks(int64_t T, int E, int H, int dtype) {
  if (dtype != MOE_BF16) return 1;
  int kc = 1;
  if (router_tiled(T)) {
    const int64_t tiles = ((T + RTT_M - 1) / RTT_M) * ((E + RTT_N - 1) / RTT_N);
    const int steps = H / 64;
    while (tiles * kc * 2 <= 256 && steps % (2 * kc) == 0 && steps / (2 * kc) >= 3) kc *= 2;
    return kc;
  }
  const int64_t tiles = ((T + RT_M - 1) / RT_M) * ((E + RT_N - 1) / RT_N);
  while (tiles * kc < 512 && H % (2 * kc * RT_KG) == 0) kc *= 2;
  return kc;
}

int router_planes(int64_t T, int H, int dtype) {
  return dtype == MOE_BF16 && router_small(T, H) ? H / 64 : 0;
}

size_t router_ws_bytes(int64_t T, int E, int H, int dtype) {
  if (dtype != MOE_BF16) return 0;
  if (router_small(T, H)) return (size_t)(H / 64) * T * E * 4;
  const int kc = router_kchunks(T, E, H, dtype);
  return (size_t)3 * E * H * 2 + 256 + (kc > 1 ? (size_t)kc * T * E * 4 : 0);
}

hipError_t launch_router_dequant_mx(const uint8_t* codes, const uint8_t* scales, float* out, int E,
                                    int H, hipStream_t st) {
  const size_t n = (size_t)E * H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(router_dequant_mx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     codes, scales, out, E, H);
  return hipGetLastError();
}

hipError_t launch_router_planes(const void* x, const float* w_router, float* part, int T, int H,
                                int E, hipStream_t st) {
  dim3 grid((T + 31) / 32, (E + 31) / 32, H / 64);
  hipLaunchKernelGGL(router_group_kernel, grid, dim3(64), 0, st, static_cast<const uint16_t*>(x),
                     w_router, part, T, H, E);
  return hipGetLastError();
}

// The router GEMM. With `chunks` given, a bf16 batch whose K range is split
// into chunks (at most ROUTER_MAX_PLANES of them) leaves the chunk partials
// [kc, T, E] in the workspace for the consumer to sum in chunk order (the
// routing kernel in the layer), and *chunks / *np say where; otherwise, and
// with *np = 0, the logits are written whole.
static hipError_t router_logits(const void* x, const float* w_router, float* logits, int T, int H,
                                int E, int dtype, void* ws, hipStream_t st, const float** chunks,
                                int* np) {
  if (np) *np = 0;
  if (dtype != MOE_BF16) {
    dim3 grid((T + RT_M - 1) / RT_M, (E + RT_N - 1) / RT_N);
    hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       w_router, logits, T, H, E);
    return hipGetLastError();
  }
  if (router_small(T, H)) {
    // one plane per K group, then their sum in plane order
    float* part = static_cast<float*>(ws);
    const hipError_t e = launch_router_planes(x, w_router, part, T, H, E, st);
    if (e != hipSuccess) return e;
    const size_t m = (size_t)T * E;
    hipLaunchKernelGGL(router_reduce_kernel, dim3(grid_blocks(m)), dim3(256), 0, st, part,
                       H / 64, m, logits);
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
  if (router_tiled(T)) {
    dim3 grid((T + RTT_M - 1) / RTT_M, (E + RTT_N - 1) / RTT_N, kc);
    hipLaunchKernelGGL(router_tile_kernel, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), planes, part, T, H, E, H / 64 / kc);
  } else {
    dim3 grid((T + RT_M - 1) / RT_M, (E + RT_N - 1) / RT_N, kc);
    hipLaunchKernelGGL(router_partial_kernel, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), planes, part, T, H, E, H / kc);
  }
  if (kc > 1 && chunks && kc <= ROUTER_MAX_PLANES) {
    *chunks = part;
    *np = kc;
  } else if (kc > 1) {
    const size_t m = (size_t)T * E;
    hipLaunchKernelGGL(router_reduce_kernel, dim3(grid_blocks(m)), dim3(256), 0, st, part, kc, m,
                       logits);
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, const float* w_router, float* logits, int T,
                                int H, int E, int dtype, void* ws, hipStream_t st) {
  return router_logits(x, w_router, logits, T, H, E, dtype, ws, st, nullptr, nullptr);
}

hipError_t launch_router_chunks(const void* x, const float* w_router, float* logits, int T, int H,
                                int E, int dtype, void* ws, hipStream_t st, const float** planes,
                                int* np) {
  return router_logits(x, w_router, logits, T, H, E, dtype, ws, st, planes, np);
}
