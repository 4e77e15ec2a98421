// Grouped expert GEMMs on MFMA (gfx950).
//
// Every stacked expert tensor is [out, in] with the reduction dimension
// contiguous (mlxcel #845 "Checkpoint weight layout": pre-stacked
// experts.{gate,up,down}_proj), and the activations are [rows, in], so both
// MFMA operands are read along K in 16-byte chunks.
//
// Workgroup tile: 128 rows x 256 weight rows, K-step of 128 bytes per row
// (64 bf16 or 32 fp32), double-buffered in LDS with an XOR swizzle of the
// 16-byte chunks. Four waves in a 2x2 arrangement; each wave owns 64 rows x
// 128 weight rows = 4 x 8 MFMA blocks of 16x16.
//   gate/up: weight rows 0..127 are gate rows n0.., 128..255 the up rows with
//            the same columns, so each wave holds matching gate and up
//            accumulators and applies the activation in registers.
//   down:    weight rows 0..255 are 256 output columns.
// Rows of a routed tile are the expert's sorted rows; the activation rows are
// gathered straight from x into LDS (token = sorted_row / k).
#include "moe_common.h"
#include "moe_kernels.h"

namespace {

constexpr int BM = 128;    // activation rows per workgroup
constexpr int BR = 256;    // weight rows per workgroup
constexpr int NCH = 8;     // 16-byte chunks per LDS row per K-step
constexpr int NTHR = 256;

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
};
template <>
struct Elem<float> {
  static constexpr int EPC = 4;
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

struct Lds {
  u32x4_t a[2][BM * NCH];
  u32x4_t b[2][BR * NCH];
};

// Per-thread global source pointers for its 4 activation rows and 8 weight
// rows (row = tid/8 + 32*j, chunk = tid%8), null = zero row.
template <typename T>
struct Src {
  const T* a[4];
  const T* b[8];
  int kseg;       // weight K segment length (elements); K-split for shared down
  long bstride;   // elements between weight K segments
};

template <typename T>
__device__ __forceinline__ void load_stage(const Src<T>& s, int kk, long bseg_off,
                                           int koff, u32x4_t (&ra)[4], u32x4_t (&rb)[8]) {
  const int c = threadIdx.x & 7;
  const int eo = c * Elem<T>::EPC;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ra[j] = s.a[j] ? *reinterpret_cast<const u32x4_t*>(s.a[j] + kk + eo) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rb[j] = s.b[j] ? *reinterpret_cast<const u32x4_t*>(s.b[j] + bseg_off + koff + eo)
                   : u32x4_t{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void store_stage(Lds& L, int buf, const u32x4_t (&ra)[4],
                                            const u32x4_t (&rb)[8]) {
  const int c = threadIdx.x & 7;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = r0 + 32 * j;
    L.a[buf][r * NCH + (c ^ swz(r))] = ra[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int r = r0 + 32 * j;
    L.b[buf][r * NCH + (c ^ swz(r))] = rb[j];
  }
}

// Weight row (within the 256-row tile) of block nb of wave wn.
template <bool GATE_UP>
__device__ __forceinline__ int wrow(int wn, int nb) {
  if (GATE_UP) return nb < 4 ? wn * 64 + nb * 16 : 128 + wn * 64 + (nb - 4) * 16;
  return wn * 128 + nb * 16;
}

template <typename T, bool GATE_UP>
__device__ __forceinline__ void compute_stage_impl(const Lds& L, int buf, floatx4_t (&acc)[4][8]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r = lane & 15;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t af[4], bfr[8];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        int row = wm * 64 + mb * 16 + r;
        u32x4_t v = L.a[buf][row * NCH + ((s * 4 + q) ^ swz(row))];
        af[mb] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        int row = wrow<GATE_UP>(wn, nb) + r;
        u32x4_t v = L.b[buf][row * NCH + ((s * 4 + q) ^ swz(row))];
        bfr[nb] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
  } else {
    // fp32: lane q holds k = 8q..8q+7 of the 32-wide step (chunks 2q, 2q+1);
    // 8 MFMA 16x16x4 steps, slot v of A pairs with slot v of B.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      int row = wm * 64 + mb * 16 + r;
      u32x4_t a0 = L.a[buf][row * NCH + ((2 * q) ^ swz(row))];
      u32x4_t a1 = L.a[buf][row * NCH + ((2 * q + 1) ^ swz(row))];
      float av[8] = {__uint_as_float(a0.x), __uint_as_float(a0.y), __uint_as_float(a0.z),
                     __uint_as_float(a0.w), __uint_as_float(a1.x), __uint_as_float(a1.y),
                     __uint_as_float(a1.z), __uint_as_float(a1.w)};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        int brw = wrow<GATE_UP>(wn, nb) + r;
        u32x4_t b0 = L.b[buf][brw * NCH + ((2 * q) ^ swz(brw))];
        u32x4_t b1 = L.b[buf][brw * NCH + ((2 * q + 1) ^ swz(brw))];
        float bv[8] = {__uint_as_float(b0.x), __uint_as_float(b0.y), __uint_as_float(b0.z),
                       __uint_as_float(b0.w), __uint_as_float(b1.x), __uint_as_float(b1.y),
                       __uint_as_float(b1.z), __uint_as_float(b1.w)};
#pragma unroll
        for (int v = 0; v < 8; ++v)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[v], bv[v], acc[mb][nb], 0, 0, 0);
      }
    }
  }
}

// Main loop: acc += A[128 x K] . B[256 x K]^T over the whole K.
template <typename T, bool GATE_UP>
__device__ __forceinline__ void mainloop(Lds& L, const Src<T>& s, int K, floatx4_t (&acc)[4][8]) {
  constexpr int KS = NCH * Elem<T>::EPC;  // elements per K-step
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[4], rb[8];
  long bseg = 0;
  int koff = 0;
  load_stage<T>(s, 0, bseg, koff, ra, rb);
  store_stage(L, 0, ra, rb);
  __syncthreads();
  const int nk = K / KS;
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      koff += KS;
      if (koff == s.kseg) {
        koff = 0;
        bseg += s.bstride;
      }
      load_stage<T>(s, (it + 1) * KS, bseg, koff, ra, rb);
    }
    compute_stage_impl<T, GATE_UP>(L, buf, acc);
    if (more) store_stage(L, buf ^ 1, ra, rb);
    __syncthreads();
  }
}

// Find which expert (and m-tile within it) routed m-slot `slot` belongs to.
// Returns false if the slot is past the last tile. Uses `cum` (E+1 ints of
// LDS): cum[e] = sum_{e'<e} ceil(n_e'/BM).
__device__ bool locate_tile(const int32_t* __restrict__ offsets, int E, int slot, int* cum,
                            int* e_out, int* mt_out) {
  // wave 0 builds the prefix of tile counts
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      int e = e0 + i;
      if (e < E) local += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      int e = e0 + i;
      if (e < E) {
        cum[e] = run;
        run += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
      }
    }
    if (lane == 63) cum[E] = incl;
  }
  __syncthreads();
  if (slot >= cum[E]) return false;
  // largest e with cum[e] <= slot and a non-empty tile range
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= slot) lo = mid;
    else hi = mid - 1;
  }
  // skip empty experts that share the same cum value: the owner is the last
  // e with cum[e] <= slot, which has cum[e+1] > slot, hence is non-empty.
  *e_out = lo;
  *mt_out = slot - cum[lo];
  return true;
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float v) {
  *reinterpret_cast<uint16_t*>(p) = f32_to_bf16_bits(v);
}
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) {
  *p = v;
}

}  // namespace

// ---------------------------------------------------------------------------
// gate/up + activation. Grid = shared blocks (mt_s x nt_s) + routed blocks
// (mt_r x nt_r). Logical block -> (n-tile, m-tile) with the m-tile fastest,
// so consecutive logical blocks reuse one weight tile.
template <typename T>
__global__ void __launch_bounds__(NTHR) moe_gate_up_kernel(GemmArgs g) {
  extern __shared__ __align__(16) unsigned char smem[];
  Lds& L = *reinterpret_cast<Lds*>(smem);
  int* cum = reinterpret_cast<int*>(smem + sizeof(Lds));

  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t nshared = (uint32_t)g.mt_shared * g.nt_shared;
  const T* x = static_cast<const T*>(g.a);
  const int H = g.H;
  bool shared;
  int n0, row0, nrows, e = 0, N;
  if (lb < nshared) {
    shared = true;
    const int nt = lb / g.mt_shared, mt = lb % g.mt_shared;
    n0 = nt * 128;
    row0 = mt * BM;
    nrows = min(BM, g.T - row0);
    N = g.S * g.Is;
  } else {
    shared = false;
    const uint32_t b = lb - nshared;
    const int nt = b / g.mt_routed, slot = b % g.mt_routed;
    int mt;
    if (!locate_tile(g.offsets, g.E, slot, cum, &e, &mt)) return;
    n0 = nt * 128;
    row0 = g.offsets[e] + mt * BM;
    nrows = min(BM, g.offsets[e + 1] - row0);
    N = g.I;
  }

  Src<T> s;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = r0 + 32 * j;
    const T* p = nullptr;
    if (R < nrows) {
      const int tok = shared ? row0 + R : g.sorted_rows[row0 + R] / g.k;
      p = x + (size_t)tok * H;
    }
    s.a[j] = p;
  }
  const T* wg = static_cast<const T*>(shared ? g.ws0 : g.w0);
  const T* wu = static_cast<const T*>(shared ? g.ws1 : g.w1);
  const size_t ebase = shared ? 0 : (size_t)e * g.I * H;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int R = r0 + 32 * j;
    const int n = n0 + (R & 127);
    const T* p = nullptr;
    if (n < N) p = (R < 128 ? wg : wu) + ebase + (size_t)n * H;
    s.b[j] = p;
  }
  s.kseg = H;
  s.bstride = 0;

  floatx4_t acc[4][8];
  mainloop<T, true>(L, s, H, acc);

  // epilogue: h = act(gate, up)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r = lane & 15;
  T* dst = static_cast<T*>(shared ? g.out_shared : g.out);
  const int ld = shared ? g.S * g.Is : g.I;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = wm * 64 + mb * 16 + q * 4 + v;
      if (m >= nrows) continue;
      T* drow = dst + (size_t)(row0 + m) * ld;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + wn * 64 + nb * 16 + r;
        if (col < N) store_out<T>(drow + col, act_apply(acc[mb][nb][v], acc[mb][nb + 4][v], g.act));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down projection of the shared experts: acc[t] = h_shared[t] . Wsd_cat^T,
// stored (this launch runs before the routed one on the same stream).
template <typename T>
__global__ void __launch_bounds__(NTHR) moe_down_shared_kernel(GemmArgs g) {
  extern __shared__ __align__(16) unsigned char smem[];
  Lds& L = *reinterpret_cast<Lds*>(smem);
  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = lb / g.mt_shared, mt = lb % g.mt_shared;
  const int n0 = nt * BR, row0 = mt * BM;
  const int nrows = min(BM, g.T - row0);
  const int H = g.H, Ks = g.S * g.Is;
  const T* hs = static_cast<const T*>(g.a);
  const T* wd = static_cast<const T*>(g.ws0);
  Src<T> s;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = r0 + 32 * j;
    s.a[j] = R < nrows ? hs + (size_t)(row0 + R) * Ks : nullptr;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + r0 + 32 * j;
    s.b[j] = n < H ? wd + (size_t)n * g.Is : nullptr;
  }
  s.kseg = g.Is;                  // shared expert s occupies K in [s*Is, (s+1)*Is)
  s.bstride = (long)H * g.Is;     // ... and lives at ws_down + s*H*Is

  floatx4_t acc[4][8];
  mainloop<T, false>(L, s, Ks, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r = lane & 15;
  float* out = static_cast<float*>(g.out);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = wm * 64 + mb * 16 + q * 4 + v;
      if (m >= nrows) continue;
      float* orow = out + (size_t)(row0 + m) * H;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int col = n0 + wn * 128 + nb * 16 + r;
        if (col < H) orow[col] = acc[mb][nb][v];
      }
    }
}

// ---------------------------------------------------------------------------
// down projection of the routed experts, fused with the weighted combine:
// ATOMIC: acc[t] += w * y (fp32 atomics); else y_perm[p] = y (dtype).
template <typename T, bool ATOMIC>
__global__ void __launch_bounds__(NTHR) moe_down_routed_kernel(GemmArgs g) {
  extern __shared__ __align__(16) unsigned char smem[];
  Lds& L = *reinterpret_cast<Lds*>(smem);
  int* cum = reinterpret_cast<int*>(smem + sizeof(Lds));
  int* etok = cum + (g.E + 1);
  float* ew = reinterpret_cast<float*>(etok + BM);

  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const int nt = lb / g.mt_routed, slot = lb % g.mt_routed;
  int e, mt;
  if (!locate_tile(g.offsets, g.E, slot, cum, &e, &mt)) return;
  const int n0 = nt * BR;
  const int row0 = g.offsets[e] + mt * BM;
  const int nrows = min(BM, g.offsets[e + 1] - row0);
  const int H = g.H, I = g.I;
  const T* h = static_cast<const T*>(g.a);
  const T* wd = static_cast<const T*>(g.w0) + (size_t)e * H * I;

  if (ATOMIC && threadIdx.x < BM) {
    const int m = threadIdx.x;
    if (m < nrows) {
      const int rr = g.sorted_rows[row0 + m];
      etok[m] = rr / g.k;
      ew[m] = g.topk_w[rr];
    }
  }

  Src<T> s;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = r0 + 32 * j;
    s.a[j] = R < nrows ? h + (size_t)(row0 + R) * I : nullptr;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + r0 + 32 * j;
    s.b[j] = n < H ? wd + (size_t)n * I : nullptr;
  }
  s.kseg = I;
  s.bstride = 0;

  floatx4_t acc[4][8];
  mainloop<T, false>(L, s, I, acc);  // ends with a barrier: etok/ew visible

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r = lane & 15;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = wm * 64 + mb * 16 + q * 4 + v;
      if (m >= nrows) continue;
      if (ATOMIC) {
        float* orow = static_cast<float*>(g.out) + (size_t)etok[m] * H;
        const float wt = ew[m];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int col = n0 + wn * 128 + nb * 16 + r;
          if (col < H) unsafeAtomicAdd(orow + col, wt * acc[mb][nb][v]);
        }
      } else {
        T* yrow = static_cast<T*>(g.y_perm) + (size_t)(row0 + m) * H;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int col = n0 + wn * 128 + nb * 16 + r;
          if (col < H) store_out<T>(yrow + col, acc[mb][nb][v]);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// host-side launchers

size_t gemm_lds_bytes(int E) {
  return sizeof(Lds) + (size_t)(E + 1) * sizeof(int) + BM * (sizeof(int) + sizeof(float));
}

int gemm_bm() { return BM; }

static hipError_t set_lds(const void* fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_gate_up(const GemmArgs& g, int dtype, hipStream_t st) {
  const size_t lds = gemm_lds_bytes(g.E);
  const uint32_t nblk = (uint32_t)g.mt_shared * g.nt_shared + (uint32_t)g.mt_routed * g.nt_routed;
  if (nblk == 0) return hipSuccess;
  if (dtype == MOE_BF16) {
    hipError_t e = set_lds((const void*)moe_gate_up_kernel<bf16_t>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_gate_up_kernel<bf16_t>, dim3(nblk), dim3(NTHR), lds, st, g);
  } else {
    hipError_t e = set_lds((const void*)moe_gate_up_kernel<float>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_gate_up_kernel<float>, dim3(nblk), dim3(NTHR), lds, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_down_shared(const GemmArgs& g, int dtype, hipStream_t st) {
  const size_t lds = gemm_lds_bytes(g.E);
  const uint32_t nblk = (uint32_t)g.mt_shared * g.nt_shared;
  if (nblk == 0) return hipSuccess;
  if (dtype == MOE_BF16) {
    hipError_t e = set_lds((const void*)moe_down_shared_kernel<bf16_t>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_down_shared_kernel<bf16_t>, dim3(nblk), dim3(NTHR), lds, st, g);
  } else {
    hipError_t e = set_lds((const void*)moe_down_shared_kernel<float>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_down_shared_kernel<float>, dim3(nblk), dim3(NTHR), lds, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_down_routed(const GemmArgs& g, int dtype, bool atomic, hipStream_t st) {
  const size_t lds = gemm_lds_bytes(g.E);
  const uint32_t nblk = (uint32_t)g.mt_routed * g.nt_routed;
  if (nblk == 0) return hipSuccess;
  hipError_t e;
#define MOE_LAUNCH_DOWN(TT, AT)                                                        \
  e = set_lds((const void*)moe_down_routed_kernel<TT, AT>, lds);                       \
  if (e != hipSuccess) return e;                                                       \
  hipLaunchKernelGGL((moe_down_routed_kernel<TT, AT>), dim3(nblk), dim3(NTHR), lds, st, g);
  if (dtype == MOE_BF16) {
    if (atomic) { MOE_LAUNCH_DOWN(bf16_t, true) } else { MOE_LAUNCH_DOWN(bf16_t, false) }
  } else {
    if (atomic) { MOE_LAUNCH_DOWN(float, true) } else { MOE_LAUNCH_DOWN(float, false) }
  }
#undef MOE_LAUNCH_DOWN
  return hipGetLastError();
}
