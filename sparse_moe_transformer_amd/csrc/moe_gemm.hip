// Grouped expert GEMMs on MFMA (gfx950).
//
// Every stacked expert tensor is [out, in] with the reduction dimension
// contiguous (mlxcel #845 "Checkpoint weight layout": pre-stacked
// experts.{gate,up,down}_proj), and the activations are [rows, in], so both
// MFMA operands are read along K in 16-byte chunks.
//
// Workgroup tile: 128 activation rows x 256 weight rows; K-step of 128 bytes
// per row (64 bf16 or 32 fp32). Four waves in a 2x2 arrangement; each wave
// owns 64 rows x 128 weight rows = 2 x 4 MFMA blocks of 32x32.
//   gate/up: weight rows 0..127 are gate rows n0.., 128..255 the up rows of
//            the same columns, so each wave holds matching gate and up
//            accumulators and applies the activation in registers.
//   down:    weight rows 0..255 are 256 output columns.
// Pipeline: three LDS stages filled by direct global->LDS loads
// (global_load_lds_dwordx4, no staging registers); loads run two K-steps
// ahead of the MFMAs; one barrier per K-step. LDS rows are 8 chunks of 16 B
// with chunk c of row r stored at c ^ ((r >> 1) & 7), which keeps the 32x32
// fragment reads free of bank conflicts on gfx950. Each wave's load
// instruction fills 1 KB of LDS (8 rows); lane i supplies physical chunk
// i % 8 of row i / 8, so it fetches the logical chunk that lands there.
// Rows past the end of a tile (activation rows beyond the segment, weight
// rows beyond N) load a valid clamped row; their results are never stored.
#include "moe_common.h"
#include "moe_kernels.h"

typedef float floatx16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int BM = 128;    // activation rows per workgroup
constexpr int BR = 256;    // weight rows per workgroup
constexpr int NCH = 8;     // 16-byte chunks per LDS row per K-step
constexpr int NTHR = 256;
constexpr int MAX_EXPERTS = 1024;

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

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// The three LDS stages live in distinct __shared__ arrays so that the
// compiler can tell a load into one stage from a read of another and does not
// wait for every outstanding load before each LDS read.
#define MOE_LDS_STAGES                              \
  __shared__ __align__(16) u32x4_t lds_a0[BM * NCH]; \
  __shared__ __align__(16) u32x4_t lds_a1[BM * NCH]; \
  __shared__ __align__(16) u32x4_t lds_a2[BM * NCH]; \
  __shared__ __align__(16) u32x4_t lds_b0[BR * NCH]; \
  __shared__ __align__(16) u32x4_t lds_b1[BR * NCH]; \
  __shared__ __align__(16) u32x4_t lds_b2[BR * NCH];

constexpr int LOADS_PER_STAGE = 12;  // per thread: 4 activation + 8 weight

// Per-thread sources of its 12 load instructions per stage. Instruction j of
// wave w fills activation rows 32w+8j .. +7 (j < 4) or weight rows
// 64w+8j .. +7 (j < 8); the lane's row is that base + lane/8.
template <typename T>
struct Src {
  const T* a[4];  // row pointer + logical chunk offset (elements)
  const T* b[8];
  int kseg;       // weight K segment length (elements); K-split for shared down
  long bstride;   // elements between weight K segments
};

__device__ __forceinline__ int a_row(int j) { return (threadIdx.x >> 6) * 32 + 8 * j + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int b_row(int j) { return (threadIdx.x >> 6) * 64 + 8 * j + ((threadIdx.x & 63) >> 3); }
// logical chunk fetched by this lane for a row
__device__ __forceinline__ int lane_chunk(int row) { return (threadIdx.x & 7) ^ swz(row); }

__device__ __forceinline__ void dma16(const void* g, u32x4_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

template <typename T>
__device__ __forceinline__ void load_stage(const Src<T>& s, int kk, long bseg, int koff,
                                           u32x4_t* la, u32x4_t* lb) {
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16(s.a[j] + kk, la + (w * 4 + j) * 64);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma16(s.b[j] + bseg + koff, lb + (w * 8 + j) * 64);
}

// First weight row (within the 256-row tile) of block nb (0..3) of wave wn.
template <bool GATE_UP>
__device__ __forceinline__ int wrow(int wn, int nb) {
  if (GATE_UP) return nb < 2 ? wn * 64 + nb * 32 : 128 + wn * 64 + (nb - 2) * 32;
  return wn * 128 + nb * 32;
}

typedef floatx16_t Acc[2][4];

// One K-step from one LDS stage.
// bf16: 4 sub-steps of K=16; lane l reads row l%32, chunk 2*s + l/32.
template <typename T, bool GATE_UP>
__device__ __forceinline__ void compute_stage(const u32x4_t* la, const u32x4_t* lb, Acc& acc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 5, r = lane & 31;
  if constexpr (sizeof(T) == 2) {
    bf16x8_t fa[2][2], fb[2][4];
    auto read = [&](int s, int slot) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + r;
        fa[slot][mb] = __builtin_bit_cast(bf16x8_t, la[row * NCH + ((2 * s + q) ^ swz(row))]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = wrow<GATE_UP>(wn, nb) + r;
        fb[slot][nb] = __builtin_bit_cast(bf16x8_t, lb[row * NCH + ((2 * s + q) ^ swz(row))]);
      }
    };
    read(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read(s + 1, (s + 1) & 1);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][mb], fb[s & 1][nb],
                                                                acc[mb][nb], 0, 0, 0);
    }
    // schedule: the 6 fragment reads of sub-step s+1 are interleaved with the
    // 8 MFMAs of sub-step s, so LDS latency hides behind matrix work
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // reads of sub-step 0
#pragma unroll
    for (int s = 0; s < 3; ++s) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  } else {
    // fp32: lane group q holds k = 16q..16q+15 (chunks 4q..4q+3); MFMA v of
    // the 16 32x32x2 steps takes slot v of both operands.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = wm * 64 + mb * 32 + r;
      float av[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x4_t v = la[row * NCH + ((4 * q + u) ^ swz(row))];
        av[4 * u] = __uint_as_float(v.x); av[4 * u + 1] = __uint_as_float(v.y);
        av[4 * u + 2] = __uint_as_float(v.z); av[4 * u + 3] = __uint_as_float(v.w);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int brw = wrow<GATE_UP>(wn, nb) + r;
        float bv[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4_t v = lb[brw * NCH + ((4 * q + u) ^ swz(brw))];
          bv[4 * u] = __uint_as_float(v.x); bv[4 * u + 1] = __uint_as_float(v.y);
          bv[4 * u + 2] = __uint_as_float(v.z); bv[4 * u + 3] = __uint_as_float(v.w);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[v], bv[v], acc[mb][nb], 0, 0, 0);
      }
    }
  }
}

// vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Main loop: acc = A[128 x K] . B[256 x K]^T over the whole K (K % KS == 0).
// Stage i lives in LDS set i % 3. Step i: wait for this wave's loads of
// stage i (stage i+1 may stay in flight), barrier (all waves' loads of stage
// i are in LDS and every wave is done with set (i+2) % 3), issue the loads of
// stage i+2 into that set, compute stage i. The look-ahead loads are issued
// on every step (past the end they re-read the last stage) so the compiler
// sees the same number of loads in flight on every path.
#define MOE_STEP(I, LA, LB, NA, NB)                                   \
  {                                                                   \
    wait_vmcnt<LOADS_PER_STAGE>();                                    \
    __builtin_amdgcn_s_barrier();                                     \
    if ((I) + 2 < nk) advance();                                      \
    load_stage<T>(s, min((I) + 2, nk - 1) * KS, bseg, koff, NA, NB); \
    compute_stage<T, GATE_UP>(LA, LB, acc);                           \
  }

template <typename T, bool GATE_UP>
__device__ __forceinline__ void mainloop(u32x4_t* lds_a0, u32x4_t* lds_a1, u32x4_t* lds_a2,
                                         u32x4_t* lds_b0, u32x4_t* lds_b1, u32x4_t* lds_b2,
                                         const Src<T>& s, int K, Acc& acc) {
  constexpr int KS = NCH * Elem<T>::EPC;  // elements per K-step
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  const int nk = K / KS;
  // weight K position of the most recently issued stage
  long bseg = 0;
  int koff = 0;
  auto advance = [&]() {
    koff += KS;
    if (koff == s.kseg) {
      koff = 0;
      bseg += s.bstride;
    }
  };
  load_stage<T>(s, 0, bseg, koff, lds_a0, lds_b0);
  if (nk > 1) advance();
  load_stage<T>(s, min(1, nk - 1) * KS, bseg, koff, lds_a1, lds_b1);
  int it = 0;
  for (; it + 3 <= nk; it += 3) {
    MOE_STEP(it, lds_a0, lds_b0, lds_a2, lds_b2)
    MOE_STEP(it + 1, lds_a1, lds_b1, lds_a0, lds_b0)
    MOE_STEP(it + 2, lds_a2, lds_b2, lds_a1, lds_b1)
  }
  if (it < nk) MOE_STEP(it, lds_a0, lds_b0, lds_a2, lds_b2)
  if (it + 1 < nk) MOE_STEP(it + 1, lds_a1, lds_b1, lds_a0, lds_b0)
  // drain the look-ahead loads before the stages' LDS can be reused
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
}
#undef MOE_STEP

// Find which expert (and m-tile within it) routed m-slot `slot` belongs to.
// Returns false if the slot is past the last tile. Uses `cum` (E+1 ints of
// LDS): cum[e] = sum_{e'<e} ceil(n_e'/BM).
__device__ bool locate_tile(const int32_t* __restrict__ offsets, int E, int slot, int* cum,
                            int* e_out, int* mt_out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) local += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        cum[e] = run;
        run += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
      }
    }
    if (lane == 63) cum[E] = incl;
  }
  __syncthreads();
  if (slot >= cum[E]) return false;
  // the owner is the largest e with cum[e] <= slot (it has cum[e+1] > slot,
  // so it is not empty)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= slot) lo = mid;
    else hi = mid - 1;
  }
  *e_out = lo;
  *mt_out = slot - cum[lo];
  return true;
}

// Grouped tile order: logical block b -> (m-slot, n-tile) with groups of gm
// m-slots; inside a group the m-slot varies fastest. The ~32 workgroups that
// an XCD runs at once then cover a compact gm x (32/gm) patch, so both the
// activation tiles and the weight tiles they read are shared through L2.
__device__ __forceinline__ void grouped_order(uint32_t b, int mt, int nt, int gm, int* m, int* n) {
  const uint32_t per_group = (uint32_t)gm * nt;
  const int g = b / per_group;
  const int first = g * gm;
  const int gsize = min(gm, mt - first);
  const int local = b - g * per_group;
  *m = first + local % gsize;
  *n = local / gsize;
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

// Row (within the wave's 64 rows) of accumulator element v of block mb:
// 32x32 MFMA lane l holds rows 8*(v/4) + 4*(l/32) + v%4 of column l%32.
__device__ __forceinline__ int acc_row(int mb, int v, int q) {
  return mb * 32 + (v >> 2) * 8 + q * 4 + (v & 3);
}

}  // namespace

// ---------------------------------------------------------------------------
// gate/up + activation. Grid = shared blocks (mt_s x nt_s) + routed blocks
// (mt_r x nt_r), both in grouped order.
template <typename T>
__global__ void __launch_bounds__(NTHR) moe_gate_up_kernel(GemmArgs g) {
  MOE_LDS_STAGES
  __shared__ int cum[MAX_EXPERTS + 1];

  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t nshared = (uint32_t)g.mt_shared * g.nt_shared;
  const T* x = static_cast<const T*>(g.a);
  const int H = g.H;
  bool shared;
  int n0, row0, nrows, e = 0, N;
  if (lb < nshared) {
    shared = true;
    int nt, mt;
    grouped_order(lb, g.mt_shared, g.nt_shared, g.gm_shared, &mt, &nt);
    n0 = nt * 128;
    row0 = mt * BM;
    nrows = min(BM, g.T - row0);
    N = g.S * g.Is;
  } else {
    shared = false;
    int nt, slot, mt;
    grouped_order(lb - nshared, g.mt_routed, g.nt_routed, g.gm_routed, &slot, &nt);
    if (!locate_tile(g.offsets, g.E, slot, cum, &e, &mt)) return;
    n0 = nt * 128;
    row0 = g.offsets[e] + mt * BM;
    nrows = min(BM, g.offsets[e + 1] - row0);
    N = g.I;
  }

  constexpr int EPC = Elem<T>::EPC;
  Src<T> s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = a_row(j);
    const int R = min(row, nrows - 1);
    const int tok = shared ? row0 + R : g.sorted_rows[row0 + R] / g.k;
    s.a[j] = x + (size_t)tok * H + lane_chunk(row) * EPC;
  }
  const T* wg = static_cast<const T*>(shared ? g.ws0 : g.w0);
  const T* wu = static_cast<const T*>(shared ? g.ws1 : g.w1);
  const size_t ebase = shared ? 0 : (size_t)e * g.I * H;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = b_row(j);
    const int n = min(n0 + (row & 127), N - 1);
    s.b[j] = (row < 128 ? wg : wu) + ebase + (size_t)n * H + lane_chunk(row) * EPC;
  }
  s.kseg = H;
  s.bstride = 0;

  Acc acc;
  mainloop<T, true>(lds_a0, lds_a1, lds_a2, lds_b0, lds_b1, lds_b2, s, H, acc);

  // epilogue: h = act(gate, up); gate block nb pairs with up block nb + 2
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 5, r = lane & 31;
  T* dst = static_cast<T*>(shared ? g.out_shared : g.out);
  const int ld = shared ? g.S * g.Is : g.I;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = wm * 64 + acc_row(mb, v, q);
      if (m >= nrows) continue;
      T* drow = dst + (size_t)(row0 + m) * ld;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + r;
        if (col < N) store_out<T>(drow + col, act_apply(acc[mb][nb][v], acc[mb][nb + 2][v], g.act));
      }
    }
}

// ---------------------------------------------------------------------------
// down projection of the shared experts: acc[t] = h_shared[t] . Wsd_cat^T,
// stored (this launch runs before the routed one on the same stream).
template <typename T>
__global__ void __launch_bounds__(NTHR) moe_down_shared_kernel(GemmArgs g) {
  MOE_LDS_STAGES
  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  int nt, mt;
  grouped_order(lb, g.mt_shared, g.nt_shared, g.gm_shared, &mt, &nt);
  const int n0 = nt * BR, row0 = mt * BM;
  const int nrows = min(BM, g.T - row0);
  const int H = g.H, Ks = g.S * g.Is;
  const T* hs = static_cast<const T*>(g.a);
  const T* wd = static_cast<const T*>(g.ws0);
  constexpr int EPC = Elem<T>::EPC;
  Src<T> s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = a_row(j);
    s.a[j] = hs + (size_t)(row0 + min(row, nrows - 1)) * Ks + lane_chunk(row) * EPC;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = b_row(j);
    s.b[j] = wd + (size_t)min(n0 + row, H - 1) * g.Is + lane_chunk(row) * EPC;
  }
  s.kseg = g.Is;               // shared expert s occupies K in [s*Is, (s+1)*Is)
  s.bstride = (long)H * g.Is;  // ... and lives at ws_down + s*H*Is

  Acc acc;
  mainloop<T, false>(lds_a0, lds_a1, lds_a2, lds_b0, lds_b1, lds_b2, s, Ks, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 5, r = lane & 31;
  float* out = static_cast<float*>(g.out);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = wm * 64 + acc_row(mb, v, q);
      if (m >= nrows) continue;
      float* orow = out + (size_t)(row0 + m) * H;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + wn * 128 + nb * 32 + r;
        if (col < H) orow[col] = acc[mb][nb][v];
      }
    }
}

// ---------------------------------------------------------------------------
// down projection of the routed experts, fused with the weighted combine:
// ATOMIC: acc[t] += w * y (fp32 atomics); else y_perm[p] = y (dtype).
template <typename T, bool ATOMIC>
__global__ void __launch_bounds__(NTHR) moe_down_routed_kernel(GemmArgs g) {
  MOE_LDS_STAGES
  __shared__ int cum[MAX_EXPERTS + 1];
  __shared__ int etok[BM];
  __shared__ float ew[BM];

  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  int nt, slot;
  grouped_order(lb, g.mt_routed, g.nt_routed, g.gm_routed, &slot, &nt);
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

  constexpr int EPC = Elem<T>::EPC;
  Src<T> s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = a_row(j);
    s.a[j] = h + (size_t)(row0 + min(row, nrows - 1)) * I + lane_chunk(row) * EPC;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = b_row(j);
    s.b[j] = wd + (size_t)min(n0 + row, H - 1) * I + lane_chunk(row) * EPC;
  }
  s.kseg = I;
  s.bstride = 0;
  // etok/ew are written before the first barrier of the main loop
  __builtin_amdgcn_s_waitcnt(0xC07F & ~(0xF << 8));  // lgkmcnt(0): LDS writes done

  Acc acc;
  mainloop<T, false>(lds_a0, lds_a1, lds_a2, lds_b0, lds_b1, lds_b2, s, I, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 5, r = lane & 31;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = wm * 64 + acc_row(mb, v, q);
      if (m >= nrows) continue;
      if (ATOMIC) {
        float* orow = static_cast<float*>(g.out) + (size_t)etok[m] * H;
        const float wt = ew[m];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = n0 + wn * 128 + nb * 32 + r;
          if (col < H) unsafeAtomicAdd(orow + col, wt * acc[mb][nb][v]);
        }
      } else {
        T* yrow = static_cast<T*>(g.y_perm) + (size_t)(row0 + m) * H;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = n0 + wn * 128 + nb * 32 + r;
          if (col < H) store_out<T>(yrow + col, acc[mb][nb][v]);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// host-side launchers

size_t gemm_lds_bytes(int) { return 0; }

int gemm_bm() { return BM; }

static hipError_t set_lds(const void*, size_t) { return hipSuccess; }

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
