// Grouped expert GEMMs on MFMA (gfx950).
//
// Every stacked expert tensor is [out, in] with the reduction dimension
// contiguous (mlxcel #845 "Checkpoint weight layout": pre-stacked
// experts.{gate,up,down}_proj), and the activations are [rows, in], so both
// MFMA operands are read along K in 16-byte chunks.
//
// Tile: 128 activation rows x 256 weight rows; K-step of 128 bytes per row
// (64 bf16 or 32 fp32). Four waves in a 2x2 arrangement; each wave owns 64
// rows x 128 weight rows = 2 x 4 MFMA blocks of 32x32.
//   gate/up: weight rows 0..127 are gate rows n0.., 128..255 the up rows of
//            the same columns, so each wave holds matching gate and up
//            accumulators and applies the activation in registers.
//   down:    weight rows 0..255 are 256 output columns.
//
// Persistent schedule: one workgroup per compute unit walks a fixed list of
// tiles. Tiles are numbered in a grouped order (m fastest inside groups of
// m-slots) and every XCD owns a contiguous range of them, so the ~32
// workgroups an XCD runs at once share activation and weight tiles in L2.
//
// Pipeline: three LDS stages filled by direct global->LDS loads
// (global_load_lds_dwordx4, no staging registers), two K-steps ahead of the
// MFMAs, one barrier per step. The load stream runs on across tiles: the last
// two steps of a tile load the first two stages of the next tile, so they are
// in flight during this tile's epilogue. Each tile's step count is padded to
// a multiple of three, so the LDS stage of every step is known at compile
// time; the padding steps (at most the tile's last two) skip their MFMAs and
// their loads re-read the tile's last real step. The three stages are
// distinct __shared__ arrays and the barrier is a raw s_barrier, so the
// compiler does not drain all loads before each LDS read. Nothing that a later
// step must wait for is loaded after the look-ahead loads of a step (vector
// memory counts complete in order), so no wait drains the pipeline. LDS rows
// are 8 chunks of 16 B with chunk c of row r stored at c ^ ((r >> 1) & 7): no
// bank conflicts for the 32x32 fragment reads (measured on gfx950). Rows past
// the end of a tile (activation rows beyond the segment, weight rows beyond
// N) load a valid clamped row; their results are never stored.
//
// MXFP8 expert weights (OCP MX: E4M3 codes, one E8M0 scale per 32 inputs,
// scales block-major [K/32, N]; the MXFP8 export of mlxcel #763
// "Validation"), with bf16 activations: a weight row holds 64 bytes per
// K-step (4 chunks, chunk c of row r at c ^ ((r >> 2) & 3)) and the step's
// two scale bytes of each row sit after the weight rows of the stage. Inside
// a step the K order is permuted, the same for both operands: lane half q
// takes inputs 32q .. 32q+31, sub-step s the eight at 32q + 8s. A lane reads
// two 16-byte weight chunks and one scale per weight block and step, turns
// the codes into bf16 with the scaled conversion (exact for these values)
// and runs the bf16 MFMAs; per step the LDS moves a third less than with
// bf16 weights (stage writes 33 KiB, fragment reads 64 KiB).
//
// MXFP4 expert weights (E2M1 codes, two per byte, input 2j in the low nibble
// of byte j; the same scales): a weight row holds 32 bytes per K-step (2
// chunks, chunk c of row r at c ^ ((r >> 3) & 1)), so chunk q is exactly
// lane half q's 32 inputs and one scale block; sub-step s takes its dword s
// (eight codes) through the scaled fp4 conversion.
#include "moe_common.h"
#include "moe_gemm_common.h"
#include "moe_kernels.h"

typedef float floatx16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int BM = 128;    // activation rows per tile
constexpr int BR = 256;    // weight rows per tile
constexpr int NCH = 8;     // 16-byte chunks per LDS row per K-step
constexpr int KSB = NCH * 16;  // bytes per row per K-step
constexpr int NTHR = 256;
constexpr int MAX_EXPERTS = 1024;
constexpr int LOADS_BF16 = 12;  // per thread: 4 activation + 8 weight
constexpr int LOADS_FP8 = 9;    // 4 activation + 4 weight + 1 scale
constexpr int LOADS_FP4 = 7;    // 4 activation + 2 weight + 1 scale
constexpr int FP8_SCALES = 1024;  // u32x4 index of the scale bytes in an MXFP8 weight stage
constexpr int FP4_SCALES = 512;   // ... in an MXFP4 weight stage
template <int WM>
constexpr int loads_of() { return WM == WF_MXFP8 ? LOADS_FP8 : WM == WF_MXFP4 ? LOADS_FP4 : LOADS_BF16; }
template <int WM>
constexpr int scales_at() { return WM == WF_MXFP4 ? FP4_SCALES : FP8_SCALES; }

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

#define MOE_LDS_STAGES                              \
  __shared__ __align__(16) u32x4_t lds_a0[BM * NCH]; \
  __shared__ __align__(16) u32x4_t lds_a1[BM * NCH]; \
  __shared__ __align__(16) u32x4_t lds_a2[BM * NCH]; \
  __shared__ __align__(16) u32x4_t lds_b0[BR * NCH]; \
  __shared__ __align__(16) u32x4_t lds_b1[BR * NCH]; \
  __shared__ __align__(16) u32x4_t lds_b2[BR * NCH];

// Load instruction j of wave w fills activation rows 32w+8j .. +7 (j < 4) or
// weight rows 64w+8j .. +7 (j < 8); the lane's row is that base + lane/8 and
// it fetches the logical chunk that lands at physical chunk lane % 8.
__device__ __forceinline__ int a_row(int j) { return (threadIdx.x >> 6) * 32 + 8 * j + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int b_row(int j) { return (threadIdx.x >> 6) * 64 + 8 * j + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int lane_chunk(int row) { return (threadIdx.x & 7) ^ swz(row); }
// MXFP8 weight rows: instruction j of wave w fills rows 64w+16j .. +15, four
// lanes per row; chunk c of row r is stored at c ^ swz4(r)
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int b_row_fp8(int j) {
  return (threadIdx.x >> 6) * 64 + 16 * j + ((threadIdx.x & 63) >> 2);
}
// MXFP4 weight rows: instruction j of wave w fills rows 64w+32j .. +31, two
// lanes per row; chunk c of row r is stored at c ^ swz2(r)
__device__ __forceinline__ int swz2(int row) { return (row >> 3) & 1; }
__device__ __forceinline__ int b_row_fp4(int j) {
  return (threadIdx.x >> 6) * 64 + 32 * j + ((threadIdx.x & 63) >> 1);
}
// the scale bytes a lane loads: lanes 0..31 of wave w take 4 rows from
// 64w + 4 (l % 16) of block l / 16 (lanes 32..63 repeat them into the unused
// half of the wave's 256-byte slot)
__device__ __forceinline__ int scale_lane_row() { return 64 * (threadIdx.x >> 6) + 4 * (threadIdx.x & 15); }
__device__ __forceinline__ int scale_lane_block() { return (threadIdx.x >> 4) & 1; }

// One tile: where its rows and weights are and how many K-steps it has.
struct Tile {
  const char* a[4];  // activation row pointers (+ lane chunk offset), bytes
  const char* b[8];  // weight row pointers (+ lane chunk offset), bytes (MXFP8: 4, MXFP4: 2)
  const char* s;     // MX: this lane's scale bytes of the first K-step
  int sstep;         // MX: scale bytes per K-step
  int nk;            // real K-steps
  int nk3;           // steps padded to a multiple of 3
  int kseg;          // weight K segment length in bytes (K-split of shared down)
  int bstride_kb;    // KiB between weight K segments
  int shared, e, row0, nrows, n0, N;
};

// Load this lane's chunks for step j of tile t into LDS stage (la, lb).
// Padding steps (j >= nk) re-read the tile's last real step: their MFMAs are
// skipped, so what they load is never used, and a valid address keeps every
// step's loads the same without a per-lane choice of source.
template <int WM>
__device__ __forceinline__ void issue_stage(const Tile& t, int j, u32x4_t* la, u32x4_t* lb) {
  const int jr = j < t.nk ? j : t.nk - 1;
  const int kb = jr * KSB;
  // weight bytes per step
  const int kw = WM == WF_MXFP8 ? jr * (KSB / 2) : WM == WF_MXFP4 ? jr * (KSB / 4) : kb;
  const int seg = kw / t.kseg;
  const long boff = (long)seg * t.bstride_kb * 1024 + (kw - seg * t.kseg);
  // wave-uniform, so the LDS addresses are scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_global_load_lds(t.a[q] + kb, la + (w * 4 + q) * 64, 16, 0, 0);
  if (WM != WF_DTYPE) {
    if (WM == WF_MXFP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds(t.b[q] + boff, lb + w * 256 + q * 64, 16, 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_global_load_lds(t.b[q] + boff, lb + w * 128 + q * 64, 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(t.s + (long)jr * t.sstep, lb + scales_at<WM>() + w * 16, 4,
                                     0, 0);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_global_load_lds(t.b[q] + boff, lb + (w * 8 + q) * 64, 16, 0, 0);
  }
}

// First weight row (within the 256-row tile) of block nb (0..3) of wave wn.
template <int KIND>
__device__ __forceinline__ int wrow(int wn, int nb) {
  if (KIND == GATE_UP) return nb < 2 ? wn * 64 + nb * 32 : 128 + wn * 64 + (nb - 2) * 32;
  return wn * 128 + nb * 32;
}

typedef floatx16_t Acc[2][4];

// One K-step from one LDS stage.
// bf16: 4 sub-steps of K=16; lane l reads row l%32, chunk 2*s + l/32.
// MXFP8 weights: lane l takes inputs 32q + 8s .. +7 (q = l/32): activation
// chunk 4q + s, weight chunks 2q, 2q+1 and the scale of block q.
// MXFP4 weights: the same inputs; weight chunk q (dword s) and its scale.
template <typename T, int KIND, int WM>
__device__ __forceinline__ void compute_stage(const u32x4_t* la, const u32x4_t* lb, Acc& acc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 5, r = lane & 31;
  if constexpr (WM == WF_MXFP4) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + FP4_SCALES);
    u32x4_t wv[4];
    float scale[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int row = wrow<KIND>(wn, nb) + r;
      wv[nb] = lb[row * 2 + (q ^ swz2(row))];
      scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * q + (row & 63)]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t fa[2], fb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + r;
        fa[mb] = __builtin_bit_cast(bf16x8_t, la[row * NCH + ((4 * q + s) ^ swz(row))]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x4_t& c = wv[nb];
        fb[nb] = fp4x8_to_bf16(s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w, scale[nb]);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
    }
  } else if constexpr (WM == WF_MXFP8) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + FP8_SCALES);
    u32x4_t wv[4][2];
    float scale[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int row = wrow<KIND>(wn, nb) + r;
      wv[nb][0] = lb[row * 4 + ((2 * q) ^ swz4(row))];
      wv[nb][1] = lb[row * 4 + ((2 * q + 1) ^ swz4(row))];
      scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * q + (row & 63)]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t fa[2], fb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + r;
        fa[mb] = __builtin_bit_cast(bf16x8_t, la[row * NCH + ((4 * q + s) ^ swz(row))]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x4_t& c = wv[nb][s >> 1];
        fb[nb] = (s & 1) ? fp8x8_to_bf16(c.z, c.w, scale[nb]) : fp8x8_to_bf16(c.x, c.y, scale[nb]);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
    }
  } else if constexpr (sizeof(T) == 2) {
    bf16x8_t fa[2][2], fb[2][4];
    auto read = [&](int s, int slot) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + r;
        fa[slot][mb] = __builtin_bit_cast(bf16x8_t, la[row * NCH + ((2 * s + q) ^ swz(row))]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = wrow<KIND>(wn, nb) + r;
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
    // schedule: the 6 fragment reads of sub-step s+1 and 3 of the step's 12
    // global->LDS loads are interleaved with the 8 MFMAs of sub-step s. Issued
    // back to back, the loads would stall the wave on a full memory queue
    // with its MFMAs waiting behind them (measured: 1768 -> 1423 cycles per
    // step with L2-resident data).
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // reads of sub-step 0
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s < 3 && i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i == 1 || i == 4 || i == 7) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
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
        const int brw = wrow<KIND>(wn, nb) + r;
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

template <int KIND>
__device__ __forceinline__ int tile_count(const GemmArgs& g, const int* cum) {
  if (KIND == GATE_UP || KIND == DOWN_BOTH) return g.mt_shared * g.nt_shared + cum[g.E] * g.nt_routed;
  if (KIND == DOWN_SHARED) return g.mt_shared * g.nt_shared;
  return cum[g.E] * g.nt_routed;
}

// Where tile `idx` is (no global memory reads: offsets and prefix are in LDS).
template <int KIND>
__device__ __forceinline__ void tile_place(const GemmArgs& g, const int* offs, const int* cum,
                                           int idx, int* shared, int* e, int* row0, int* nrows,
                                           int* nt) {
  const int nshared = KIND == DOWN_ROUTED ? 0 : g.mt_shared * g.nt_shared;
  int mt;
  *e = 0;
  if (idx < nshared) {
    *shared = 1;
    grouped_order(idx, g.mt_shared, g.nt_shared, g.gm_shared, &mt, nt);
    *row0 = mt * BM;
    *nrows = min(BM, g.T - *row0);
  } else {
    // routed tiles are expert-major: expert e owns tiles
    // [cum[e] * nt_routed, cum[e+1] * nt_routed), so concurrent tiles share
    // one expert's weights; inside an expert, groups of gm m-slots with the
    // m-slot varying fastest
    *shared = 0;
    const int t = idx - nshared;
    *e = owner(cum, g.E, t / g.nt_routed);
    const int ms = cum[*e + 1] - cum[*e];
    int m;
    grouped_order(t - cum[*e] * g.nt_routed, ms, g.nt_routed, g.gm_routed, &m, nt);
    *row0 = offs[*e] + m * BM;
    *nrows = min(BM, offs[*e + 1] - *row0);
  }
}

// A tile's place: row0 (x), nrows | shared << 16 (y), expert (z), n-tile (w).
// A workgroup computes the places of its first MAX_WG_TILES tiles once, in
// parallel, into LDS; later tiles (very large batches) are placed on the fly.
constexpr int MAX_WG_TILES = 256;

template <int KIND>
__device__ __forceinline__ int4 place_of(const GemmArgs& g, const int* offs, const int* cum,
                                         int idx) {
  int shared, e, row0, nrows, nt;
  tile_place<KIND>(g, offs, cum, idx, &shared, &e, &row0, &nrows, &nt);
  return make_int4(row0, nrows | (shared << 16), e, nt);
}

// Tokens of this lane's 4 activation rows of routed gate/up tile p (global
// loads; shared tiles need none).
template <int KIND>
__device__ __forceinline__ void load_tokens(const GemmArgs& g, int4 p, int (&tok)[4]) {
  if (KIND != GATE_UP) return;
  const int row0 = p.x, nrows = p.y & 0xFFFF, shared = p.y >> 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = min(a_row(j), nrows - 1);
    tok[j] = shared ? row0 + R : g.sorted_rows[row0 + R];
  }
}

template <typename T, int KIND, int WM>
__device__ void make_tile(const GemmArgs& g, int4 p, const int (&tok)[4], Tile& t) {
  constexpr int EPC = Elem<T>::EPC;
  const int H = g.H;
  t.row0 = p.x;
  t.nrows = p.y & 0xFFFF;
  t.shared = p.y >> 16;
  t.e = p.z;
  const int nt = p.w;
  if (KIND == GATE_UP) {
    const T* x = static_cast<const T*>(g.a);
    t.n0 = nt * 128;
    t.N = t.shared ? g.S * g.Is : g.I;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = a_row(j);
      const int token = t.shared ? tok[j] : div_k(tok[j], g.k, g.kmagic);
      t.a[j] = reinterpret_cast<const char*>(x + (size_t)token * H + lane_chunk(row) * EPC);
    }
    if (WM != WF_DTYPE) {
      // codes [., N, H] (MXFP8: one byte per weight; MXFP4: [., N, H/2]);
      // scales [., H/32, N_s] per matrix, the shared experts' matrices of
      // width Is one after another
      const char* wg = static_cast<const char*>(t.shared ? g.ws0 : g.w0);
      const char* wu = static_cast<const char*>(t.shared ? g.ws1 : g.w1);
      const int rb = WM == WF_MXFP4 ? H / 2 : H;  // bytes per weight row
      const size_t ebase = t.shared ? 0 : (size_t)t.e * g.I * rb;
      if (WM == WF_MXFP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = b_row_fp8(j);
          const int n = min(t.n0 + (row & 127), t.N - 1);
          t.b[j] = (row < 128 ? wg : wu) + ebase + (size_t)n * rb + ((threadIdx.x & 3) ^ swz4(row)) * 16;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = b_row_fp4(j);
          const int n = min(t.n0 + (row & 127), t.N - 1);
          t.b[j] = (row < 128 ? wg : wu) + ebase + (size_t)n * rb + ((threadIdx.x & 1) ^ swz2(row)) * 16;
        }
      }
      const int w = threadIdx.x >> 6;
      const int ns = t.shared ? g.Is : g.I;
      const uint8_t* sm = w < 2 ? (t.shared ? g.sws0 : g.sw0) : (t.shared ? g.sws1 : g.sw1);
      const int n = min(t.n0 + (scale_lane_row() & 127), t.N - 4);
      const int se = t.shared ? n / ns : 0;
      const size_t mat = t.shared ? (size_t)se * (H / 32) * ns : (size_t)t.e * (H / 32) * ns;
      t.s = reinterpret_cast<const char*>(sm) + mat + (n - se * ns) + (size_t)scale_lane_block() * ns;
      t.sstep = 2 * ns;
      t.kseg = rb;
    } else {
      const T* wg = static_cast<const T*>(t.shared ? g.ws0 : g.w0);
      const T* wu = static_cast<const T*>(t.shared ? g.ws1 : g.w1);
      const size_t ebase = t.shared ? 0 : (size_t)t.e * g.I * H;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = b_row(j);
        const int n = min(t.n0 + (row & 127), t.N - 1);
        t.b[j] = reinterpret_cast<const char*>((row < 128 ? wg : wu) + ebase + (size_t)n * H +
                                               lane_chunk(row) * EPC);
      }
      t.kseg = H * (int)sizeof(T);
    }
    t.nk = H / (NCH * EPC);
    t.bstride_kb = 0;
  } else {
    // down: shared tiles read h_shared [T, S*Is] against the S shared down
    // matrices [H, Is] (K segment s at ws_down + s*H*Is); routed tiles read
    // h [T*k, I] against expert e's down matrix [H, I]
    const bool sh = KIND == DOWN_SHARED || (KIND == DOWN_BOTH && t.shared);
    const int Ks = sh ? g.S * g.Is : g.I;  // row length of the activations
    const int ldb = sh ? g.Is : g.I;       // row length of a weight K segment
    const T* act = static_cast<const T*>(KIND == DOWN_BOTH && sh ? g.a_shared : g.a);
    t.n0 = nt * BR;
    t.N = H;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = a_row(j);
      t.a[j] = reinterpret_cast<const char*>(act + (size_t)(t.row0 + min(row, t.nrows - 1)) * Ks +
                                             lane_chunk(row) * EPC);
    }
    if (WM != WF_DTYPE) {
      // scales [K/32, H]: the S shared matrices' blocks follow one another
      // along K, so K-step j of a shared tile reads blocks 2j, 2j+1
      const int half = WM == WF_MXFP4 ? 1 : 0;  // MXFP4: two weights per byte
      const char* wd = sh ? static_cast<const char*>(g.ws0)
                          : static_cast<const char*>(g.w0) + (((size_t)t.e * H * g.I) >> half);
      const int rb = ldb >> half;  // bytes per weight row of a K segment
      if (WM == WF_MXFP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = b_row_fp8(j);
          t.b[j] = wd + (size_t)min(t.n0 + row, H - 1) * rb + ((threadIdx.x & 3) ^ swz4(row)) * 16;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = b_row_fp4(j);
          t.b[j] = wd + (size_t)min(t.n0 + row, H - 1) * rb + ((threadIdx.x & 1) ^ swz2(row)) * 16;
        }
      }
      const uint8_t* sm = sh ? g.sws0 : g.sw0 + (size_t)t.e * (g.I / 32) * H;
      const int n = min(t.n0 + scale_lane_row(), H - 4);
      t.s = reinterpret_cast<const char*>(sm) + n + (size_t)scale_lane_block() * H;
      t.sstep = 2 * H;
      t.kseg = rb;
      t.bstride_kb = sh ? (int)((((long)H * g.Is) >> half) >> 10) : 0;
    } else {
      const T* wd = sh ? static_cast<const T*>(g.ws0)
                       : static_cast<const T*>(g.w0) + (size_t)t.e * H * g.I;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = b_row(j);
        t.b[j] = reinterpret_cast<const char*>(wd + (size_t)min(t.n0 + row, H - 1) * ldb +
                                               lane_chunk(row) * EPC);
      }
      t.kseg = ldb * (int)sizeof(T);
      t.bstride_kb = sh ? (int)(((long)H * g.Is * (long)sizeof(T)) >> 10) : 0;
    }
    t.nk = Ks / (NCH * EPC);
  }
  t.nk3 = (t.nk + 2) / 3 * 3;
}

}  // namespace

// ---------------------------------------------------------------------------
// The persistent kernel. Grid: one workgroup per compute unit (or fewer).
// Step j of a tile: wait for this wave's loads of stage j (only the next
// stage's loads are younger), barrier (all waves' loads of stage j are in LDS
// and every wave is done with stage j-1's set), issue the loads of the stage
// two ahead into that set, compute stage j.
#define MOE_STEP(TL, J, LA, LB, NA, NB)                       \
  {                                                           \
    wait_vmcnt<loads_of<WM>()>();                             \
    __builtin_amdgcn_s_barrier();                             \
    issue_stage<WM>(TL, J, NA, NB);                           \
    compute_stage<T, KIND, WM>(LA, LB, acc);                  \
  }
// The same step, its MFMAs skipped when C is false (a padding step of zeros,
// which would add exactly zero; its loads still run, so every step issues the
// same loads and the waits stay as they are).
#define MOE_STEP_IF(TL, J, LA, LB, NA, NB, C)                 \
  {                                                           \
    wait_vmcnt<loads_of<WM>()>();                             \
    __builtin_amdgcn_s_barrier();                             \
    issue_stage<WM>(TL, J, NA, NB);                           \
    if (C) compute_stage<T, KIND, WM>(LA, LB, acc);           \
  }

template <typename T, int KIND, bool ATOMIC, int WM>
__device__ __forceinline__ void moe_gemm_body(const GemmArgs& g) {
  MOE_LDS_STAGES
  __shared__ int offs[MAX_EXPERTS + 1];
  __shared__ int cum[MAX_EXPERTS + 1];
  __shared__ int ep_tok[BM];   // routed down epilogue: token and weight of each row
  __shared__ float ep_w[BM];
  __shared__ int4 places[MAX_WG_TILES];

  if (KIND != DOWN_SHARED) build_tile_prefix<BM>(g.offsets, g.E, offs, cum);
  __syncthreads();
  const int ntiles = tile_count<KIND>(g, cum);
  // this workgroup's tiles: its XCD's contiguous range of the shared-expert
  // tiles and of the routed ones, each split over the XCDs separately, so
  // every XCD streams its share of the routed experts' weights (with the
  // shared tiles first in one range, two XCDs would take the dense shared
  // expert and the other six every routed weight)
  const WgTiles wt = wg_tiles(ntiles, KIND == DOWN_BOTH || KIND == GATE_UP ? g.mt_shared * g.nt_shared : 0);
  const int n_my = wt.n_my;
  if (n_my == 0) return;
  auto gtile = [&](int i) { return wt.global(i); };
  for (int i = threadIdx.x; i < min(n_my, MAX_WG_TILES); i += NTHR)
    places[i] = place_of<KIND>(g, offs, cum, gtile(i));
  __syncthreads();
  // the place of tile i (the last tile stands in for any i past the end)
  // (workgroup-uniform: moved to scalar registers)
  auto place = [&](int i) -> int4 {
    i = min(i, n_my - 1);
    const int4 p = i < MAX_WG_TILES ? places[i] : place_of<KIND>(g, offs, cum, gtile(i));
    return make_int4(__builtin_amdgcn_readfirstlane(p.x), __builtin_amdgcn_readfirstlane(p.y),
                     __builtin_amdgcn_readfirstlane(p.z), __builtin_amdgcn_readfirstlane(p.w));
  };

  // Row ids are loaded one tile ahead, just before the first stage loads of
  // the tile before theirs: the wait of that tile's first step then covers
  // them (loads complete in order), so using them never drains the pipeline.
  int li = 0;  // local index of the current tile
  int tok[4] = {0, 0, 0, 0};
  load_tokens<KIND>(g, place(0), tok);
  Tile cur, nxt;
  make_tile<T, KIND, WM>(g, place(0), tok, cur);
  load_tokens<KIND>(g, place(1), tok);
  int ep_r = 0;  // routed down epilogue: the sorted row id of row threadIdx.x
  if (KIND == DOWN_ROUTED && threadIdx.x < BM)
    ep_r = g.sorted_rows[cur.row0 + min((int)threadIdx.x, cur.nrows - 1)];
  issue_stage<WM>(cur, 0, lds_a0, lds_b0);
  issue_stage<WM>(cur, 1, lds_a1, lds_b1);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 5, r = lane & 31;

  for (;;) {
    const bool has_next = li + 1 < n_my;
    Acc acc;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

    const int nk3 = cur.nk3;
    int j = 0;
    for (; j + 3 < nk3; j += 3) {
      MOE_STEP(cur, j + 2, lds_a0, lds_b0, lds_a2, lds_b2)
      MOE_STEP(cur, j + 3, lds_a1, lds_b1, lds_a0, lds_b0)
      MOE_STEP(cur, j + 4, lds_a2, lds_b2, lds_a1, lds_b1)
    }
    // last three steps: the look-ahead loads are the next tile's first stages
    MOE_STEP(cur, j + 2, lds_a0, lds_b0, lds_a2, lds_b2)
    int ep_t = 0;
    float ep_wt = 0.f;
    if (KIND == DOWN_ROUTED && threadIdx.x < BM) {
      if (ATOMIC) ep_wt = g.topk_w[ep_r];
      ep_t = div_k(ep_r, g.k, g.kmagic);
    }
    make_tile<T, KIND, WM>(g, place(li + 1), tok, nxt);
    // ids of the tile after next, then (below) the next tile's first stages
    load_tokens<KIND>(g, place(li + 2), tok);
    if (KIND == DOWN_ROUTED && threadIdx.x < BM)
      ep_r = g.sorted_rows[nxt.row0 + min((int)threadIdx.x, nxt.nrows - 1)];
    const int s0 = has_next ? 0 : nxt.nk3;  // nothing to load after the last tile
    // the tile's last two steps; padding steps (at most the last two: nk3 -
    // nk <= 2) skip their MFMAs
    MOE_STEP_IF(nxt, s0, lds_a1, lds_b1, lds_a0, lds_b0, j + 1 < cur.nk)
    MOE_STEP_IF(nxt, s0 + 1, lds_a2, lds_b2, lds_a1, lds_b1, j + 2 < cur.nk)

    // ---- epilogue of the current tile (next tile's first stages in flight).
    // Full tiles (all rows present, all columns inside N) take a path with no
    // per-element bounds checks: lane (q, r) of wave (wm, wn) writes rows
    // base + acc_row(mb, v, q) of column r of each 32-column block.
    const bool full_rows = cur.nrows == BM;
    if (KIND == GATE_UP) {
      T* dst = static_cast<T*>(cur.shared ? g.out_shared : g.out);
      const int ld = cur.shared ? g.S * g.Is : g.I;
      T* base = dst + (size_t)(cur.row0 + wm * 64) * ld + cur.n0 + wn * 64 + r;
      if (full_rows && cur.n0 + 128 <= cur.N) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            T* p = base + (size_t)acc_row(mb, v, q) * ld;
            store_out<T>(p, act_apply(acc[mb][0][v], acc[mb][2][v], g.act));
            store_out<T>(p + 32, act_apply(acc[mb][1][v], acc[mb][3][v], g.act));
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            // whole groups of 8 rows past the tile's rows: a uniform skip
            if (wm * 64 + mb * 32 + (v >> 2) * 8 >= cur.nrows) continue;
            const int m = wm * 64 + acc_row(mb, v, q);
            if (m >= cur.nrows) continue;
            T* p = base + (size_t)acc_row(mb, v, q) * ld;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              const int col = cur.n0 + wn * 64 + nb * 32 + r;
              if (col < cur.N) store_out<T>(p + nb * 32, act_apply(acc[mb][nb][v], acc[mb][nb + 2][v], g.act));
            }
          }
      }
    } else if (KIND == DOWN_SHARED || (KIND == DOWN_BOTH && cur.shared)) {
      float* base = static_cast<float*>(g.out) + (size_t)(cur.row0 + wm * 64) * g.H + cur.n0 +
                    wn * 128 + r;
      if (full_rows && cur.n0 + BR <= cur.N) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float* p = base + (size_t)acc_row(mb, v, q) * g.H;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) p[nb * 32] = acc[mb][nb][v];
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            // whole groups of 8 rows past the tile's rows: a uniform skip
            if (wm * 64 + mb * 32 + (v >> 2) * 8 >= cur.nrows) continue;
            const int m = wm * 64 + acc_row(mb, v, q);
            if (m >= cur.nrows) continue;
            float* p = base + (size_t)acc_row(mb, v, q) * g.H;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const int col = cur.n0 + wn * 128 + nb * 32 + r;
              if (col < cur.N) p[nb * 32] = acc[mb][nb][v];
            }
          }
      }
    } else {
      if (ATOMIC) {
        if (threadIdx.x < BM) {
          ep_tok[threadIdx.x] = ep_t;
          ep_w[threadIdx.x] = ep_wt;
        }
        // raw barrier: only the LDS writes above must be complete
        __builtin_amdgcn_s_waitcnt(0xC07F & ~(0xF << 8));  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
      }
      const bool full = full_rows && cur.n0 + BR <= cur.N;
      if (ATOMIC) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (!full && wm * 64 + mb * 32 + (v >> 2) * 8 >= cur.nrows) continue;
            const int m = wm * 64 + acc_row(mb, v, q);
            if (!full && m >= cur.nrows) continue;
            float* orow = static_cast<float*>(g.out) + (size_t)ep_tok[m] * g.H + cur.n0 + wn * 128 + r;
            const float wt = ep_w[m];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              if (full || cur.n0 + wn * 128 + nb * 32 + r < cur.N)
                unsafeAtomicAdd(orow + nb * 32, wt * acc[mb][nb][v]);
          }
      } else {
        T* base = static_cast<T*>(g.y_perm) + (size_t)(cur.row0 + wm * 64) * g.H + cur.n0 +
                  wn * 128 + r;
        if (full) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              T* p = base + (size_t)acc_row(mb, v, q) * g.H;
#pragma unroll
              for (int nb = 0; nb < 4; ++nb) store_out<T>(p + nb * 32, acc[mb][nb][v]);
            }
        } else {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              if (wm * 64 + mb * 32 + (v >> 2) * 8 >= cur.nrows) continue;
              const int m = wm * 64 + acc_row(mb, v, q);
              if (m >= cur.nrows) continue;
              T* p = base + (size_t)acc_row(mb, v, q) * g.H;
#pragma unroll
              for (int nb = 0; nb < 4; ++nb)
                if (cur.n0 + wn * 128 + nb * 32 + r < cur.N) store_out<T>(p + nb * 32, acc[mb][nb][v]);
            }
        }
      }
      // ep_tok/ep_w are rewritten by the next tile only after its steps'
      // barriers
    }
    if (!has_next) break;
    ++li;
    cur = nxt;
  }
  // the look-ahead loads after the last tile are not used: let them land
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
}
#undef MOE_STEP
#undef MOE_STEP_IF

// one entry per kind, so that profiles name them (WM: the weight format)
template <typename T, int WM>
__global__ void __launch_bounds__(NTHR) moe_gate_up_kernel(GemmArgs g) {
  moe_gemm_body<T, GATE_UP, false, WM>(g);
}
template <typename T, int WM>
__global__ void __launch_bounds__(NTHR) moe_down_shared_kernel(GemmArgs g) {
  moe_gemm_body<T, DOWN_SHARED, false, WM>(g);
}
template <typename T, bool ATOMIC, int WM>
__global__ void __launch_bounds__(NTHR) moe_down_routed_kernel(GemmArgs g) {
  moe_gemm_body<T, DOWN_ROUTED, ATOMIC, WM>(g);
}
template <typename T, int WM>
__global__ void __launch_bounds__(NTHR) moe_down_kernel(GemmArgs g) {
  moe_gemm_body<T, DOWN_BOTH, false, WM>(g);
}

// ---------------------------------------------------------------------------
// host-side launchers

int gemm_bm() { return BM; }

static int g_num_cus = 0;
static int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

static int grid_for(long max_tiles) { return (int)(max_tiles < num_cus() ? max_tiles : num_cus()); }

// The kernel instance for the weight format and dtype: MX weights always
// take bf16 activations (the host checks).
#define GEMM_LAUNCH(KERN, n, g, dtype, st)                                                       \
  do {                                                                                           \
    const dim3 grid_(grid_for(n));                                                               \
    if ((g).wfmt == WF_MXFP8)                                                                    \
      hipLaunchKernelGGL((KERN<bf16_t, WF_MXFP8>), grid_, dim3(NTHR), 0, st, g);                 \
    else if ((g).wfmt == WF_MXFP4)                                                               \
      hipLaunchKernelGGL((KERN<bf16_t, WF_MXFP4>), grid_, dim3(NTHR), 0, st, g);                 \
    else if ((dtype) == MOE_BF16)                                                                \
      hipLaunchKernelGGL((KERN<bf16_t, WF_DTYPE>), grid_, dim3(NTHR), 0, st, g);                 \
    else                                                                                         \
      hipLaunchKernelGGL((KERN<float, WF_DTYPE>), grid_, dim3(NTHR), 0, st, g);                  \
  } while (0)

template <bool ATOMIC>
struct RoutedKernel {
  template <typename T, int WM>
  static void launch(dim3 grid, const GemmArgs& g, hipStream_t st) {
    hipLaunchKernelGGL((moe_down_routed_kernel<T, ATOMIC, WM>), grid, dim3(NTHR), 0, st, g);
  }
};

hipError_t launch_gate_up(const GemmArgs& g, int dtype, hipStream_t st) {
  const long n = (long)g.mt_shared * g.nt_shared + (long)g.mt_routed * g.nt_routed;
  if (n <= 0) return hipSuccess;
  GEMM_LAUNCH(moe_gate_up_kernel, n, g, dtype, st);
  return hipGetLastError();
}

hipError_t launch_down_shared(const GemmArgs& g, int dtype, hipStream_t st) {
  const long n = (long)g.mt_shared * g.nt_shared;
  if (n <= 0) return hipSuccess;
  GEMM_LAUNCH(moe_down_shared_kernel, n, g, dtype, st);
  return hipGetLastError();
}

hipError_t launch_down_both(const GemmArgs& g, int dtype, hipStream_t st) {
  const long n = (long)g.mt_shared * g.nt_shared + (long)g.mt_routed * g.nt_routed;
  if (n <= 0) return hipSuccess;
  GEMM_LAUNCH(moe_down_kernel, n, g, dtype, st);
  return hipGetLastError();
}

template <bool ATOMIC>
static void launch_routed(const GemmArgs& g, int dtype, dim3 grid, hipStream_t st) {
  if (g.wfmt == WF_MXFP8) RoutedKernel<ATOMIC>::template launch<bf16_t, WF_MXFP8>(grid, g, st);
  else if (g.wfmt == WF_MXFP4) RoutedKernel<ATOMIC>::template launch<bf16_t, WF_MXFP4>(grid, g, st);
  else if (dtype == MOE_BF16) RoutedKernel<ATOMIC>::template launch<bf16_t, WF_DTYPE>(grid, g, st);
  else RoutedKernel<ATOMIC>::template launch<float, WF_DTYPE>(grid, g, st);
}

hipError_t launch_down_routed(const GemmArgs& g, int dtype, bool atomic, hipStream_t st) {
  const long n = (long)g.mt_routed * g.nt_routed;
  if (n <= 0) return hipSuccess;
  const dim3 grid(grid_for(n));
  if (atomic) launch_routed<true>(g, dtype, grid, st);
  else launch_routed<false>(g, dtype, grid, st);
  return hipGetLastError();
}
