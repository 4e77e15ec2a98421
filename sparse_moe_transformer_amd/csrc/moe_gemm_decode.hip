// Grouped expert GEMMs for decode-sized batches (bf16, gfx950): 32-row tiles.
//
// Same operands, tile order and outputs as the 128-row kernel in
// moe_gemm.hip (stacked [out, in] expert weights, mlxcel #845 "Checkpoint
// weight layout"; activation rows gathered by sorted_rows). With a handful of
// rows per expert the work is a stream of expert weights, so the tile is 32
// activation rows x 256 weight rows and the LDS holds four stages of 36 KiB
// (32 + 256 rows x 128 B of K): three K-steps of weights are in flight while
// one is computed, against two with the 128-row tile's 48 KiB stages
// (MXFP8 stages are 21 KiB: six of them when the K lengths allow).
//
// Four waves each own the 32 rows x 64 weight rows: for gate/up, 32 gate and
// the 32 up rows of the same columns (the activation is applied in
// registers); for down, 64 output columns. Two 32x32x16 bf16 MFMAs per
// sub-step.
//
// Persistent schedule and tile order as in moe_gemm.hip. Every K length is
// a multiple of the stage count in K-steps (four steps, 256 elements, or six
// for the six-stage MXFP8 kernels; the host checks); the last NST-1 steps of
// a tile load the next tile's first NST-1 stages. Every store of an epilogue is
// a buffer store whose offset is pushed past the buffer's range when the
// element is outside the tile, so each wave issues a fixed number of vector
// memory operations per tile and the load-counter waits of a tile's first
// steps can let the previous epilogue's stores stay in flight.
//
// MXFP8 expert weights (OCP MX: E4M3 codes, one E8M0 scale per 32 inputs,
// scales block-major [K/32, N]; the MXFP8 export of mlxcel #763
// "Validation"): a weight row holds 64 bytes per K-step, so the weight part
// of a stage is 16 KiB, and the step's two scale bytes of each row ride in
// the stage's spare LDS. Within a step the K order is permuted, the same way
// for both operands: lane half q takes inputs 32q .. 32q+31, sub-step s the
// eight at 32q + 8s, so a lane reads two 16-byte weight chunks and one scale
// per row and step. Codes become bf16 with the scaled conversion
// (v_cvt_scalef32_pk_bf16_fp8: exact for these values, the scale's exponent
// taken as the E8M0 value) and the bf16 MFMAs run unchanged.
//
// MXFP4 expert weights (E2M1 codes, two per byte, input 2j in the low nibble
// of byte j; the same scales): K-steps of 128 inputs, so a weight row holds
// 64 bytes per step in the MXFP8 64-input layout, the activation rows are
// stored as two 128-byte halves and the step's four scale blocks ride along
// as in the 128-input MXFP8 mode. Each 16-byte weight chunk is one scale
// block of 32 inputs; sub-step s of lane half q takes dword s % 4 of chunk
// 2q + s / 4 through the scaled fp4 conversion.
#include <algorithm>
#include <cstdlib>

#include "moe_common.h"
#include "moe_gemm_common.h"
#include "moe_kernels.h"
#include "moe_small_sort.h"

typedef float floatx16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int DBM = 32;        // activation rows per tile
constexpr int DBR = 256;       // weight rows per tile
constexpr int NCH = 8;         // 16-byte chunks per LDS row per K-step
constexpr int KSB = NCH * 16;  // bytes per row per K-step
constexpr int NTHR = 256;
// LDS stages: four (three K-steps of weights in flight while one is
// computed); MXFP8 stages are smaller, so six when every K length of the
// launch is a multiple of six steps.
// Weight modes: W_BF16; W_FP8 (MXFP8, K-steps of 64 inputs: 64-byte weight
// rows); W_FP8L (MXFP8, K-steps of 128 inputs: whole 128-byte weight rows,
// 256-byte activation rows, the step's four scale blocks); W_FP4 (MXFP4,
// K-steps of 128 inputs: 64-byte weight rows, 256-byte activation rows,
// four scale blocks).
constexpr int W_BF16 = 0, W_FP8 = 1, W_FP8L = 2, W_FP4 = 3;
// activation rows of a K-step stored as two 128-byte halves
template <int M>
constexpr bool halves() { return M == W_FP8L || M == W_FP4; }
// 64-byte weight rows per K-step (4 chunks, swz4 layout)
template <int M>
constexpr bool row64() { return M == W_FP8 || M == W_FP4; }
// bytes of a weight row of K inputs
template <int M>
__host__ __device__ constexpr int row_bytes(int K) { return M == W_BF16 ? 2 * K : M == W_FP4 ? K / 2 : K; }
// loads per thread per stage: activation + weight (+ scale)
template <int M>
constexpr int loads_of() {
  return M == W_BF16 ? 1 + 8 : M == W_FP8 ? 1 + 4 + 1 : M == W_FP4 ? 2 + 4 + 1 : 2 + 8 + 1;
}
// u32x4 index of the scale bytes inside a stage's weight part
template <int M>
constexpr int scales_at() { return row64<M>() ? 1024 : DBR * NCH; }
// inputs per K-step
template <int M>
constexpr int k_of() { return halves<M>() ? 128 : 64; }
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_WG_TILES = 128;
constexpr int EPI_GU = 16;     // vector memory ops of a gate/up epilogue (per thread)
constexpr int EPI_DN = 32;     // ... of a down epilogue

// A stage: the DBM activation rows (W_FP8L: two halves of 128 bytes per row,
// each laid out like a 128-byte step), then the weight rows (bf16 and
// W_FP8L: DBR x 128 B; W_FP8: DBR x 64 B) and, for MXFP8, the step's scale
// bytes (1 KiB), in 16-byte units.
template <int M>
constexpr int stage_a() { return halves<M>() ? 2 * DBM * NCH : DBM * NCH; }
template <int M>
constexpr int stage_u4() { return stage_a<M>() + (M == W_BF16 ? DBR * NCH : scales_at<M>() + 64); }
static_assert(4 * stage_u4<W_BF16>() * 16 <= 144 * 1024, "bf16 stages exceed their LDS budget");
static_assert(6 * stage_u4<W_FP8>() * 16 <= 128 * 1024, "MXFP8 stages exceed their LDS budget");
static_assert(3 * stage_u4<W_FP8L>() * 16 <= 128 * 1024, "MXFP8 stages exceed their LDS budget");
static_assert(4 * stage_u4<W_FP4>() * 16 <= 128 * 1024, "MXFP4 stages exceed their LDS budget");

// Wave w loads activation rows 8w .. 8w+7 (one instruction) and weight rows
// 64w + 8j .. +7 (instruction j < 8); the lane's row is that base + lane/8
// and it fetches the logical chunk that lands at physical chunk lane % 8.
__device__ __forceinline__ int a_row() { return 8 * (threadIdx.x >> 6) + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int b_row(int j) {
  return 64 * (threadIdx.x >> 6) + 8 * j + ((threadIdx.x & 63) >> 3);
}
__device__ __forceinline__ int lane_chunk(int row) { return (threadIdx.x & 7) ^ swz(row); }
// MXFP8 weight rows: 4 chunks of 16 B per step, chunk c of row r at c ^ swz4(r)
// (rows r .. r+15 then spread a chunk over every bank)
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int b_row_fp8(int j) {
  return 64 * (threadIdx.x >> 6) + 16 * j + ((threadIdx.x & 63) >> 2);
}

// Direct global->LDS loads (global_load_lds_dword / _dwordx4: each lane's
// bytes land at LDS address m0 + lane * size), issued from inline assembly so
// that the compiler does not track them: its tracking merges pending LDS
// writes conservatively at every join and then waits for all loads before the
// next LDS read. All waits for these loads are the explicit vmcnt waits and
// barriers of the step loop. Every direct load of this kernel goes through
// these two functions, so the compiler itself never relies on m0 here.
// a wave-uniform pointer, moved to scalar registers
__device__ __forceinline__ const char* sptr(const char* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}
// A kernel-argument pointer as an opaque scalar value. A select between two
// such values stays a scalar select; between the plain arguments the compiler
// turns it into a load from a selected argument address, one more dependent
// round trip.
template <typename T>
__device__ __forceinline__ T* sval(T* p) {
  uint64_t u = (uint64_t)(uintptr_t)p;
  asm volatile("" : "+s"(u));
  return reinterpret_cast<T*>((uintptr_t)u);
}
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, const void* lds) {
  const char* sbase = sptr(base);
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(l)
               : "memory");
}
__device__ __forceinline__ void dma4(const char* base, uint32_t voff, const void* lds) {
  const char* sbase = sptr(base);
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(l)
               : "memory");
}

// Loads use a scalar base that advances with the K-step and a 32-bit per-lane
// offset fixed for the whole tile: the offset registers stay live, so the
// compiler never reuses a load's address registers while the load is in
// flight (a reuse it would guard with a wait for every load).
struct DTile {
  const char* abase;  // activations (x, h or h_shared)
  const char* bbase;  // this wave's weight matrix (gate or up rows for gate/up)
  const char* sbase;  // MXFP8: this wave's scale matrix (block-major)
  uint32_t aoff;      // this lane's activation row + chunk, bytes from abase
  uint32_t boff[8];   // this lane's weight rows + chunks, bytes from bbase
  uint32_t soff;      // MXFP8: this lane's 4 scale bytes of the step's first block
  int sstep;          // MXFP8: scale bytes per K-step (two blocks)
  int nk;             // K-steps (a multiple of 4)
  int kseg;           // weight K segment length in bytes (K-split of shared down)
  int bstride;        // bytes between weight K segments (0: one segment)
  int shared, e, row0, nrows, n0, N;
};

// The loads of this lane for step j of tile t into stage (la, lb). Every K
// length is a multiple of the stage count in steps (the host checks), so
// there are no padding steps and no branch here: a branch would merge two
// load states and make the compiler wait for every load before the next LDS
// read.
template <int M>
__device__ __forceinline__ void issue_stage(const DTile& t, int j, u32x4_t* la, u32x4_t* lb) {
  const int w = threadIdx.x >> 6;
  const long kb = (long)j * (halves<M>() ? 2 * KSB : KSB);  // activation bytes per step
  const long wb = (long)j * (row64<M>() ? KSB / 2 : KSB);    // weight bytes per step
  long bk = wb;
  if (t.bstride) {
    const long seg = wb / t.kseg;
    bk = seg * t.bstride + (wb - seg * t.kseg);
  }
  const char* ab = t.abase + kb;
  const char* bb = t.bbase + bk;
  dma16(ab, t.aoff, la + 8 * w * NCH);
  if (halves<M>()) dma16(ab + KSB, t.aoff, la + DBM * NCH + 8 * w * NCH);
  if (row64<M>()) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(bb, t.boff[q], lb + (64 * w + 16 * q) * 4);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(bb, t.boff[q], lb + (64 * w + 8 * q) * NCH);
  }
  // scales: wave w loads rows 64w .. 64w+63 (W_FP8: lanes 0..31 for blocks
  // 0, 1, lanes 32..63 the same bytes again into the slot's unused half;
  // W_FP8L, W_FP4: lanes 16b .. 16b+15 block b)
  if (M != W_BF16)
    dma4(t.sbase + (long)j * t.sstep, t.soff,
         reinterpret_cast<const char*>(lb + scales_at<M>()) + 256 * w);
}

// First weight row (within the 256-row tile) of block nb (0..1) of wave w.
template <int KIND>
__device__ __forceinline__ int wrow(int w, int nb) {
  if (KIND == GATE_UP) return nb == 0 ? 32 * w : 128 + 32 * w;
  return 64 * w + 32 * nb;
}

typedef floatx16_t Acc2[2];

// One K-step (4 sub-steps of K = 16).
//   bf16 weights: lane l reads row l%32, chunk 2s + l/32.
//   MXFP8 weights: lane l takes inputs 32q + 8s .. +7 (q = l/32): activation
//   chunk 4q + s; weight bytes of chunks 2q, 2q+1 and the scale of block q.
template <int KIND, int M>
__device__ __forceinline__ void compute_stage(const u32x4_t* la, const u32x4_t* lb, Acc2& acc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 5, r = lane & 31;
  if (M == W_FP4) {
    // eight sub-steps: lane half q takes inputs 64q .. 64q+63 (activation
    // half q, weight chunks 2q, 2q+1 = scale blocks 2q, 2q+1), sub-step
    // s = 4h + s4 the eight at 64q + 8s: dword s4 of chunk 2q + h
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + scales_at<M>());
    const u32x4_t* lah = la + q * DBM * NCH;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t wv[2];
      float scale[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = wrow<KIND>(w, nb) + r;
        wv[nb] = lb[row * 4 + ((2 * q + h) ^ swz4(row))];
        scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * (2 * q + h) + (row & 63)]);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s = 4 * h + s4;
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, lah[r * NCH + (s ^ swz(r))]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4_t& c = wv[nb];
          const bf16x8_t fb =
              fp4x8_to_bf16(s4 == 0 ? c.x : s4 == 1 ? c.y : s4 == 2 ? c.z : c.w, scale[nb]);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[nb], 0, 0, 0);
        }
      }
    }
    return;
  }
  if (M == W_FP8L) {
    // eight sub-steps: lane half q takes inputs 64q .. 64q+63 (activation
    // half q, weight chunks 4q .. 4q+3, scale blocks 2q, 2q+1), sub-step s the
    // eight at 64q + 8s
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + scales_at<M>());
    const u32x4_t* lah = la + q * DBM * NCH;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t wv[2][2];
      float scale[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = wrow<KIND>(w, nb) + r;
        wv[nb][0] = lb[row * NCH + ((4 * q + 2 * h) ^ swz(row))];
        wv[nb][1] = lb[row * NCH + ((4 * q + 2 * h + 1) ^ swz(row))];
        scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * (2 * q + h) + (row & 63)]);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s = 4 * h + s4;
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, lah[r * NCH + (s ^ swz(r))]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4_t& c = wv[nb][s4 >> 1];
          const bf16x8_t fb = (s4 & 1) ? fp8x8_to_bf16(c.z, c.w, scale[nb])
                                       : fp8x8_to_bf16(c.x, c.y, scale[nb]);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[nb], 0, 0, 0);
        }
      }
    }
    return;
  }
  if (M == W_FP8) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + scales_at<M>());
    u32x4_t wv[2][2];
    float scale[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = wrow<KIND>(w, nb) + r;
      wv[nb][0] = lb[row * 4 + ((2 * q) ^ swz4(row))];
      wv[nb][1] = lb[row * 4 + ((2 * q + 1) ^ swz4(row))];
      scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * q + (row & 63)]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, la[r * NCH + ((4 * q + s) ^ swz(r))]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const u32x4_t& c = wv[nb][s >> 1];
        const bf16x8_t fb = (s & 1) ? fp8x8_to_bf16(c.z, c.w, scale[nb])
                                    : fp8x8_to_bf16(c.x, c.y, scale[nb]);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[nb], 0, 0, 0);
      }
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, la[r * NCH + ((2 * s + q) ^ swz(r))]);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = wrow<KIND>(w, nb) + r;
      const bf16x8_t fb = __builtin_bit_cast(bf16x8_t, lb[row * NCH + ((2 * s + q) ^ swz(row))]);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[nb], 0, 0, 0);
    }
  }
}

template <int KIND>
__device__ __forceinline__ int tile_count(const GemmArgs& g, const int* cum) {
  if (KIND == DOWN_SHARED) return g.mt_shared * g.nt_shared;
  if (KIND == DOWN_ROUTED) return cum[g.E] * g.nt_routed;
  return g.mt_shared * g.nt_shared + cum[g.E] * g.nt_routed;
}

// Where tile `idx` is: row0 (x), nrows | shared << 16 (y), expert (z),
// n-tile (w). Offsets and the prefix are in LDS.
template <int KIND>
__device__ __forceinline__ int4 place_of(const GemmArgs& g, const int* offs, const int* cum,
                                         int idx) {
  const int nshared = KIND == DOWN_ROUTED ? 0 : g.mt_shared * g.nt_shared;
  int mt, nt, e = 0, row0, nrows, shared;
  if (idx < nshared) {
    shared = 1;
    grouped_order(idx, g.mt_shared, g.nt_shared, g.gm_shared, &mt, &nt);
    row0 = mt * DBM;
    nrows = min(DBM, g.T - row0);
  } else {
    shared = 0;
    const int t = idx - nshared;
    e = owner(cum, g.E, t / g.nt_routed);
    const int ms = cum[e + 1] - cum[e];
    grouped_order(t - cum[e] * g.nt_routed, ms, g.nt_routed, g.gm_routed, &mt, &nt);
    row0 = offs[e] + mt * DBM;
    nrows = min(DBM, offs[e + 1] - row0);
  }
  return make_int4(row0, nrows | (shared << 16), e, nt);
}

// Row ids of a tile's (up to 32) activation rows, gathered by wave 0 straight
// into LDS (dst: 64 ints) with one direct global->LDS load, a tile ahead of
// their use. Kept out of registers on purpose: a register loaded from memory
// in one tile and read in the next makes the compiler drain every load in
// flight before the read. Lanes past the tile's rows repeat its last row.
__device__ __forceinline__ void gather_rows(const GemmArgs& g, int4 p, int* dst) {
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63;
  const int nrows = p.y & 0xFFFF;
  dma4(reinterpret_cast<const char*>(g.sorted_rows),
       (uint32_t)(p.x + min(lane, nrows - 1)) * 4u, dst);
}

// The token of this lane's activation row of gate/up tile p (rows: the tile's
// gathered row ids in LDS).
__device__ __forceinline__ int token_of(const GemmArgs& g, int4 p, const int* rows) {
  const int row0 = p.x, nrows = p.y & 0xFFFF, shared = p.y >> 16;
  const int R = min(a_row(), nrows - 1);
  return shared ? row0 + R : div_k(rows[R], g.k, g.kmagic);
}

// The scale bytes this lane loads for MXFP8 tile rows 64w .. 64w+63 of
// the stage: lanes 0..31 cover (block l/16, four rows from 4 * (l%16)),
// lanes 32..63 repeat them. col(tr) maps a tile row to its matrix column.
__device__ __forceinline__ int scale_lane_row() { return 64 * (threadIdx.x >> 6) + 4 * (threadIdx.x & 15); }
__device__ __forceinline__ int scale_lane_block() { return (threadIdx.x >> 4) & 1; }

// tok: gate/up only, the token of this lane's activation row (token_of).
template <int KIND, int M>
__device__ __forceinline__ void make_tile(const GemmArgs& g, int4 p, int tok, DTile& t) {
  constexpr int EPC = 8;
  constexpr bool FP8 = M != W_BF16;  // MX weights (MXFP8 or MXFP4)
  // W_FP8: lanes 32..63 repeat the scale bytes of lanes 0..31; W_FP8L and
  // W_FP4: lane l takes block l / 16
  const int sblock = halves<M>() ? (threadIdx.x & 63) >> 4 : scale_lane_block();
  constexpr int SBLK = halves<M>() ? 4 : 2;  // scale blocks per K-step
  const int H = g.H;
  t.row0 = p.x;
  t.nrows = p.y & 0xFFFF;
  t.shared = p.y >> 16;
  t.e = p.z;
  const int nt = p.w;
  const int row = a_row();
  // the wave index as a scalar: the gate / up weight and scale pointers are
  // then picked with scalar selects (from a per-lane index the compiler
  // loads the chosen kernel argument with a vector load, whose wait would
  // also drain the weight loads in flight)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (KIND == GATE_UP) {
    t.n0 = nt * 128;
    t.N = t.shared ? g.S * g.Is : g.I;
    t.abase = static_cast<const char*>(g.a);
    t.aoff = ((uint32_t)tok * (uint32_t)H + (uint32_t)(lane_chunk(row) * EPC)) * 2u;
    // waves 0, 1 load gate rows (weight rows 0..127), waves 2, 3 the up rows
    const char* wm = static_cast<const char*>(w < 2 ? (t.shared ? sval(g.ws0) : sval(g.w0))
                                                    : (t.shared ? sval(g.ws1) : sval(g.w1)));
    const uint32_t rb = (uint32_t)row_bytes<M>(H);
    t.bbase = wm + (t.shared ? 0 : (size_t)t.e * g.I * rb);
    if (row64<M>()) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int br = b_row_fp8(j);
        const uint32_t n = (uint32_t)min(t.n0 + (br & 127), t.N - 1);
        t.boff[j] = n * rb + (uint32_t)(((threadIdx.x & 3) ^ swz4(br)) * 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int br = b_row(j);
        const uint32_t n = (uint32_t)min(t.n0 + (br & 127), t.N - 1);
        t.boff[j] = n * rb + (uint32_t)(lane_chunk(br) * 16);
      }
    }
    if (FP8) {
      // scales [., H/32, N_s] per matrix; the shared experts are S matrices
      // of width Is one after another (one, slot E, when packed), so a
      // shared column n is column n - s*Is of matrix s = n / Is
      const int ns = t.shared ? g.Is : g.I;
      const uint8_t* sm = w < 2 ? (t.shared ? sval(g.sws0) : sval(g.sw0))
                                : (t.shared ? sval(g.sws1) : sval(g.sw1));
      const int n = min(t.n0 + (scale_lane_row() & 127), t.N - 4);
      const int se = t.shared ? n / ns : 0;
      t.sbase = reinterpret_cast<const char*>(sm) + (t.shared ? 0 : (size_t)t.e * (H / 32) * ns);
      t.soff = (uint32_t)((size_t)se * (H / 32) * ns + (n - se * ns) + (size_t)sblock * ns);
      t.sstep = SBLK * ns;
    }
    t.nk = H / k_of<M>();
    t.kseg = (int)rb;
    t.bstride = 0;
  } else {
    // down: shared tiles read h_shared [T, S*Is] against the S shared down
    // matrices [H, Is] (K segment s at ws_down + s*H*Is); routed tiles read
    // h [T*k, I] against expert e's down matrix [H, I]
    const bool sh = KIND == DOWN_SHARED || (KIND == DOWN_BOTH && t.shared);
    const int Ks = sh ? g.S * g.Is : g.I;
    const int ldb = sh ? g.Is : g.I;
    t.abase = static_cast<const char*>(KIND == DOWN_BOTH && sh ? g.a_shared : g.a);
    const uint32_t rb = (uint32_t)row_bytes<M>(ldb);  // bytes per weight row of a K segment
    t.bbase = sh ? static_cast<const char*>(g.ws0)
                 : static_cast<const char*>(g.w0) + (size_t)t.e * H * row_bytes<M>(g.I);
    t.n0 = nt * DBR;
    t.N = H;
    const uint32_t arow = (uint32_t)(t.row0 + min(row, t.nrows - 1));
    t.aoff = (arow * (uint32_t)Ks + (uint32_t)(lane_chunk(row) * EPC)) * 2u;
    if (row64<M>()) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int br = b_row_fp8(j);
        const uint32_t n = (uint32_t)min(t.n0 + br, H - 1);
        t.boff[j] = n * rb + (uint32_t)(((threadIdx.x & 3) ^ swz4(br)) * 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int br = b_row(j);
        const uint32_t n = (uint32_t)min(t.n0 + br, H - 1);
        t.boff[j] = n * rb + (uint32_t)(lane_chunk(br) * 16);
      }
    }
    if (FP8) {
      // scales [K/32, H]: the S shared matrices' blocks follow one another
      // along K, so a shared tile's K-step j always reads blocks 2j, 2j+1
      const uint8_t* sm = sh ? g.sws0 : g.sw0 + (size_t)t.e * (g.I / 32) * H;
      const int n = min(t.n0 + scale_lane_row(), H - 4);
      t.sbase = reinterpret_cast<const char*>(sm);
      t.soff = (uint32_t)(n + sblock * H);
      t.sstep = SBLK * H;
    }
    t.nk = Ks / k_of<M>();
    t.kseg = (int)rb;
    t.bstride = sh && g.S > 1 ? H * (int)rb : 0;
  }
}

// Buffer resource over [p, p + 2^31): the hardware range check drops stores
// at offsets >= 2^31, which masks elements without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, 0x7FFFFFFF, 0x00020000);
}
constexpr uint32_t kDropped = 0x80000000u;

// Epilogue: exactly EPI_GU (gate/up) or EPI_DN (down) buffer stores or
// atomics per thread, masked by offset. Lane (q, r) holds rows
// acc_row(0, v, q) of column r of each 32-column block.
template <int KIND, bool ATOMIC>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const DTile& cur, const Acc2& acc,
                                         const int* ep_tok, const float* ep_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 5, r = lane & 31;
  if (KIND == GATE_UP) {
    bf16_t* dst = static_cast<bf16_t*>(cur.shared ? g.out_shared : g.out);
    const int ld = cur.shared ? g.S * g.Is : g.I;
    const int c = cur.n0 + 32 * w + r;
    const __amdgpu_buffer_rsrc_t rs = out_rsrc(dst + (size_t)cur.row0 * ld);
    const bool cok = c < cur.N;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = acc_row(0, v, q);
      const bool ok = cok && m < cur.nrows;
      __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(act_apply(acc[0][v], acc[1][v], g.act)),
                                            rs, ok ? (uint32_t)(m * ld + c) * 2u : kDropped, 0, 0);
    }
    return;
  }
  const int c0 = cur.n0 + 64 * w + r;
  const bool sh = KIND == DOWN_SHARED || (KIND == DOWN_BOTH && cur.shared);
  if (sh || !ATOMIC) {
    if (sh) {
      // shared rows: fp32 into acc (weight exactly 1)
      const __amdgpu_buffer_rsrc_t rs =
          out_rsrc(static_cast<float*>(g.out) + (size_t)cur.row0 * g.H);
#pragma unroll
      for (int v = 0; v < 16; ++v)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int m = acc_row(0, v, q), c = c0 + 32 * nb;
          const bool ok = c < cur.N && m < cur.nrows;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[nb][v]), rs,
                                                ok ? (uint32_t)(m * g.H + c) * 4u : kDropped, 0, 0);
        }
    } else {
      // routed rows, unweighted, into y_perm (moe_combine sums them in a fixed order)
      const __amdgpu_buffer_rsrc_t rs =
          out_rsrc(static_cast<bf16_t*>(g.y_perm) + (size_t)cur.row0 * g.H);
#pragma unroll
      for (int v = 0; v < 16; ++v)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int m = acc_row(0, v, q), c = c0 + 32 * nb;
          const bool ok = c < cur.N && m < cur.nrows;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[nb][v]), rs,
                                                ok ? (uint32_t)(m * g.H + c) * 2u : kDropped, 0, 0);
        }
    }
  } else {
    // routed rows, weighted by topk_w, added into acc[token] with fp32 atomics
    const __amdgpu_buffer_rsrc_t rs = out_rsrc(g.out);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = acc_row(0, v, q);
      const int tok = ep_tok[m];
      const float wt = ep_w[m];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int c = c0 + 32 * nb;
        const bool ok = c < cur.N && m < cur.nrows;
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
            wt * acc[nb][v], rs, ok ? (uint32_t)((size_t)tok * g.H + c) * 4u : kDropped, 0, 0);
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// The persistent kernel. Step j of a tile: wait until this wave's loads of
// stage j have landed (only the two younger stages, plus the previous tile's
// epilogue stores in a tile's first three steps, may still be in flight),
// barrier, issue the loads of step j+3 into the stage freed at step j-1
// (the next tile's first stages when j+3 passes the end), compute stage j.
template <int KIND, bool ATOMIC, int M, int NST>
__device__ __forceinline__ void decode_body(const GemmArgs& g) {
  constexpr int STAGE = stage_u4<M>();
  constexpr int STAGE_A = stage_a<M>();
  __shared__ __align__(16) u32x4_t lds_st[NST][STAGE];
  __shared__ int offs[MAX_EXPERTS + 1];
  __shared__ int cum[MAX_EXPERTS + 1];
  __shared__ int4 places[MAX_WG_TILES];
  __shared__ int rows_buf[3][64];  // gathered row ids of tiles li, li+1, li+2 (slot i % 3)
  __shared__ int sorted[KIND == GATE_UP ? 256 : 1];  // grouped rows, when this kernel groups
  __shared__ int ep_tok[2][64];    // atomic down epilogue: token and weight of each
  __shared__ float ep_w[2][64];    // row (by tile parity: written while the other
                                   // waves may still read the previous tile's)

  // gate/up of a small decode batch: group the routed rows here (scratch in
  // stage 0, before any load into it); workgroup 0 also stores the grouping
  // for the later stages
  const bool grouped_here = KIND == GATE_UP && g.topk_idx != nullptr;
  if (grouped_here) {
    static_assert(sizeof(lds_st[0]) >= (256 + 3 * MAX_EXPERTS + 4) * sizeof(int),
                  "a stage holds the grouping scratch");
    int* scratch = reinterpret_cast<int*>(lds_st[0]);
    const bool pub = blockIdx.x == 0;
    block_sort_rows_256(g.topk_idx, g.T, g.k, g.E, scratch, offs, sorted,
                        pub ? g.offsets_out : nullptr, pub ? g.sorted_out : nullptr,
                        pub ? g.row_pos_out : nullptr);
  }
  if (KIND != DOWN_SHARED) build_tile_prefix<DBM>(grouped_here ? offs : g.offsets, g.E, offs, cum);
  __syncthreads();
  const int ntiles = tile_count<KIND>(g, cum);
  const WgTiles wt = wg_tiles(ntiles, KIND == DOWN_BOTH ? g.mt_shared * g.nt_shared : 0);
  const int n_my = wt.n_my;
  if (n_my == 0) return;
  for (int i = threadIdx.x; i < min(n_my, MAX_WG_TILES); i += NTHR)
    places[i] = place_of<KIND>(g, offs, cum, wt.global(i));
  __syncthreads();
  auto place = [&](int i) -> int4 {
    i = min(i, n_my - 1);
    const int4 p = i < MAX_WG_TILES ? places[i] : place_of<KIND>(g, offs, cum, wt.global(i));
    return make_int4(__builtin_amdgcn_readfirstlane(p.x), __builtin_amdgcn_readfirstlane(p.y),
                     __builtin_amdgcn_readfirstlane(p.z), __builtin_amdgcn_readfirstlane(p.w));
  };

  constexpr int EPI = KIND == GATE_UP ? EPI_GU : EPI_DN;
  constexpr int LOADS = loads_of<M>();
  // the row ids of tile i: from the grouping in LDS, or gathered into
  // rows_buf slot i % 3
  auto rows_of = [&](int i) -> const int* {
    return grouped_here ? sorted + place(i).x : rows_buf[i % 3];
  };
  const bool ROWS = (KIND == GATE_UP && !grouped_here) || (KIND == DOWN_ROUTED && ATOMIC);
  if (ROWS) {
    gather_rows(g, place(0), rows_buf[0]);
    gather_rows(g, place(1), rows_buf[1]);
    // the first tile's row ids are read right away (later gathers are a tile
    // ahead: waited for by wave 0's step waits and published by the step
    // barriers)
    wait_vmcnt<0>();
    __syncthreads();
  }
  DTile cur, nxt;
  make_tile<KIND, M>(g, place(0), KIND == GATE_UP ? token_of(g, place(0), rows_of(0)) : 0, cur);
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue_stage<M>(cur, st, lds_st[st], lds_st[st] + STAGE_A);

  bool first = true;
  for (int li = 0;; ++li) {
    const bool has_next = li + 1 < n_my;
    // the next tile (its row ids were gathered a tile ago), then the row ids
    // of the one after it
    make_tile<KIND, M>(g, place(li + 1),
                    KIND == GATE_UP ? token_of(g, place(li + 1), rows_of(li + 1)) : 0, nxt);
    if (KIND == DOWN_ROUTED && ATOMIC && threadIdx.x < 64) {
      // this tile's rows: token and routing weight of each (the weights are
      // gathered straight into LDS as well)
      const int r = rows_buf[li % 3][threadIdx.x];
      ep_tok[li & 1][threadIdx.x] = div_k(r, g.k, g.kmagic);
      dma4(reinterpret_cast<const char*>(g.topk_w), (uint32_t)r * 4u, ep_w[li & 1]);
    }
    if (ROWS) gather_rows(g, place(li + 2), rows_buf[(li + 2) % 3]);
    // after the last tile, the look-ahead reloads its own first stages (never read)
    const int nk4 = cur.nk;
    Acc2 acc;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nb][v] = 0.f;

#define DEC_STEP(J, TL, JL, SC, SN)                                                     \
  {                                                                                    \
    if ((J) < NST - 1 && !first) wait_vmcnt<(NST - 2) * LOADS + EPI>();                \
    else wait_vmcnt<(NST - 2) * LOADS>();                                              \
    __builtin_amdgcn_s_barrier();                                                      \
    issue_stage<M>(TL, JL, lds_st[SN], lds_st[SN] + STAGE_A);                          \
    compute_stage<KIND, M>(lds_st[SC], lds_st[SC] + STAGE_A, acc);                     \
  }
    // a group of NST steps uses stages 0 .. NST-1 and loads NST-1 steps ahead;
    // the tile's last group loads its last step and the next tile's first
    // NST-1 steps (nk is a multiple of NST)
    int j = 0;
    for (; j + NST < nk4; j += NST) {
#pragma unroll
      for (int u = 0; u < NST; ++u) DEC_STEP(j + u, cur, j + u + NST - 1, u, (u + NST - 1) % NST)
    }
    DEC_STEP(j, cur, j + NST - 1, 0, NST - 1)
#pragma unroll
    for (int u = 1; u < NST; ++u) DEC_STEP(j + u, nxt, u - 1, u, u - 1)
#undef DEC_STEP
    epilogue<KIND, ATOMIC>(g, cur, acc, ep_tok[li & 1], ep_w[li & 1]);
    if (!has_next) break;
    first = false;
    cur = nxt;
  }
  // the look-ahead loads after the last tile are not used: let them land
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
}

template <int M, int NST>
__global__ void __launch_bounds__(NTHR) moe_gate_up_decode_kernel(GemmArgs g) {
  decode_body<GATE_UP, false, M, NST>(g);
}
template <int M, int NST>
__global__ void __launch_bounds__(NTHR) moe_down_decode_kernel(GemmArgs g) {
  decode_body<DOWN_BOTH, false, M, NST>(g);
}
template <int M, int NST>
__global__ void __launch_bounds__(NTHR) moe_down_shared_decode_kernel(GemmArgs g) {
  decode_body<DOWN_SHARED, false, M, NST>(g);
}
template <int M, int NST>
__global__ void __launch_bounds__(NTHR) moe_down_routed_decode_kernel(GemmArgs g) {
  decode_body<DOWN_ROUTED, false, M, NST>(g);
}
template <int M, int NST>
__global__ void __launch_bounds__(NTHR) moe_down_routed_atomic_decode_kernel(GemmArgs g) {
  decode_body<DOWN_ROUTED, true, M, NST>(g);
}

// ---------------------------------------------------------------------------
// Fused expert FFN of a small decode batch (bf16 weights; at most 32 tokens
// and 256 routed rows; H = 256 * NT2 with NT2 = 2 or 4; the routed and
// shared intermediate widths multiples of 128; E <= FFN_MAX_E).
//
// An expert's output down(act(gate x, up x)) (mlxcel #845 "Routing detail")
// is a sum over the columns of h, so it splits into 128-column slices of I:
// a work item is slice c of one expert (or of the shared experts' combined
// width). Phase 1 is the gate/up tile above for n-tile c (K = H); its
// epilogue keeps the activated 32 x 128 slice as bf16 in LDS, the values the
// two-kernel path stores to h. Phase 2 multiplies that slice by columns
// 128c .. 128c+127 of the down matrix for all H outputs: NT2 n-tiles of 256
// weight rows, two 64-input K-steps each, accumulated side by side. Both
// phases stream weight K-steps through the same four LDS stages, so the
// weight stream runs on from the gate/up rows into the down rows and into
// the next item. Phase-2 stages still carry the activation rows' load (of x,
// never read) so that every stage is the same nine loads per thread and the
// fixed load-counter waits hold. The fp32 product of slice c for routed row
// r = t*k + j goes to row r of partial plane c (shared slices: row t of the
// shared planes); the combine adds a row's planes in plane order and then
// weights the sum. Phase-2 MFMAs take the weight rows as the A operand, so a
// lane holds four consecutive output columns of one row and stores them at
// once.
//
// Schedule. The potential items are the ns = S*Is/128 shared slices, then
// slice q % (I/128) of expert q / (I/128) for q = p - ns. Workgroup b owns
// potential item b and issues the weight loads of its first three K-steps
// at once, before it knows whether the expert was chosen by any token (the
// shared slices, first, always run at once); meanwhile it
// copies the routed experts to LDS and works out, the same way in every
// workgroup, which items are real and who runs those beyond the grid. A
// workgroup whose own item is real keeps its loads and adds only the
// activation rows; the real items beyond the grid go one each to the
// workgroups whose own item is not (in order), any left over round-robin to
// all workgroups.
namespace {

constexpr int FFN_CH = 128;      // intermediate columns per work item
constexpr int FFN_MAX_E = 256;
constexpr int FFN_MAX_ITEMS = 8; // work items per workgroup (the host checks)
constexpr int FFN_MAX_GRID = 256;
static_assert(FFN_MAX_E % 64 == 0, "chosen-expert mask words");

// Phase-2 weight rows of an item: columns 128c .. 128c+127 of the down
// matrix (routed: expert e's [H, I]; shared: matrix s of the S [H, Is]
// matrices, the one that holds concatenated column 128c), every H row; MX
// weights also the slice's four scale blocks.
struct FTile {
  const char* bbase;  // row 0 of the slice's down matrix, at the slice's first input
  const char* sbase;  // MX: the slice's first scale block of that matrix
  uint32_t boff[8];   // this lane's rows (within a 256-row n-tile) + chunks
  uint32_t soff;      // MX: this lane's scale bytes within the step's blocks
  int rb;             // bytes per down-matrix row
};

template <int M>
__device__ __forceinline__ void make_ftile(const GemmArgs& g, int4 p, FTile& f) {
  const int shared = p.y >> 16, e = p.z;
  const int col = p.w * FFN_CH;
  const int s = shared ? col / g.Is : 0;
  const int K = shared ? g.Is : g.I;      // inputs per down-matrix row
  const int c0 = col - s * g.Is * shared;  // the slice's first column in that matrix
  f.rb = row_bytes<M>(K);
  const char* mat = shared ? static_cast<const char*>(g.ws2) + (size_t)s * g.H * f.rb
                           : static_cast<const char*>(g.w2) + (size_t)e * g.H * f.rb;
  f.bbase = mat + row_bytes<M>(c0);
  if (M != W_BF16) {
    // scales [K/32, H] per matrix; lanes 16b .. 16b+15 load block b
    const uint8_t* sm = shared ? g.sws2 + (size_t)s * (K / 32) * g.H
                               : g.sw2 + (size_t)e * (K / 32) * g.H;
    f.sbase = reinterpret_cast<const char*>(sm) + (size_t)(c0 / 32) * g.H;
    f.soff = (uint32_t)(scale_lane_row() + ((threadIdx.x & 63) >> 4) * g.H);
  }
  if (row64<M>()) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int br = b_row_fp8(j);
      f.boff[j] = (uint32_t)br * (uint32_t)f.rb + (uint32_t)(((threadIdx.x & 3) ^ swz4(br)) * 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int br = b_row(j);
      f.boff[j] = (uint32_t)br * (uint32_t)f.rb + (uint32_t)(lane_chunk(br) * 16);
    }
  }
}

// activation-row loads per stage: one, or two 128-byte halves
template <int M>
constexpr int a_loads() { return halves<M>() ? 2 : 1; }

// The activation-row loads of gate/up K-step j, then its weight-row loads
// (with the scale bytes of MX weights): together the loads of issue_stage.
template <int M>
__device__ __forceinline__ void issue_gu_a(const DTile& t, int j, u32x4_t* la) {
  const int w = threadIdx.x >> 6;
  const char* ab = t.abase + (long)j * (halves<M>() ? 2 * KSB : KSB);
  dma16(ab, t.aoff, la + 8 * w * NCH);
  if (halves<M>()) dma16(ab + KSB, t.aoff, la + DBM * NCH + 8 * w * NCH);
}
template <int M>
__device__ __forceinline__ void weight_rows(const char* bb, const uint32_t (&boff)[8],
                                            u32x4_t* lb) {
  const int w = threadIdx.x >> 6;
  if (row64<M>()) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(bb, boff[q], lb + (64 * w + 16 * q) * 4);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(bb, boff[q], lb + (64 * w + 8 * q) * NCH);
  }
}
template <int M>
__device__ __forceinline__ void issue_gu_b(const DTile& t, int j, u32x4_t* lb) {
  weight_rows<M>(t.bbase + (long)j * (row64<M>() ? KSB / 2 : KSB), t.boff, lb);
  if (M != W_BF16)
    dma4(t.sbase + (long)j * t.sstep, t.soff,
         reinterpret_cast<const char*>(lb + scales_at<M>()) + 256 * (threadIdx.x >> 6));
}

// Loads of phase-2 step jj: n-tile jj / SPN, K-step jj % SPN of the slice
// (SPN = 128 / inputs per K-step: two bf16 steps, one MX step): the
// activation rows of gate/up K-step jj (x, not read), 256 down-matrix rows
// and their scale bytes.
template <int M>
__device__ __forceinline__ void issue_ffn_down(const DTile& t, const FTile& f, int jj,
                                               u32x4_t* la, u32x4_t* lb) {
  constexpr int SPN = FFN_CH / k_of<M>();
  issue_gu_a<M>(t, jj, la);
  const int nt = jj / SPN, kk = jj % SPN;
  weight_rows<M>(f.bbase + (long)nt * 256 * f.rb + (long)kk * (row64<M>() ? KSB / 2 : KSB),
                 f.boff, lb);
  if (M != W_BF16)
    dma4(f.sbase + (long)nt * 256, f.soff,
         reinterpret_cast<const char*>(lb + scales_at<M>()) + 256 * (threadIdx.x >> 6));
}

// One phase-2 K-step: h slice rows (la: the LDS copy, one 64-input block
// for bf16, both for MX) against the stage's down rows, the weights as the
// MFMA's A operand (so the accumulators hold output columns down a lane's
// four rows); wave w owns output columns 64w .. 64w+63 of the n-tile, block
// nb the 32 at 64w + 32nb. The fragments and conversions are those of
// compute_stage for the same weight mode.
template <int M>
__device__ __forceinline__ void compute_ffn_down(const u32x4_t* la, const u32x4_t* lb, Acc2& acc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 5, r = lane & 31;
  if (M == W_FP4) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + scales_at<M>());
    const u32x4_t* lah = la + q * DBM * NCH;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t wv[2];
      float scale[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = 64 * w + 32 * nb + r;
        wv[nb] = lb[row * 4 + ((2 * q + h) ^ swz4(row))];
        scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * (2 * q + h) + (row & 63)]);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s = 4 * h + s4;
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, lah[r * NCH + (s ^ swz(r))]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4_t& c = wv[nb];
          const bf16x8_t fb =
              fp4x8_to_bf16(s4 == 0 ? c.x : s4 == 1 ? c.y : s4 == 2 ? c.z : c.w, scale[nb]);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc[nb], 0, 0, 0);
        }
      }
    }
    return;
  }
  if (M == W_FP8L) {
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(lb + scales_at<M>());
    const u32x4_t* lah = la + q * DBM * NCH;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t wv[2][2];
      float scale[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = 64 * w + 32 * nb + r;
        wv[nb][0] = lb[row * NCH + ((4 * q + 2 * h) ^ swz(row))];
        wv[nb][1] = lb[row * NCH + ((4 * q + 2 * h + 1) ^ swz(row))];
        scale[nb] = e8m0_scale(sc[256 * (row >> 6) + 64 * (2 * q + h) + (row & 63)]);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s = 4 * h + s4;
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, lah[r * NCH + (s ^ swz(r))]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4_t& c = wv[nb][s4 >> 1];
          const bf16x8_t fb = (s4 & 1) ? fp8x8_to_bf16(c.z, c.w, scale[nb])
                                       : fp8x8_to_bf16(c.x, c.y, scale[nb]);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc[nb], 0, 0, 0);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, la[r * NCH + ((2 * s + q) ^ swz(r))]);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int row = 64 * w + 32 * nb + r;
      const bf16x8_t fb = __builtin_bit_cast(bf16x8_t, lb[row * NCH + ((2 * s + q) ^ swz(row))]);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc[nb], 0, 0, 0);
    }
  }
}

// Phase-1 epilogue: act(gate, up) as bf16 into the LDS slice (two K-steps of
// 64 columns, rows laid out like a stage's activation rows). Lane (q, r) of
// wave w holds column 32w + r of rows acc_row(0, v, q).
__device__ __forceinline__ void ffn_h_to_lds(const GemmArgs& g, const Acc2& acc, u32x4_t* lds_h) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 5, r = lane & 31;
  const int ch = 4 * (w & 1) + (r >> 3);
  uint16_t* hb = reinterpret_cast<uint16_t*>(lds_h + (w >> 1) * DBM * NCH);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = acc_row(0, v, q);
    hb[(m * NCH + (ch ^ swz(m))) * 8 + (r & 7)] =
        f32_to_bf16_bits(act_apply(acc[0][v], acc[1][v], g.act));
  }
}

// Phase-2 epilogue: 2 * NT2 * 4 16-byte stores per thread into the item's
// partial plane (routed planes [I/128][T*k][H] by routed row, then the
// shared [S*Is/128][T][H] by token); rows past the item's are pushed out of
// range. rows: the item's row ids (LDS).
template <int NT2>
__device__ __forceinline__ void ffn_epilogue(const GemmArgs& g, int4 p, const int* rows,
                                             const Acc2 (&dacc)[NT2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 5, r = lane & 31;
  const int nrows = p.y & 0xFFFF, shared = p.y >> 16, c = p.w;
  const size_t routed_rows = (size_t)g.T * g.k;
  float* plane = shared ? g.parts + ((size_t)g.nt_routed * routed_rows + (size_t)c * g.T) * g.H
                        : g.parts + (size_t)c * routed_rows * g.H;
  const __amdgpu_buffer_rsrc_t rs = out_rsrc(plane);
  const bool ok = r < nrows;
  const uint32_t row = (uint32_t)rows[min(r, nrows - 1)];
#pragma unroll
  for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int n = nt * 256 + 64 * w + 32 * nb + acc_row(0, 4 * v4, q);
        const u32x4_t val = {__float_as_uint(dacc[nt][nb][4 * v4]),
                             __float_as_uint(dacc[nt][nb][4 * v4 + 1]),
                             __float_as_uint(dacc[nt][nb][4 * v4 + 2]),
                             __float_as_uint(dacc[nt][nb][4 * v4 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(
            val, rs, ok ? (row * (uint32_t)g.H + (uint32_t)n) * 4u : kDropped, 0, 0);
      }
}

// Potential item p as a place (row-list slot 0, nrows, expert, slice).
__device__ __forceinline__ int4 ffn_potential(const GemmArgs& g, int p, int nrows) {
  const int nr = g.nt_routed;
  const int ns = g.nt_shared;
  if (p < ns) return make_int4(0, nrows | (1 << 16), 0, p);
  return make_int4(0, nrows, (p - ns) / nr, (p - ns) % nr);
}

// The token of this lane's activation row (rows: the item's row ids).
__device__ __forceinline__ int ffn_token(const GemmArgs& g, int4 p, const int* rows) {
  const int R = min(a_row(), (p.y & 0xFFFF) - 1);
  return (p.y >> 16) ? rows[R] : div_k(rows[R], g.k, g.kmagic);
}

}  // namespace

// For the own first item the weight loads of its first NST-1 K-steps went
// out before their activation loads: the loads younger than stage s's are
// the activation loads of the later early stages and the full stages issued
// since.
template <int NST, int AL, int LOADS>
__device__ __forceinline__ void spec_wait(int s) {
  static_assert(NST >= 3 && NST <= 4, "the early steps below");
  if (s == 0) wait_vmcnt<(NST - 2) * AL>();
  else if (s == 1) wait_vmcnt<(NST - 3) * AL + LOADS>();
  else wait_vmcnt<(NST - 2) * LOADS>();
}

// M: weight mode (W_BF16, W_FP4 or W_FP8L, the K-steps of the 32-row
// kernels above); NST LDS stages.
template <int M, int NT2, int NST>
__global__ void __launch_bounds__(NTHR) moe_ffn_decode_kernel(GemmArgs g) {
  constexpr int LOADS = loads_of<M>();
  constexpr int AL = a_loads<M>();
  constexpr int NK1 = 256 * NT2 / k_of<M>();  // gate/up K-steps (K = H = 256 NT2)
  constexpr int SPN = FFN_CH / k_of<M>();     // down K-steps per n-tile
  constexpr int NK = NK1 + NT2 * SPN;         // + down: NT2 n-tiles of the 128-input slice
  static_assert(NK % NST == 0, "an item is a whole number of stage rounds");
  // vector memory ops of a phase-2 epilogue per thread (exact: the waits of
  // the next item's first steps count them)
  constexpr int EPI = 8 * NT2;
  static_assert((NST - 2) * LOADS + EPI < 64, "waits within the load counter's range");
  constexpr int STAGE = stage_u4<M>();
  constexpr int STAGE_A = stage_a<M>();
  __shared__ __align__(16) u32x4_t lds_st[NST][STAGE];
  __shared__ __align__(16) u32x4_t lds_h[2 * DBM * NCH];  // the item's activated slice
  __shared__ __align__(16) int tk[256];          // routed experts of the batch's rows
  __shared__ int chosen[FFN_MAX_E];              // expert chosen by any row
  __shared__ int4 items[FFN_MAX_ITEMS];          // this workgroup's items (x: row-list slot)
  __shared__ int rows_of[FFN_MAX_ITEMS][DBM];    // their row ids
  __shared__ int n_items, own_real;

  // the kernel arguments the prologue needs, fetched in one batch of scalar
  // loads (left to itself the compiler fetches them one by one as the
  // prologue reaches them: a round trip each before the first weight load)
  asm volatile("" ::"s"(g.topk_idx), "s"(g.a), "s"(g.w0), "s"(g.w1), "s"(g.ws0), "s"(g.ws1),
               "s"(g.T), "s"(g.k), "s"(g.E), "s"(g.H), "s"(g.I), "s"(g.S), "s"(g.Is),
               "s"(g.nt_routed), "s"(g.nt_shared));
  if (M != W_BF16)
    asm volatile("" ::"s"(g.sw0), "s"(g.sw1), "s"(g.sws0), "s"(g.sws1));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x, G = gridDim.x;
  const int rows = g.T * g.k, nr = g.nt_routed, E = g.E;
  const int P = E * nr + g.nt_shared;  // potential items (G <= P: the host checks)
  const uint64_t lt = (1ull << lane) - 1;

  // the routed experts into LDS (one load per thread; lanes past the rows
  // repeat the last), then the weight rows of the own item's first three
  // K-steps
  for (int e = threadIdx.x; e < E; e += NTHR) chosen[e] = 0;
  dma4(reinterpret_cast<const char*>(g.topk_idx), (uint32_t)min((int)threadIdx.x, rows - 1) * 4u,
       tk + 64 * w);
  DTile cur, nxt;
  FTile fd;
  make_tile<GATE_UP, M>(g, ffn_potential(g, b, 1), 0, cur);
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue_gu_b<M>(cur, st, lds_st[st] + STAGE_A);
  wait_vmcnt<(NST - 1) * (LOADS - AL)>();  // the expert ids have landed
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  if ((int)threadIdx.x < rows && (unsigned)tk[threadIdx.x] < (unsigned)E) chosen[tk[threadIdx.x]] = 1;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();

  // wave 0: which potential items are real (every shared slice; a routed
  // slice when its expert was chosen) and this workgroup's list: its own item
  // if real, then the real items p >= G handed to it. Every workgroup derives
  // the same assignment: the i-th real item beyond the grid goes to the i-th
  // workgroup (in index order) whose own item is not real, or round-robin
  // over all workgroups once those are used up. Counts come from the chosen
  // experts' bit mask; only the items beyond the grid are visited.
  if (w == 0) {
    uint64_t cm[FFN_MAX_E / 64];
#pragma unroll
    for (int j = 0; j < FFN_MAX_E / 64; ++j)
      cm[j] = __ballot(lane + 64 * j < E && chosen[lane + 64 * j] != 0);
    auto chosen_e = [&](int e) -> bool { return (cm[e >> 6] >> (e & 63)) & 1; };
    // unreal potential items below p: the slices of unchosen experts
    const int ns = g.nt_shared;
    auto unreal_below = [&](int p) -> int {
      const int pr = min(max(p - ns, 0), E * nr);
      const int e = pr / nr, c = pr - e * nr;
      int chosen_lt = 0;
#pragma unroll
      for (int j = 0; j < FFN_MAX_E / 64; ++j) {
        const int lo = 64 * j;
        if (e >= lo + 64) chosen_lt += __popcll(cm[j]);
        else if (e > lo) chosen_lt += __popcll(cm[j] & ((1ull << (e - lo)) - 1));
      }
      return (e - chosen_lt) * nr + (c > 0 && !chosen_e(e) ? c : 0);
    };
    const bool own = b < ns || chosen_e((b - ns) / nr);
    const int nfree = unreal_below(G);
    const int my_rank = own ? -1 : unreal_below(b);
    if (own && lane == 0) items[0] = ffn_potential(g, b, 0);
    int mine = own ? 1 : 0, i0 = 0;
    for (int p0 = G; p0 < P; p0 += 64) {
      const int p = p0 + lane;
      const bool beyond = p < P && (p < ns || chosen_e((p - ns) / nr));
      const uint64_t bm = __ballot(beyond);
      const int i = i0 + __popcll(bm & lt);
      const bool to_me = beyond && (i < nfree ? i == my_rank : (i - nfree) % G == b);
      const uint64_t tm = __ballot(to_me);
      const int slot = mine + __popcll(tm & lt);
      if (to_me && slot < FFN_MAX_ITEMS) items[slot] = ffn_potential(g, p, 0);
      mine += __popcll(tm);
      i0 += __popcll(bm);
    }
    if (lane == 0) {
      n_items = min(mine, FFN_MAX_ITEMS);
      own_real = own;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  const int n_my = n_items;

  // each item's rows: routed slices the rows that chose the expert, in row
  // order (at most T, one per token; lane l checks rows 4l .. 4l+3); shared
  // slices the T tokens
  for (int it = w; it < n_my; it += NTHR / 64) {
    const int4 p = items[it];
    int cnt = 0;
    if (p.y >> 16) {
      if (lane < g.T) rows_of[it][lane] = lane;
      cnt = g.T;
    } else {
      const int4 v = reinterpret_cast<const int4*>(tk)[lane];
      const int r0 = 4 * lane;
      const bool h0 = r0 < rows && v.x == p.z, h1 = r0 + 1 < rows && v.y == p.z;
      const bool h2 = r0 + 2 < rows && v.z == p.z, h3 = r0 + 3 < rows && v.w == p.z;
      const uint64_t m0 = __ballot(h0), m1 = __ballot(h1), m2 = __ballot(h2), m3 = __ballot(h3);
      int at = __popcll(m0 & lt) + __popcll(m1 & lt) + __popcll(m2 & lt) + __popcll(m3 & lt);
      if (h0 && at < DBM) rows_of[it][at] = r0;
      at += h0;
      if (h1 && at < DBM) rows_of[it][at] = r0 + 1;
      at += h1;
      if (h2 && at < DBM) rows_of[it][at] = r0 + 2;
      at += h2;
      if (h3 && at < DBM) rows_of[it][at] = r0 + 3;
      // a token chooses an expert at most once: cnt <= T <= 32
      cnt = min(__popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3), DBM);
    }
    if (lane == 0) items[it] = make_int4(it, cnt | (p.y & 0x10000), p.z, p.w);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  if (n_my == 0) {
    // nothing to run: let the own item's loads land before leaving
    wait_vmcnt<0>();
    return;
  }
  auto place = [&](int i) -> int4 {
    const int4 p = items[min(i, n_my - 1)];
    return make_int4(__builtin_amdgcn_readfirstlane(p.x), __builtin_amdgcn_readfirstlane(p.y),
                     __builtin_amdgcn_readfirstlane(p.z), __builtin_amdgcn_readfirstlane(p.w));
  };

  // the first item: the own one (its weight loads are in flight; add the
  // activation rows' loads) or a handed-over one (wait for the own item's
  // loads to land, then load all of its first three K-steps)
  const int4 p0 = place(0);
  const bool own = __builtin_amdgcn_readfirstlane(own_real) != 0;
  make_tile<GATE_UP, M>(g, p0, ffn_token(g, p0, rows_of[p0.x]), cur);
  if (own) {
#pragma unroll
    for (int st = 0; st < NST - 1; ++st) issue_gu_a<M>(cur, st, lds_st[st]);
  } else {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int st = 0; st < NST - 1; ++st) {
      issue_gu_a<M>(cur, st, lds_st[st]);
      issue_gu_b<M>(cur, st, lds_st[st] + STAGE_A);
    }
  }

  bool first = true;
  for (int li = 0;; ++li) {
    const bool has_next = li + 1 < n_my;
    const int4 pc = place(li), pn = place(li + 1);
    make_ftile<M>(g, pc, fd);
    make_tile<GATE_UP, M>(g, pn, ffn_token(g, pn, rows_of[pn.x]), nxt);
    Acc2 acc;
    Acc2 dacc[NT2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[nb][v] = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT2; ++nt) dacc[nt][nb][v] = 0.f;
      }
    // step s: wait for stage s, barrier, issue step s + NST-1 (this item's
    // gate/up or down rows, or the next item's first steps), compute stage
    // s; after the last gate/up step the slice goes to LDS. Waits: loads
    // issued after stage s's are NST-2 stages, plus the previous item's
    // epilogue stores in an item's first NST-1 steps (spec_wait for the own
    // first item)
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      if (s < NST - 1 && first && own) spec_wait<NST, AL, LOADS>(s);
      else if (s < NST - 1 && !first) wait_vmcnt<(NST - 2) * LOADS + EPI>();
      else wait_vmcnt<(NST - 2) * LOADS>();
      __builtin_amdgcn_s_barrier();
      const int sl = s + NST - 1;
      u32x4_t* la = lds_st[sl % NST];
      if (sl < NK1) {
        issue_gu_a<M>(cur, sl, la);
        issue_gu_b<M>(cur, sl, la + STAGE_A);
      } else if (sl < NK) {
        issue_ffn_down<M>(cur, fd, sl - NK1, la, la + STAGE_A);
      } else {
        issue_gu_a<M>(nxt, sl - NK, la);
        issue_gu_b<M>(nxt, sl - NK, la + STAGE_A);
      }
      const u32x4_t* lc = lds_st[s % NST];
      if (s < NK1) {
        compute_stage<GATE_UP, M>(lc, lc + STAGE_A, acc);
        if (s == NK1 - 1) {
          ffn_h_to_lds(g, acc, lds_h);
          // the slice is in LDS before the next step's barrier
          __asm__ __volatile__("" ::: "memory");
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __asm__ __volatile__("" ::: "memory");
        }
      } else {
        // bf16: the 64-input block of the slice for this K-step; MX: both
        compute_ffn_down<M>(lds_h + (M == W_BF16 ? ((s - NK1) % SPN) * DBM * NCH : 0),
                            lc + STAGE_A, dacc[(s - NK1) / SPN]);
      }
    }
    ffn_epilogue<NT2>(g, pc, rows_of[pc.x], dacc);
    if (!has_next) break;
    first = false;
    cur = nxt;
  }
  // the look-ahead loads after the last item are not used: let them land
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
}

// ---------------------------------------------------------------------------
// host side

int gemm_decode_bm() { return DBM; }

// Every K length is a whole number of four K-steps, and the per-lane 32-bit
// offsets reach every row: x, h, h_shared, one expert's weights, the shared
// weights, and acc rows of the atomic epilogue (< 2^31).
bool gemm_decode_fits(int64_t T, int H, int I, int k, int S, int Is, int wfmt) {
  if (H % 256 || I % 256 || (S && (S * Is) % 256)) return false;
  // MXFP4 K-steps of 128 inputs must not straddle two shared experts
  if (wfmt == WF_MXFP4 && S > 1 && Is % 128) return false;
  const uint64_t lim = 1ull << 32;
  const uint64_t x = (uint64_t)T * H * 2, h = (uint64_t)T * k * I * 2,
                 hs = (uint64_t)T * S * Is * 2, w = (uint64_t)H * I * 2,
                 ws = (uint64_t)S * H * Is * 2, acc = (uint64_t)T * H * 4;
  return x < lim && h < lim && hs < lim && w < lim && ws < lim && acc < (1ull << 31);
}

static int g_dec_cus = 0;
static int dec_num_cus() {
  if (g_dec_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_dec_cus = n;
    else
      g_dec_cus = 256;
  }
  return g_dec_cus;
}

static hipError_t launch_decode(void (*kern)(GemmArgs), long n, const GemmArgs& g,
                                hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long grid = n < dec_num_cus() ? n : dec_num_cus();
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTHR), 0, st, g);
  return hipGetLastError();
}

// g.wfmt selects the MX-weight kernels (scales in g.sw0 / sw1 / sws0 / sws1).
// MXFP8: 128-input K-steps with three stages when every K length the launch
// streams is a multiple of three such steps (and a separate shared expert's
// width a multiple of 128), else 64-input steps with six stages (K a
// multiple of six steps) or four. MXFP4: 128-input K-steps with four stages
// when every K length is a multiple of four steps, else two (every K length
// is a multiple of 256, and a K-split shared width a multiple of 128: the
// host checks with gemm_decode_fits).
static bool steps_div(int K, int k_step, int n) { return K % k_step == 0 && (K / k_step) % n == 0; }

enum Variant { V_BF16, V_FP8L3, V_FP8_6, V_FP8_4, V_FP4_4, V_FP4_2 };

static Variant pick(const GemmArgs& g, bool gate_up, bool routed, bool shared) {
  if (g.wfmt == WF_DTYPE) return V_BF16;
  if (g.wfmt == WF_MXFP4) {
    bool four = true;
    if (gate_up) four = steps_div(g.H, 128, 4);
    else {
      if (routed) four = four && steps_div(g.I, 128, 4);
      if (shared) four = four && steps_div(g.S * g.Is, 128, 4);
    }
    return four ? V_FP4_4 : V_FP4_2;
  }
  bool l3 = true, six = true;
  if (gate_up) {
    l3 = steps_div(g.H, 128, 3);
    six = steps_div(g.H, 64, 6);
  } else {
    if (routed) {
      l3 = l3 && steps_div(g.I, 128, 3);
      six = six && steps_div(g.I, 64, 6);
    }
    if (shared) {
      l3 = l3 && steps_div(g.S * g.Is, 128, 3) && g.Is % 128 == 0;
      six = six && steps_div(g.S * g.Is, 64, 6);
    }
  }
  return l3 ? V_FP8L3 : six ? V_FP8_6 : V_FP8_4;
}

#define DEC_LAUNCH(KERN, V, n, g, st)                                                  \
  ((V) == V_BF16    ? launch_decode(KERN<W_BF16, 4>, n, g, st)                          \
   : (V) == V_FP8L3 ? launch_decode(KERN<W_FP8L, 3>, n, g, st)                          \
   : (V) == V_FP8_6 ? launch_decode(KERN<W_FP8, 6>, n, g, st)                           \
   : (V) == V_FP8_4 ? launch_decode(KERN<W_FP8, 4>, n, g, st)                           \
   : (V) == V_FP4_4 ? launch_decode(KERN<W_FP4, 4>, n, g, st)                           \
                    : launch_decode(KERN<W_FP4, 2>, n, g, st))

hipError_t launch_gate_up_decode(const GemmArgs& g, hipStream_t st) {
  const long n = (long)g.mt_shared * g.nt_shared + (long)g.mt_routed * g.nt_routed;
  return DEC_LAUNCH(moe_gate_up_decode_kernel, pick(g, true, true, g.S > 0), n, g, st);
}
hipError_t launch_down_both_decode(const GemmArgs& g, hipStream_t st) {
  const long n = (long)g.mt_shared * g.nt_shared + (long)g.mt_routed * g.nt_routed;
  return DEC_LAUNCH(moe_down_decode_kernel, pick(g, false, true, true), n, g, st);
}
hipError_t launch_down_shared_decode(const GemmArgs& g, hipStream_t st) {
  const long n = (long)g.mt_shared * g.nt_shared;
  return DEC_LAUNCH(moe_down_shared_decode_kernel, pick(g, false, false, true), n, g, st);
}
hipError_t launch_down_routed_decode(const GemmArgs& g, bool atomic, hipStream_t st) {
  const long n = (long)g.mt_routed * g.nt_routed;
  const Variant v = pick(g, false, true, false);
  if (atomic) return DEC_LAUNCH(moe_down_routed_atomic_decode_kernel, v, n, g, st);
  return DEC_LAUNCH(moe_down_routed_decode_kernel, v, n, g, st);
}

// Shapes the fused FFN kernel takes: H = 512 or 1024 (NT2 = 2 or 4; MXFP4
// weights H = 1024, whose 12 K-steps per item fill the four stages), the
// intermediate widths whole 128-column slices, E within the kernel's LDS
// arrays, and one expert's (and all shared experts') weights within the
// per-lane 32-bit offsets. The batch limits (T <= 32 tokens, T * k <= 256
// rows) and bf16 activations are the caller's to check.
bool ffn_decode_fits(int H, int I, int E, int S, int Is, int wfmt) {
  if (H != 512 && H != 1024) return false;
  if (wfmt == WF_MXFP4 && H != 1024) return false;
  if (I <= 0 || I % FFN_CH || E > FFN_MAX_E) return false;
  if (S && (Is <= 0 || Is % FFN_CH)) return false;
  const uint64_t lim = 1ull << 31;
  return (uint64_t)H * I * 2 < lim && (uint64_t)S * H * Is * 2 < lim;
}

int ffn_decode_slice() { return FFN_CH; }

// Grid of the fused kernel for P potential items: one workgroup per compute
// unit at most (MOE_FFN_GRID=n caps it further: a testing knob that makes
// workgroups run several items).
static int ffn_grid(int P) {
  int G = std::min(P, std::min(dec_num_cus(), FFN_MAX_GRID));
  if (const char* e = std::getenv("MOE_FFN_GRID")) {
    const int cap = std::atoi(e);
    if (cap > 0) G = std::min(G, cap);
  }
  return G;
}

// The items of a workgroup fit its list: its own item plus the real items
// beyond the grid handed to it, at most ceil((P - G) / G) of them.
static bool ffn_items_fit(int P, int G) {
  return G > 0 && 1 + (P - G + G - 1) / G <= FFN_MAX_ITEMS;
}

bool ffn_decode_schedulable(int E, int I, int S, int Is) {
  const int P = E * (I / FFN_CH) + (S ? S * Is / FFN_CH : 0);
  return ffn_items_fit(P, ffn_grid(P));
}

hipError_t launch_ffn_decode(const GemmArgs& g, hipStream_t st) {
  const int P = g.E * g.nt_routed + g.nt_shared;
  const int G = ffn_grid(P);
  if (!ffn_items_fit(P, G) || g.T < 1 || g.T > DBM || g.T * g.k > 256 || g.E > FFN_MAX_E)
    return hipErrorInvalidValue;
  void (*kern)(GemmArgs) = nullptr;
  if (g.wfmt == WF_DTYPE)
    kern = g.H == 1024 ? moe_ffn_decode_kernel<W_BF16, 4, 4>
         : g.H == 512  ? moe_ffn_decode_kernel<W_BF16, 2, 4> : nullptr;
  else if (g.wfmt == WF_MXFP4)
    kern = g.H == 1024 ? moe_ffn_decode_kernel<W_FP4, 4, 4> : nullptr;
  else if (g.wfmt == WF_MXFP8)
    kern = g.H == 1024 ? moe_ffn_decode_kernel<W_FP8L, 4, 3>
         : g.H == 512  ? moe_ffn_decode_kernel<W_FP8L, 2, 3> : nullptr;
  if (!kern) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(NTHR), 0, st, g);
  return hipGetLastError();
}
