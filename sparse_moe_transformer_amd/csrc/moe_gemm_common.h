// Device helpers of the grouped-GEMM kernels: tile ordering, the per-expert
// tile prefix, the split of a persistent launch's tiles over the XCDs,
// load-counter waits and output stores. Everything here is header-local
// (anonymous namespace), so each translation unit gets its own copy.
#pragma once

#include "moe_common.h"
#include "moe_kernels.h"

namespace {

// What a grouped-GEMM launch computes. DOWN_BOTH: shared tiles (stored to
// acc) then routed tiles (unweighted rows to y_perm) in one launch; used with
// the fixed-order combine.
enum Kind { GATE_UP = 0, DOWN_SHARED = 1, DOWN_ROUTED = 2, DOWN_BOTH = 3 };

// A 128-byte line of zeros: the source of the padding K-steps (they add
// exactly zero to the accumulators).
__device__ __align__(128) uint32_t g_zero_line[32] = {};

// LDS rows are 8 chunks of 16 B; chunk c of row r is stored at c ^ swz(r).
// No bank conflicts for the 32x32 MFMA fragment reads (measured on gfx950).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// MX weight conversions (exact): E4M3 and E2M1 codes to bf16, times the
// block's E8M0 scale. The scaled conversions read only the exponent field of
// the scale operand, so e8m0_scale builds a float whose exponent field is the
// E8M0 byte (byte 0 becomes the subnormal 2^-127 exactly).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : e << 23);
}

// Eight E4M3 codes (two dwords) -> eight bf16, times the block scale.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t d0, uint32_t d1, float scale) {
  const u32x4_t u = {
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true))};
  return __builtin_bit_cast(bf16x8_t, u);
}

// Eight E2M1 codes (one dword, input 2b in the low nibble of byte b) ->
// eight bf16, times the block scale.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t d, float scale) {
  const u32x4_t u = {
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3))};
  return __builtin_bit_cast(bf16x8_t, u);
}

// vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Grouped tile order: logical index b -> (m-slot, n-tile) with groups of gm
// m-slots; inside a group the m-slot varies fastest.
__device__ __forceinline__ void grouped_order(int b, int mt, int nt, int gm, int* m, int* n) {
  const int per_group = gm * nt;
  const int g = b / per_group;
  const int first = g * gm;
  const int gsize = min(gm, mt - first);
  const int local = b - g * per_group;
  *m = first + local % gsize;
  *n = local / gsize;
}

// offs <- expert_offsets (E+1 ints); cum[e] = sum_{e'<e} ceil(n_e'/BM), e <= E.
// Needs blockDim.x >= 64 and a barrier before offs/cum are read.
template <int BM>
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int* offs, int* cum) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offs[e] = offsets[e];
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
}

// the expert that owns routed m-slot `slot` (largest e with cum[e] <= slot;
// it has cum[e+1] > slot, so it is not empty)
__device__ __forceinline__ int owner(const int* cum, int E, int slot) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= slot) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// row / k for row ids (0 <= row < 2^31): multiply-high by floor(2^32 / k)
// falls short by at most one, which the fix-up restores
__device__ __forceinline__ int div_k(int row, int k, uint32_t kmagic) {
  int t = (int)__umulhi((uint32_t)row, kmagic);
  if ((t + 1) * k <= row) ++t;
  return t;
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

// Row (within a run of 32-row MFMA blocks) of accumulator element v of block
// mb: 32x32 MFMA lane l holds rows 8*(v/4) + 4*(l/32) + v%4 of column l%32.
__device__ __forceinline__ int acc_row(int mb, int v, int q) {
  return mb * 32 + (v >> 2) * 8 + q * 4 + (v & 3);
}

// This workgroup's share of a persistent launch over `ntiles` tiles, of
// which the first `nsh` are of one kind (shared-expert down tiles) and are
// split over the XCDs separately from the rest, so every XCD gets its share
// of each kind. Workgroups go to the XCDs round-robin; each XCD owns a
// contiguous range of tiles proportional to its workgroup count and its
// workgroups walk that range with a stride of their number.
struct WgTiles {
  int n_my;                  // tiles of this workgroup
  int slot, gx, ns_x, slo, nsh, rlo;
  __device__ __forceinline__ int global(int i) const {
    const int L = slot + i * gx;
    return L < ns_x ? slo + L : nsh + rlo + (L - ns_x);
  }
};

__device__ __forceinline__ WgTiles wg_tiles(int ntiles, int nsh) {
  const int G = gridDim.x, b = blockIdx.x;
  const int nx = G < 8 ? G : 8;
  const int x = b % nx;
  WgTiles w;
  w.slot = b / nx;
  w.gx = G / nx + (x < G % nx ? 1 : 0);
  const int before = x * (G / nx) + min(x, G % nx);  // workgroups on XCDs < x
  const int nrt = ntiles - nsh;
  w.nsh = nsh;
  w.slo = (int)((long)nsh * before / G);
  const int shi = (int)((long)nsh * (before + w.gx) / G);
  w.rlo = (int)((long)nrt * before / G);
  const int rhi = (int)((long)nrt * (before + w.gx) / G);
  w.ns_x = shi - w.slo;
  const int n_x = w.ns_x + (rhi - w.rlo);
  w.n_my = w.slot >= n_x ? 0 : (n_x - w.slot + w.gx - 1) / w.gx;
  return w;
}

}  // namespace
