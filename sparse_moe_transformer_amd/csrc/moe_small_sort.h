// Stable counting sort of up to 1024 routed rows by expert inside one
// workgroup of 1024 threads (row = thread): the grouping step for decode
// batches. ex[r] holds row r's expert (any value for r >= rows); ex is
// 16-byte aligned. Writes expert_offsets [E+1] (exclusive scan of the
// counts), sorted_rows (rows of expert 0 in ascending row order, then expert
// 1, ...) and row_pos (its inverse). E <= 1024.
#pragma once

#include "moe_common.h"

__device__ __forceinline__ void block_sort_rows_1024(const int* ex, int rows, int E, int* cnt,
                                                     int* wsum, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_rows,
                                                     int32_t* __restrict__ row_pos) {
  const int t = threadIdx.x;
  cnt[t] = 0;
  __syncthreads();
  const int my = t < rows ? ex[t] : -1;
  int rank = 0;  // earlier rows with the same expert
  if (my >= 0) {
    // four rows per LDS read (ex is 16-byte aligned); every lane of a wave
    // reads the same address, a broadcast
    const int4* ex4 = reinterpret_cast<const int4*>(ex);
    const int n4 = t >> 2;
#pragma unroll 4
    for (int j = 0; j < n4; ++j) {
      const int4 v = ex4[j];
      rank += (v.x == my) + (v.y == my) + (v.z == my) + (v.w == my);
    }
    for (int j = n4 * 4; j < t; ++j) rank += (ex[j] == my);
    atomicAdd(&cnt[my], 1);
  }
  __syncthreads();
  const int c = t < E ? cnt[t] : 0;
  const int lane = t & 63, wave = t >> 6;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (t < 64) {
    const int v = t < 16 ? wsum[t] : 0;
    int vi = v;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(vi, off);
      if (t >= off) vi += o;
    }
    if (t < 16) wsum[t] = vi - v;
  }
  __syncthreads();
  const int excl = incl - c + wsum[wave];
  if (t < E) {
    cnt[t] = excl;  // every read of cnt happened before the barriers above
    offsets[t] = excl;
    if (t == E - 1) offsets[E] = excl + c;
  }
  __syncthreads();
  if (my >= 0) {
    const int pos = cnt[my] + rank;
    sorted_rows[pos] = t;
    row_pos[t] = pos;
  }
}

// The same sort for at most 256 rows (T tokens x k) in a workgroup of 256
// threads (row = thread), reading the experts from idx (global, [rows]).
// Scratch (LDS, 16-byte aligned, 256 + 3 * E + 4 ints): ex, cnt, wsum and,
// for T <= 64, one 64-bit token mask per expert. Results in LDS: offs [E+1]
// (expert offsets) and sorted [rows]; when g_offsets is not NULL also
// expert_offsets, sorted_rows and row_pos in global memory. Starts and ends
// with a workgroup barrier. E <= 1024; a token's k experts are distinct.
//
// With T <= 64 the rank of row r = t*k + j among its expert's rows is the
// number of earlier tokens that chose the same expert (each token chooses an
// expert at most once, so token order is row order): the popcount of the
// expert's token mask below bit t. Larger batches count earlier equal rows.
__device__ __forceinline__ void block_sort_rows_256(const int32_t* __restrict__ idx, int T,
                                                    int k, int E, int* scratch, int* offs,
                                                    int* sorted,
                                                    int32_t* __restrict__ g_offsets,
                                                    int32_t* __restrict__ g_sorted,
                                                    int32_t* __restrict__ g_row_pos) {
  const int t = threadIdx.x;
  const int rows = T * k;
  const bool masks = T <= 64;
  int* ex = scratch;
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(scratch + 256);
  int* cnt = scratch + 256 + 2 * E;
  int* wsum = cnt + E;
  __syncthreads();
  const int my = t < rows ? idx[t] : -1;
  ex[t] = my;
  for (int e = t; e < E; e += 256) {
    cnt[e] = 0;
    mask[e] = 0ull;
  }
  __syncthreads();
  int rank = 0;  // earlier rows with the same expert
  const int tok = t / k;
  if (my >= 0) {
    if (masks) {
      atomicOr(&mask[my], 1ull << tok);
    } else {
      const int4* ex4 = reinterpret_cast<const int4*>(ex);
      const int n4 = t >> 2;
      for (int j = 0; j < n4; ++j) {
        const int4 v = ex4[j];
        rank += (v.x == my) + (v.y == my) + (v.z == my) + (v.w == my);
      }
      for (int j = n4 * 4; j < t; ++j) rank += (ex[j] == my);
      atomicAdd(&cnt[my], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the counts: thread t takes experts 4t .. 4t+3
  int c[4], s4 = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * t + u;
    c[u] = e < E ? (masks ? __popcll(mask[e]) : cnt[e]) : 0;
    s4 += c[u];
  }
  const int lane = t & 63, wave = t >> 6;
  int incl = s4;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int run = before + incl - s4;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * t + u;
    if (e < E) {
      cnt[e] = run;  // every read of cnt happened before the barrier above
      offs[e] = run;
      if (g_offsets) g_offsets[e] = run;
    }
    run += c[u];
    if (e == E - 1) {
      offs[E] = run;
      if (g_offsets) g_offsets[E] = run;
    }
  }
  __syncthreads();
  if (my >= 0) {
    if (masks) rank = __popcll(mask[my] & ((1ull << tok) - 1ull));
    const int pos = cnt[my] + rank;
    sorted[pos] = t;
    if (g_sorted) {
      g_sorted[pos] = t;
      g_row_pos[t] = pos;
    }
  }
  __syncthreads();
}
