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
