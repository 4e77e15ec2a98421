// Grouping of the T*k routed rows by expert: a stable counting sort on device.
//
//  1. chunk pass: each workgroup takes 256 consecutive rows, builds their
//     expert histogram in LDS and the rank of every row among the earlier
//     rows of its chunk with the same expert;
//  2. scan pass (one workgroup): per expert, the running count over chunks
//     (column scan, split over up to 16 threads per expert) and the
//     exclusive scan over experts -> expert_offsets;
//  3. scatter pass: pos = offsets[e] + rows of e in earlier chunks + rank.
// Up to 1024 rows (decode batches) the same sort runs in one workgroup.
// Nothing returns to the host; the result does not depend on timing.
#include "moe_common.h"
#include "moe_kernels.h"
#include "moe_small_sort.h"

namespace {

constexpr int CH = 256;  // rows per chunk (one per thread)

__global__ void __launch_bounds__(CH) permute_chunk_kernel(const int32_t* __restrict__ idx,
                                                           int rows, int E,
                                                           int32_t* __restrict__ local_rank,
                                                           int32_t* __restrict__ chunk_hist) {
  __shared__ int ex[CH];
  extern __shared__ int hist[];  // [E]
  const int c = blockIdx.x;
  const int r = c * CH + threadIdx.x;
  for (int e = threadIdx.x; e < E; e += CH) hist[e] = 0;
  const int my = r < rows ? idx[r] : -1;
  ex[threadIdx.x] = my;
  __syncthreads();
  if (my >= 0) {
    int rank = 0;
    for (int j = 0; j < (int)threadIdx.x; ++j) rank += (ex[j] == my);
    local_rank[r] = rank;
    atomicAdd(&hist[my], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += CH) chunk_hist[(size_t)c * E + e] = hist[e];
}

// One workgroup of 1024 threads. chunk_hist is rewritten in place with the
// exclusive column prefix (rows of expert e in chunks before c). P threads
// share an expert (P * E <= 1024, P <= 16): thread (e, p) owns the chunks
// [p * L, (p + 1) * L), sums them (pass 1), takes the sum of the ranges
// before its own from LDS, and writes its range's running prefix (pass 2,
// re-reading the same L2-resident values). Each pass keeps 16 loads in
// flight, so a pass takes about L / 16 round trips instead of nchunks / 16.
__global__ void __launch_bounds__(1024) permute_scan_kernel(int nchunks, int E, int P,
                                                            int32_t* __restrict__ chunk_hist,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int psum[1024];  // [P][E]: the sum of each thread's range
  __shared__ int wsum[16];
  constexpr int B = 16;
  const int e = threadIdx.x % E, p = threadIdx.x / E;
  const bool active = p < P;
  const int L = (nchunks + P - 1) / P;
  const int c_lo = min(nchunks, p * L), c_hi = min(nchunks, c_lo + L);
  int mine = 0;
  if (active) {
    for (int c0 = c_lo; c0 < c_hi; c0 += B) {
      int v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = (c0 + u < c_hi) ? chunk_hist[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < B; ++u) mine += v[u];
    }
    psum[p * E + e] = mine;
  }
  __syncthreads();
  int before = 0, run = 0;  // rows of e in the ranges before p; in all ranges
  if (active) {
    for (int q = 0; q < P; ++q) {
      const int s = psum[q * E + e];
      if (q < p) before += s;
      run += s;
    }
    int acc = before;
    for (int c0 = c_lo; c0 < c_hi; c0 += B) {
      int v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = (c0 + u < c_hi) ? chunk_hist[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < B; ++u) {
        if (c0 + u < c_hi) chunk_hist[(size_t)(c0 + u) * E + e] = acc;
        acc += v[u];
      }
    }
  }
  // exclusive scan over experts of the totals (threads e < E, E <= 1024)
  if (threadIdx.x >= E) run = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (threadIdx.x < 64) {
    int v = threadIdx.x < 16 ? wsum[threadIdx.x] : 0;
    int vi = v;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(vi, off);
      if (threadIdx.x >= off) vi += o;
    }
    if (threadIdx.x < 16) wsum[threadIdx.x] = vi - v;
  }
  __syncthreads();
  const int excl = incl - run + wsum[wave];
  if ((int)threadIdx.x < E) offsets[threadIdx.x] = excl;
  if ((int)threadIdx.x == E - 1) offsets[E] = excl + run;
}

__global__ void __launch_bounds__(256) permute_scatter_kernel(const int32_t* __restrict__ idx,
                                                              int rows, int E,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ chunk_pre,
                                                              const int32_t* __restrict__ local_rank,
                                                              int32_t* __restrict__ sorted_rows,
                                                              int32_t* __restrict__ row_pos) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int e = idx[r];
  const int c = r / CH;
  const int pos = offsets[e] + chunk_pre[(size_t)c * E + e] + local_rank[r];
  sorted_rows[pos] = r;
  row_pos[r] = pos;
}

// The whole counting sort in one workgroup, for at most 1024 rows (decode
// batches).
__global__ void __launch_bounds__(1024) permute_small_kernel(const int32_t* __restrict__ idx,
                                                             int rows, int E,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_rows,
                                                             int32_t* __restrict__ row_pos) {
  __shared__ __align__(16) int ex[1024];
  __shared__ int cnt[1024];
  __shared__ int wsum[16];
  ex[threadIdx.x] = threadIdx.x < rows ? idx[threadIdx.x] : -1;
  block_sort_rows_1024(ex, rows, E, cnt, wsum, offsets, sorted_rows, row_pos);
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

int permute_chunk_rows() { return CH; }

hipError_t launch_permute(const int32_t* idx, int rows, int E, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* row_pos, int32_t* local_rank,
                          int32_t* chunk_hist, hipStream_t st) {
  if (rows <= 1024) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, st, idx, rows, E, offsets,
                       sorted_rows, row_pos);
    return hipGetLastError();
  }
  const int nch = (rows + CH - 1) / CH;
  hipLaunchKernelGGL(permute_chunk_kernel, dim3(nch), dim3(CH), E * sizeof(int), st, idx, rows,
                     E, local_rank, chunk_hist);
  int P = 1024 / E;  // threads per expert (E <= 1024)
  if (P > 16) P = 16;
  if (P > nch) P = nch;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, st, nch, E, P, chunk_hist,
                     offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, idx,
                     rows, E, offsets, chunk_hist, local_rank, sorted_rows, row_pos);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  // bytes is a multiple of 4 (all callers clear int32/fp32 arrays)
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}
