// Host-visible launch interface of the libmoe kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_common.h"

enum WeightFormat { WF_DTYPE = 0, WF_MXFP8 = 1, WF_MXFP4 = 2 };

// Arguments of the grouped expert GEMMs (passed by value to the kernels).
struct GemmArgs {
  const void* a;      // activations: x (gate/up), h (routed down), h_shared (shared down)
  const void* a_shared;  // h_shared when shared and routed down tiles share a launch
  const void* w0;     // gate or down stacked weights [E_tot, ., .]
  const void* w1;     // up stacked weights
  const void* ws0;    // shared gate (or shared down) weights
  const void* ws1;    // shared up weights
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted_rows;  // [T*k]
  const float* topk_w;         // [T*k]
  void* out;          // h (gate/up) or acc (down)
  void* out_shared;   // h_shared (gate/up)
  void* y_perm;       // unweighted routed rows (fixed-order combine)
  int T, H, I, E, k, S, Is;
  uint32_t kmagic;    // min(floor(2^32 / k), 2^32 - 1): row / k by multiply-high + one fix-up
  int mt_routed, nt_routed, mt_shared, nt_shared;
  int gm_routed, gm_shared;  // m-slots per group of the tile order
  ActParams act;
  // Expert weight format (wfmt): WF_DTYPE (the layer dtype), WF_MXFP8 (E4M3
  // codes, one byte per weight) or WF_MXFP4 (E2M1 codes, two weights per
  // byte, input 2j in the low nibble of byte j). MX formats carry E8M0
  // scales, block-major [K/32, N] per matrix, of the stacked gate (or down)
  // and up weights and of the shared gate (or down) and up weights (the
  // shared ones start at slot E when packed).
  int wfmt;
  const uint8_t* sw0;
  const uint8_t* sw1;
  const uint8_t* sws0;
  const uint8_t* sws1;
  // Gate/up of a decode batch of at most 256 routed rows on the 32-row
  // kernels (else NULL): the routed experts [T*k]. Every workgroup groups
  // the rows itself (the stable counting sort, in LDS) instead of reading
  // offsets and sorted_rows, and workgroup 0 stores expert_offsets,
  // sorted_rows and row_pos to the *_out arrays for the later stages.
  const int32_t* topk_idx;
  int32_t* offsets_out;
  int32_t* sorted_out;
  int32_t* row_pos_out;
  // Fused decode FFN (launch_ffn_decode, which also reads topk_idx): the
  // routed and shared down weights (MX: their scales too) and the fp32
  // partial planes, [I/128][T*k][H] (by routed row t*k + j) then
  // [S*Is/128][T][H].
  const void* w2;
  const void* ws2;
  const uint8_t* sw2;
  const uint8_t* sws2;
  float* parts;
};

int gemm_bm();
hipError_t launch_gate_up(const GemmArgs& g, int dtype, hipStream_t st);
hipError_t launch_down_shared(const GemmArgs& g, int dtype, hipStream_t st);
// shared and routed down tiles in one launch (fixed-order combine only)
hipError_t launch_down_both(const GemmArgs& g, int dtype, hipStream_t st);
hipError_t launch_down_routed(const GemmArgs& g, int dtype, bool atomic, hipStream_t st);

// 32-row tile kernels for decode-sized batches (bf16 activations; every K
// length a multiple of 256; per-lane 32-bit offsets: gemm_decode_fits).
int gemm_decode_bm();
bool gemm_decode_fits(int64_t T, int H, int I, int k, int S, int Is, int wfmt);
hipError_t launch_gate_up_decode(const GemmArgs& g, hipStream_t st);
hipError_t launch_down_both_decode(const GemmArgs& g, hipStream_t st);
hipError_t launch_down_shared_decode(const GemmArgs& g, hipStream_t st);
hipError_t launch_down_routed_decode(const GemmArgs& g, bool atomic, hipStream_t st);
// Fused gate/up + down of decode batches of at most 32 tokens and 256 routed
// rows (bf16 activations, bf16 / MXFP8 / MXFP4 weights; shapes:
// ffn_decode_fits), by 128-column slices of the intermediate width
// (ffn_decode_slice) into fp32 partial planes.
bool ffn_decode_fits(int H, int I, int E, int S, int Is, int wfmt);
// ... and every workgroup's share of the work items fits its list (depends
// on the device's compute units)
bool ffn_decode_schedulable(int E, int I, int S, int Is);
int ffn_decode_slice();
hipError_t launch_ffn_decode(const GemmArgs& g, hipStream_t st);

// 256-row tile kernels for prefill-sized bf16 batches (every K length a
// multiple of 64; per-lane 32-bit offsets: gemm_wide_fits).
int gemm_wide_bm();
bool gemm_wide_fits(int64_t T, int H, int I, int k, int S, int Is);
hipError_t launch_gate_up_wide(const GemmArgs& g, hipStream_t st);
hipError_t launch_down_shared_wide(const GemmArgs& g, hipStream_t st);
hipError_t launch_down_routed_wide(const GemmArgs& g, bool atomic, hipStream_t st);

// router GEMM scratch: bf16 split planes of the router weight + K-chunk partials
int router_kchunks(int64_t T, int E, int H, int dtype);
size_t router_ws_bytes(int64_t T, int E, int H, int dtype);
// MXFP8 router weights (codes [E,H], scales [H/32,E]) -> fp32 [E,H], exactly
hipError_t launch_router_dequant_mx(const uint8_t* codes, const uint8_t* scales, float* out, int E,
                                    int H, hipStream_t st);
hipError_t launch_router_logits(const void* x, const float* w_router, float* logits, int T,
                                int H, int E, int dtype, void* ws, hipStream_t st);
// Small bf16 batches (T < 128, H <= 64 * ROUTER_MAX_PLANES): the router's
// per-K-group partial planes ([H/64][T][E]
// fp32, router_planes() of them, 0 when the batch takes another path) for a
// consumer that sums them in plane order (launch_route with planes).
constexpr int ROUTER_MAX_PLANES = 32;
int router_planes(int64_t T, int H, int dtype);
hipError_t launch_router_planes(const void* x, const float* w_router, float* part, int T, int H,
                                int E, hipStream_t st);
// Larger batches: the router GEMM with its K-chunk partials ([kc][T][E] fp32,
// kc <= ROUTER_MAX_PLANES) left for the routing kernel to sum in chunk order
// (*planes, *np = kc), or, when there is one chunk or more than that many,
// the logits written whole (*np = 0).
hipError_t launch_router_chunks(const void* x, const float* w_router, float* logits, int T, int H,
                                int E, int dtype, void* ws, hipStream_t st, const float** planes,
                                int* np);

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int score_func, int route_norm, float route_scale, int32_t* idx,
                        float* w, int32_t* counts, hipStream_t st,
                        int n_group = 1, int topk_group = 1, const float* planes = nullptr,
                        int np = 0, float* logits_out = nullptr);

// permutation scratch: chunk histograms and per-row ranks
int permute_chunk_rows();
hipError_t launch_permute(const int32_t* idx, int rows, int E, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* row_pos, int32_t* local_rank,
                          int32_t* chunk_hist, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

hipError_t launch_combine(const float* acc, const void* y_perm, const int32_t* row_pos,
                          const float* topk_w, void* out, int T, int H, int k, int dtype,
                          hipStream_t st);

// fp32 partial planes of the fused decode FFN: nr routed planes [rows][H]
// (rows = T*k, indexed by routed row t*k + j), then ns shared planes [T][H].
struct PartsSrc {
  const float* p;
  int nr, ns, rows;
};
// out[t] = sum of the shared planes + sum_j topk_w[t,j] * (sum of the routed
// planes at row t*k+j), every sum in index order
hipError_t launch_combine_parts(const PartsSrc& parts, const float* topk_w, void* out, int T,
                                int H, int k, int dtype, hipStream_t st);

// RMSNorm rows (one workgroup per row, H <= 8192) and the finalising combine
// with the post-norm and the residual add
bool norm_fits(int H);
hipError_t launch_rmsnorm(const void* x, const float* w, int add_one, float eps, void* y, int T,
                          int H, int dtype, hipStream_t st);
hipError_t launch_combine_norm(const float* acc, const void* y_perm, const int32_t* row_pos,
                               const float* topk_w, const float* w, int add_one, float eps,
                               const void* residual, void* out, int T, int H, int k, int dtype,
                               hipStream_t st);
hipError_t launch_combine_norm_parts(const PartsSrc& parts, const float* topk_w, const float* w,
                                     int add_one, float eps, const void* residual, void* out,
                                     int T, int H, int k, int dtype, hipStream_t st);
