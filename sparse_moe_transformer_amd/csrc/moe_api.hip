// C ABI of libmoe: argument checks, workspace carving and kernel launches.
// All checks run before the first launch of a call; nothing here allocates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "moe.h"
#include "moe_kernels.h"

namespace {

struct Dims {
  int64_t T;
  int H, E, k, S, I, Is, packed, dtype;
  size_t es;   // element size of dtype tensors
  int wfmt;    // expert weight format (WF_DTYPE, WF_MXFP8, WF_MXFP4)
  int wbits;   // bits per expert weight (dtype: 8 * es; MXFP8 8; MXFP4 4)
  int rq;      // MXFP8 router weights
};

constexpr int64_t kMaxTokens = 1 << 24;

moe_status check_cfg(const moe_config* c, int64_t T, Dims* d) {
  if (!c || T < 0 || T > kMaxTokens) return MOE_ERR_INVALID_ARG;
  if (c->hidden_size <= 0 || c->hidden_size % 64) return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->num_experts > 1024) return MOE_ERR_INVALID_ARG;
  if (c->num_experts_per_tok < 1 || c->num_experts_per_tok > c->num_experts ||
      c->num_experts_per_tok > 32)
    return MOE_ERR_INVALID_ARG;
  if (c->num_shared_experts < 0 || c->num_shared_experts > 64) return MOE_ERR_INVALID_ARG;
  if (c->moe_intermediate_size <= 0 || c->moe_intermediate_size % 64) return MOE_ERR_INVALID_ARG;
  const int Is = c->shared_intermediate_size == 0 ? c->moe_intermediate_size
                                                  : c->shared_intermediate_size;
  if (Is < 0 || Is % 64) return MOE_ERR_INVALID_ARG;
  if (c->shared_packed != 0 && c->shared_packed != 1) return MOE_ERR_INVALID_ARG;
  if (c->shared_packed && (c->num_shared_experts != 1 || Is != c->moe_intermediate_size))
    return MOE_ERR_INVALID_ARG;
  if (c->score_func != MOE_SCORE_SIGMOID && c->score_func != MOE_SCORE_SOFTMAX)
    return MOE_ERR_INVALID_ARG;
  if (c->route_norm != 0 && c->route_norm != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->route_scale)) return MOE_ERR_INVALID_ARG;
  if (c->hidden_act != MOE_ACT_SILU && c->hidden_act != MOE_ACT_SWIGLUOAI)
    return MOE_ERR_INVALID_ARG;
  if (c->hidden_act == MOE_ACT_SWIGLUOAI &&
      !(std::isfinite(c->act_alpha) && std::isfinite(c->act_limit) && std::isfinite(c->act_beta)))
    return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->n_group < 0 || c->n_group > 64) return MOE_ERR_INVALID_ARG;
  if (c->n_group > 1) {
    const int gs = c->num_experts / c->n_group;
    if (c->num_experts % c->n_group || gs < 2 || c->topk_group < 1 ||
        c->topk_group > c->n_group || c->num_experts_per_tok > c->topk_group * gs)
      return MOE_ERR_INVALID_ARG;
  }
  if (c->weight_format != MOE_WEIGHTS_DTYPE && c->weight_format != MOE_WEIGHTS_MXFP8 &&
      c->weight_format != MOE_WEIGHTS_MXFP4)
    return MOE_ERR_INVALID_ARG;
  if (c->router_format != MOE_ROUTER_F32 && c->router_format != MOE_ROUTER_MXFP8)
    return MOE_ERR_INVALID_ARG;
  if (T * c->num_experts_per_tok > INT32_MAX / 2) return MOE_ERR_INVALID_ARG;
  d->T = T;
  d->H = c->hidden_size;
  d->E = c->num_experts;
  d->k = c->num_experts_per_tok;
  d->S = c->num_shared_experts;
  d->I = c->moe_intermediate_size;
  d->Is = Is;
  d->packed = c->shared_packed;
  d->dtype = c->dtype;
  d->es = c->dtype == MOE_BF16 ? 2 : 4;
  d->wfmt = c->weight_format == MOE_WEIGHTS_MXFP8   ? WF_MXFP8
            : c->weight_format == MOE_WEIGHTS_MXFP4 ? WF_MXFP4
                                                    : WF_DTYPE;
  d->wbits = d->wfmt == WF_MXFP8 ? 8 : d->wfmt == WF_MXFP4 ? 4 : 8 * (int)d->es;
  d->rq = c->router_format == MOE_ROUTER_MXFP8;
  // MX weights take bf16 activations
  if (d->wfmt != WF_DTYPE && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Workspace carving (every segment 256-byte aligned).
struct Ws {
  void* router;  // router GEMM scratch
  float* router_f32;  // MXFP8 router weights, dequantised (or NULL)
  float* logits;
  int32_t* idx;
  float* w;
  int32_t* offsets;
  int32_t* sorted_rows;
  int32_t* row_pos;
  int32_t* local_rank;
  int32_t* chunk_hist;
  void* h;
  void* h_shared;
  float* acc;
  void* y_perm;
  float* parts;  // fused decode FFN partial planes (empty when the shapes never take it)
  size_t total;
};

// The fused decode FFN (gate/up and down in one kernel, by 128-column slices
// of the intermediate width into fp32 partial planes that the combine sums):
// bf16 activations (bf16, MXFP8 or MXFP4 weights), shapes the kernel takes,
// at most 32 tokens and 256 routed rows. Testing knobs: MOE_DECODE_FFN=0 turns it off, and so
// does MOE_GEMM_TILE=128 (the 128-row tile kernels forced).
bool ffn_shape(const Dims& d) {
  return d.dtype == MOE_BF16 && ffn_decode_fits(d.H, d.I, d.E, d.S, d.Is, d.wfmt);
}

// the batch and the launch fit too (T = 0 aside)
bool ffn_supported(const Dims& d) {
  return ffn_shape(d) && d.T <= 32 && d.T * d.k <= 256 &&
         ffn_decode_schedulable(d.E, d.I, d.S, d.Is);
}

bool use_ffn(const Dims& d) {
  if (!ffn_supported(d)) return false;
  if (const char* e = std::getenv("MOE_DECODE_FFN"))
    if (std::strcmp(e, "0") == 0) return false;
  if (const char* e = std::getenv("MOE_GEMM_TILE"))
    if (std::strcmp(e, "128") == 0) return false;
  return true;
}

// Partial planes for min(T, 32) tokens whenever the shapes allow the fused
// path (whatever the batch and the knobs), so a workspace sized for T tokens
// serves every smaller batch too.
size_t ffn_planes_bytes(const Dims& d, int64_t T) {
  const size_t slice = (size_t)ffn_decode_slice();
  const size_t planes_rows =
      (size_t)d.I / slice * (size_t)T * d.k + (size_t)d.S * d.Is / slice * (size_t)T;
  return planes_rows * d.H * 4;
}

size_t ffn_parts_bytes(const Dims& d) {
  if (!ffn_shape(d)) return 0;
  return ffn_planes_bytes(d, std::min<int64_t>(d.T, 32));
}

Ws carve(const Dims& d, void* base) {
  Ws w{};
  const size_t rows = (size_t)d.T * d.k;
  const size_t nch = (rows + permute_chunk_rows() - 1) / permute_chunk_rows();
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.router = take(router_ws_bytes(d.T, d.E, d.H, d.dtype));
  w.router_f32 = d.rq ? (float*)take((size_t)d.E * d.H * 4) : nullptr;
  w.logits = (float*)take((size_t)d.T * d.E * 4);
  w.idx = (int32_t*)take(rows * 4);
  w.w = (float*)take(rows * 4);
  w.offsets = (int32_t*)take((size_t)(d.E + 1) * 4);
  w.sorted_rows = (int32_t*)take(rows * 4);
  w.row_pos = (int32_t*)take(rows * 4);
  w.local_rank = (int32_t*)take(rows * 4);
  w.chunk_hist = (int32_t*)take(nch * d.E * 4);
  w.h = take(rows * d.I * d.es);
  w.h_shared = take((size_t)d.T * d.S * d.Is * d.es);
  w.acc = (float*)take((size_t)d.T * d.H * 4);
  w.y_perm = take(rows * d.H * d.es);
  w.parts = (float*)take(ffn_parts_bytes(d));
  w.total = off;
  return w;
}

moe_status check_ws(const Dims& d, const void* ws, size_t ws_bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < carve(d, nullptr).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

inline moe_status hip_ok(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                  \
  do {                                 \
    moe_status _s = (expr);            \
    if (_s != MOE_OK) return _s;       \
  } while (0)

ActParams act_of(const moe_config* c) {
  if (c->hidden_act == MOE_ACT_SWIGLUOAI)
    return ActParams{c->act_alpha, c->act_limit, c->act_limit, c->act_beta};
  return ActParams{1.0f, INFINITY, INFINITY, 0.0f};  // silu
}

GemmArgs base_args(const moe_config* c, const Dims& d) {
  GemmArgs g{};
  g.T = (int)d.T;
  g.H = d.H;
  g.I = d.I;
  g.E = d.E;
  g.k = d.k;
  g.kmagic = (uint32_t)std::min<uint64_t>((1ull << 32) / (uint64_t)d.k, 0xFFFFFFFFull);
  g.S = d.S;
  g.Is = d.Is;
  g.act = act_of(c);
  return g;
}

const void* shared_slot(const void* stacked, const Dims& d, size_t per_expert_elems) {
  return static_cast<const char*>(stacked) + (size_t)d.E * per_expert_elems * d.wbits / 8;
}

// MX scales: present and complete exactly when the weights are MXFP8 or MXFP4
moe_status check_mx(const Dims& d, const moe_mx_scales* mx, bool gate_up, bool down) {
  if (d.wfmt == WF_DTYPE) return MOE_OK;
  if (!mx) return MOE_ERR_INVALID_ARG;
  if (gate_up && (!mx->gate || !mx->up)) return MOE_ERR_INVALID_ARG;
  if (down && !mx->down) return MOE_ERR_INVALID_ARG;
  if (d.S && !d.packed) {
    if (gate_up && (!mx->shared_gate || !mx->shared_up)) return MOE_ERR_INVALID_ARG;
    if (down && !mx->shared_down) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

const uint8_t* scale_slot(const uint8_t* stacked, const Dims& d, size_t per_expert) {
  return stacked + (size_t)d.E * per_expert;
}

// Grouped-GEMM tile choice. Decode-sized batches (at most 32 rows per expert
// on average) stream expert weights: the 32-row tile kernel keeps more weight
// K-steps in flight per compute unit. MOE_GEMM_TILE=32 or =128 forces one
// kernel (a testing knob; 32 still needs bf16 and gemm_decode_fits).
bool use_decode(const Dims& d) {
  if (d.dtype != MOE_BF16 || !gemm_decode_fits(d.T, d.H, d.I, d.k, d.S, d.Is, d.wfmt)) return false;
  if (const char* e = std::getenv("MOE_GEMM_TILE")) {
    if (std::strcmp(e, "128") == 0) return false;
    if (std::strcmp(e, "32") == 0) return true;
  }
  return d.T * d.k <= (int64_t)32 * d.E;
}

// The 256-row tiles for prefill-sized bf16 batches with many rows per expert
// (at least 384 on average) and long K (H and I at least 1024): there a
// weight tile is reused by several row tiles from L2 and the wider tile
// moves less data per FLOP (measured faster on the AFMoE-default and skewed
// layers; slower where weights stream from HBM with ~256 rows per expert, or
// K is short). MOE_GEMM_TILE=128 / =256 force one kernel (testing knobs).
bool use_wide(const Dims& d) {
  if (d.dtype != MOE_BF16 || d.wfmt != WF_DTYPE || use_decode(d)) return false;
  if (!gemm_wide_fits(d.T, d.H, d.I, d.k, d.S, d.Is)) return false;
  if (const char* e = std::getenv("MOE_GEMM_TILE")) {
    if (std::strcmp(e, "128") == 0) return false;
    if (std::strcmp(e, "256") == 0) return true;
  }
  return d.T * d.k >= (int64_t)384 * d.E && d.H >= 1024 && d.I >= 1024;
}

// --- stages (arguments already checked) ---

// Decode batches of at most 256 routed rows: the gate/up kernel groups the
// rows itself (no separate grouping launch).
bool group_in_gate_up(const Dims& d) { return use_decode(d) && d.T * d.k <= 256; }

// group: (group_in_gate_up) the routed experts and the grouping's outputs,
// which the gate/up kernel then computes and stores; else offsets and
// sorted_rows are inputs.
struct Grouping {
  const int32_t* topk_idx;
  int32_t* offsets;
  int32_t* sorted_rows;
  int32_t* row_pos;
};

moe_status do_gate_up(const moe_config* c, const Dims& d, const void* x, const void* w_gate,
                      const void* w_up, const void* ws_gate, const void* ws_up,
                      const moe_mx_scales* mx, const int32_t* offsets,
                      const int32_t* sorted_rows, void* h, void* h_shared, hipStream_t st,
                      const Grouping* group = nullptr) {
  GemmArgs g = base_args(c, d);
  if (d.wfmt != WF_DTYPE) {
    g.wfmt = d.wfmt;
    g.sw0 = mx->gate;
    g.sw1 = mx->up;
    const size_t per = (size_t)(d.H / 32) * d.I;
    g.sws0 = d.packed ? scale_slot(mx->gate, d, per) : mx->shared_gate;
    g.sws1 = d.packed ? scale_slot(mx->up, d, per) : mx->shared_up;
  }
  const bool dec = use_decode(d);
  const bool wide = use_wide(d);
  const int BM = dec ? gemm_decode_bm() : wide ? gemm_wide_bm() : gemm_bm();
  const int64_t rows = d.T * d.k;
  g.a = x;
  g.w0 = w_gate;
  g.w1 = w_up;
  if (d.packed) {
    g.ws0 = shared_slot(w_gate, d, (size_t)d.I * d.H);
    g.ws1 = shared_slot(w_up, d, (size_t)d.I * d.H);
  } else {
    g.ws0 = ws_gate;
    g.ws1 = ws_up;
  }
  g.offsets = offsets;
  g.sorted_rows = sorted_rows;
  g.out = h;
  g.out_shared = h_shared;
  g.mt_routed = (int)((rows + BM - 1) / BM + (rows < d.E ? rows : d.E));
  g.nt_routed = (d.I + 127) / 128;
  g.mt_shared = d.S ? (int)((d.T + BM - 1) / BM) : 0;
  g.nt_shared = d.S ? (d.S * d.Is + 127) / 128 : 0;
  g.gm_routed = 8;
  g.gm_shared = 8;
  if (group) {
    g.topk_idx = group->topk_idx;
    g.offsets_out = group->offsets;
    g.sorted_out = group->sorted_rows;
    g.row_pos_out = group->row_pos;
  }
  if (dec) return hip_ok(launch_gate_up_decode(g, st));
  if (wide) return hip_ok(launch_gate_up_wide(g, st));
  return hip_ok(launch_gate_up(g, d.dtype, st));
}

moe_status do_down(const moe_config* c, const Dims& d, const void* h, const void* w_down,
                   const void* h_shared, const void* ws_down, const moe_mx_scales* mx,
                   const int32_t* offsets, const int32_t* sorted_rows, const float* topk_w,
                   float* acc, void* y_perm, hipStream_t st) {
  GemmArgs g = base_args(c, d);
  if (d.wfmt != WF_DTYPE) {
    g.wfmt = d.wfmt;
    g.sw0 = mx->down;
    g.sws0 = d.packed ? scale_slot(mx->down, d, (size_t)(d.I / 32) * d.H) : mx->shared_down;
  }
  const bool dec = use_decode(d);
  const bool wide = use_wide(d);
  const int BM = dec ? gemm_decode_bm() : wide ? gemm_wide_bm() : gemm_bm();
  const int64_t rows = d.T * d.k;
  g.offsets = offsets;
  g.sorted_rows = sorted_rows;
  g.topk_w = topk_w;
  g.out = acc;
  g.y_perm = y_perm;
  g.mt_routed = (int)((rows + BM - 1) / BM + (rows < d.E ? rows : d.E));
  g.nt_routed = (d.H + 255) / 256;
  g.gm_routed = 4;
  if (d.S) {
    g.ws0 = d.packed ? shared_slot(w_down, d, (size_t)d.H * d.I) : ws_down;
    g.mt_shared = (int)((d.T + BM - 1) / BM);
    g.nt_shared = (d.H + 255) / 256;
    g.gm_shared = 4;
    if (y_perm) {
      // fixed-order combine: shared rows (to acc) and routed rows (to y_perm)
      // do not touch the same memory, so one launch takes both
      g.a = h;
      g.a_shared = h_shared;
      g.w0 = w_down;
      if (dec) return hip_ok(launch_down_both_decode(g, st));
      if (!wide) return hip_ok(launch_down_both(g, d.dtype, st));
      // 256-row tiles: shared rows, then routed rows, in two launches (one
      // output type per kernel keeps its accumulators in registers)
      g.a = h_shared;
      MOE_TRY(hip_ok(launch_down_shared_wide(g, st)));
      g.mt_shared = 0;
      g.nt_shared = 0;
      g.a = h;
      return hip_ok(launch_down_routed_wide(g, false, st));
    }
    g.a = h_shared;
    MOE_TRY(hip_ok(dec    ? launch_down_shared_decode(g, st)
                   : wide ? launch_down_shared_wide(g, st)
                          : launch_down_shared(g, d.dtype, st)));
  } else {
    MOE_TRY(hip_ok(launch_fill_zero(acc, (size_t)d.T * d.H * 4, st)));
  }
  g.mt_shared = 0;
  g.nt_shared = 0;
  g.a = h;
  g.w0 = w_down;
  if (dec) return hip_ok(launch_down_routed_decode(g, y_perm == nullptr, st));
  if (wide) return hip_ok(launch_down_routed_wide(g, y_perm == nullptr, st));
  return hip_ok(launch_down_routed(g, d.dtype, y_perm == nullptr, st));
}

moe_status check_layer_args(const Dims& d, const void* x, const void* w_router,
                            const void* w_gate, const void* w_up, const void* w_down,
                            const void* ws_gate, const void* ws_up, const void* ws_down,
                            const float* router_logits_in, int32_t deterministic,
                            const moe_mx_scales* mx) {
  if (!x || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if (!router_logits_in && !w_router) return MOE_ERR_INVALID_ARG;
  if (!router_logits_in && d.rq && (!mx || !mx->router)) return MOE_ERR_INVALID_ARG;
  if (d.S && !d.packed && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_INVALID_ARG;
  if (deterministic != 0 && deterministic != 1) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status check_norm(const Dims& d, const moe_norm_config* n) {
  if (!n || !(std::isfinite(n->rms_norm_eps) && n->rms_norm_eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (n->add_one != 0 && n->add_one != 1) return MOE_ERR_INVALID_ARG;
  if (!norm_fits(d.H)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t block_ws_bytes(const Dims& d) {
  return carve(d, nullptr).total + align256((size_t)d.T * d.H * d.es);
}

struct LayerOut {
  float* topk_w;  // routed weights the combine reads
  void* y_perm;   // unweighted routed rows (fixed-order combine) or NULL
  PartsSrc parts; // the fused decode FFN's partial planes (parts.p NULL: not taken)
};

// Expert FFN of a small decode batch in one launch (use_ffn): every slice of
// every chosen expert and of the shared experts into the partial planes.
moe_status do_ffn(const moe_config* c, const Dims& d, const void* x, const void* w_gate,
                  const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                  const void* ws_down, const moe_mx_scales* mx, const int32_t* topk_idx,
                  float* parts, hipStream_t st, PartsSrc* src) {
  GemmArgs g = base_args(c, d);
  if (d.wfmt != WF_DTYPE) {
    g.wfmt = d.wfmt;
    g.sw0 = mx->gate;
    g.sw1 = mx->up;
    g.sw2 = mx->down;
    const size_t per_gu = (size_t)(d.H / 32) * d.I, per_dn = (size_t)(d.I / 32) * d.H;
    g.sws0 = d.packed ? scale_slot(mx->gate, d, per_gu) : mx->shared_gate;
    g.sws1 = d.packed ? scale_slot(mx->up, d, per_gu) : mx->shared_up;
    g.sws2 = d.packed ? scale_slot(mx->down, d, per_dn) : mx->shared_down;
  }
  const int slice = ffn_decode_slice();
  const int64_t rows = d.T * d.k;
  g.a = x;
  g.w0 = w_gate;
  g.w1 = w_up;
  g.w2 = w_down;
  if (d.packed) {
    g.ws0 = shared_slot(w_gate, d, (size_t)d.I * d.H);
    g.ws1 = shared_slot(w_up, d, (size_t)d.I * d.H);
    g.ws2 = shared_slot(w_down, d, (size_t)d.H * d.I);
  } else {
    g.ws0 = ws_gate;
    g.ws1 = ws_up;
    g.ws2 = ws_down;
  }
  // slices per routed expert and of the shared width (T <= 32 rows each)
  g.nt_routed = d.I / slice;
  g.nt_shared = d.S ? d.S * d.Is / slice : 0;
  g.topk_idx = topk_idx;
  g.parts = parts;
  *src = PartsSrc{parts, g.nt_routed, g.nt_shared, (int)rows};
  return hip_ok(launch_ffn_decode(g, st));
}

// The router weights the router GEMM reads: as given (fp32), or MXFP8 codes
// dequantised exactly into the workspace first.
moe_status router_weights(const Dims& d, const void* w_router, const moe_mx_scales* mx,
                          const Ws& w, hipStream_t st, const float** out) {
  if (!d.rq) {
    *out = static_cast<const float*>(w_router);
    return MOE_OK;
  }
  MOE_TRY(hip_ok(launch_router_dequant_mx(static_cast<const uint8_t*>(w_router), mx->router,
                                          w.router_f32, d.E, d.H, st)));
  *out = w.router_f32;
  return MOE_OK;
}

// Router GEMM through the down projection; the caller finalises from w.acc.
moe_status run_layer(const moe_config* cfg, const Dims& d, const void* x, const void* w_router,
                     const float* expert_bias, const void* w_gate, const void* w_up,
                     const void* w_down, const void* ws_gate, const void* ws_up,
                     const void* ws_down, const moe_mx_scales* mx, const float* router_logits_in,
                     float* router_logits_out, int32_t* topk_idx_out, float* topk_w_out,
                     int32_t deterministic, const Ws& w, hipStream_t st, LayerOut* res) {
  const int T = (int)d.T;
  const float* logits = router_logits_in;
  // bf16 batches: the router leaves per-K-group planes (small batches) or
  // its K-chunk partials (larger ones) and the routing kernel sums them in
  // order (storing the logits) before it routes
  const float* planes = nullptr;
  int np = 0;
  float* lo = router_logits_out ? router_logits_out : w.logits;
  if (!logits) {
    const float* wr = nullptr;
    MOE_TRY(router_weights(d, w_router, mx, w, st, &wr));
    np = router_planes(T, d.H, d.dtype);
    if (np > 0) {
      planes = static_cast<const float*>(w.router);
      MOE_TRY(hip_ok(launch_router_planes(x, wr, static_cast<float*>(w.router), T, d.H, d.E, st)));
    } else {
      MOE_TRY(hip_ok(launch_router_chunks(x, wr, lo, T, d.H, d.E, d.dtype, w.router, st, &planes,
                                          &np)));
    }
    logits = lo;
  }
  int32_t* idx = topk_idx_out ? topk_idx_out : w.idx;
  float* tw = topk_w_out ? topk_w_out : w.w;
  // routing: one wavefront per token over many workgroups; grouping: inside
  // the gate/up kernel for decode batches of at most 256 routed rows, one
  // workgroup up to 1024 rows, else three small kernels
  MOE_TRY(hip_ok(launch_route(logits, expert_bias, T, d.E, d.k, cfg->score_func,
                              cfg->route_norm, cfg->route_scale, idx, tw, nullptr, st,
                              cfg->n_group, cfg->topk_group, planes, np, planes ? lo : nullptr)));
  const Grouping grp{idx, w.offsets, w.sorted_rows, w.row_pos};
  res->topk_w = tw;
  res->y_perm = nullptr;
  res->parts = PartsSrc{nullptr, 0, 0, 0};
  if (use_ffn(d))
    return do_ffn(cfg, d, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, mx, idx, w.parts, st,
                  &res->parts);
  const bool fused = group_in_gate_up(d);
  if (!fused)
    MOE_TRY(hip_ok(launch_permute(idx, T * d.k, d.E, w.offsets, w.sorted_rows, w.row_pos,
                                  w.local_rank, w.chunk_hist, st)));
  MOE_TRY(do_gate_up(cfg, d, x, w_gate, w_up, ws_gate, ws_up, mx, w.offsets, w.sorted_rows, w.h,
                     w.h_shared, st, fused ? &grp : nullptr));
  void* yp = deterministic ? w.y_perm : nullptr;
  MOE_TRY(do_down(cfg, d, w.h, w_down, w.h_shared, ws_down, mx, w.offsets, w.sorted_rows, tw,
                  w.acc, yp, st));
  res->topk_w = tw;
  res->y_perm = yp;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes) {
  Dims d;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_cfg(cfg, T, &d));
  *bytes = carve(d, nullptr).total;
  return MOE_OK;
}

moe_status moe_router_logits(const moe_config* cfg, int64_t T, const void* x,
                             const void* w_router, const moe_mx_scales* mx, float* logits,
                             void* ws, size_t ws_bytes, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (d.rq && (!mx || !mx->router)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(d, ws, ws_bytes));
  Ws w = carve(d, ws);
  const float* wr = nullptr;
  MOE_TRY(router_weights(d, w_router, mx, w, (hipStream_t)stream, &wr));
  return hip_ok(launch_router_logits(x, wr, logits, (int)T, d.H, d.E, d.dtype, w.router,
                                     (hipStream_t)stream));
}

moe_status moe_route(const moe_config* cfg, int64_t T, const float* logits,
                     const float* expert_bias, int32_t* topk_idx, float* topk_w,
                     int32_t* expert_counts, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (T == 0) {
    if (expert_counts) return hip_ok(launch_fill_zero(expert_counts, (size_t)d.E * 4, (hipStream_t)stream));
    return MOE_OK;
  }
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (expert_counts) MOE_TRY(hip_ok(launch_fill_zero(expert_counts, (size_t)d.E * 4, st)));
  return hip_ok(launch_route(logits, expert_bias, (int)T, d.E, d.k, cfg->score_func,
                             cfg->route_norm, cfg->route_scale, topk_idx, topk_w, expert_counts,
                             st, cfg->n_group, cfg->topk_group));
}

moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                       int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_pos,
                       void* ws, size_t ws_bytes, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (!expert_offsets) return MOE_ERR_INVALID_ARG;
  if (T == 0) return hip_ok(launch_fill_zero(expert_offsets, (size_t)(d.E + 1) * 4, (hipStream_t)stream));
  if (!topk_idx || !sorted_rows || !row_pos) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(d, ws, ws_bytes));
  Ws w = carve(d, ws);
  return hip_ok(launch_permute(topk_idx, (int)(T * d.k), d.E, expert_offsets, sorted_rows,
                               row_pos, w.local_rank, w.chunk_hist, (hipStream_t)stream));
}

moe_status moe_grouped_gate_up_swiglu(const moe_config* cfg, int64_t T, const void* x,
                                      const void* w_gate, const void* w_up, const void* ws_gate,
                                      const void* ws_up, const moe_mx_scales* mx,
                                      const int32_t* expert_offsets,
                                      const int32_t* sorted_rows, void* h, void* h_shared,
                                      void* ws, size_t ws_bytes, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !w_up || !expert_offsets || !sorted_rows || !h) return MOE_ERR_INVALID_ARG;
  if (d.S && !h_shared) return MOE_ERR_INVALID_ARG;
  if (d.S && !d.packed && (!ws_gate || !ws_up)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_mx(d, mx, true, false));
  (void)ws;
  (void)ws_bytes;
  return do_gate_up(cfg, d, x, w_gate, w_up, ws_gate, ws_up, mx, expert_offsets, sorted_rows, h,
                    h_shared, (hipStream_t)stream);
}

moe_status moe_grouped_down(const moe_config* cfg, int64_t T, const void* h, const void* w_down,
                            const void* h_shared, const void* ws_down, const moe_mx_scales* mx,
                            const int32_t* expert_offsets, const int32_t* sorted_rows,
                            const float* topk_w, float* acc, void* y_perm, void* ws,
                            size_t ws_bytes, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (T == 0) return MOE_OK;
  if (!h || !w_down || !expert_offsets || !sorted_rows || !acc) return MOE_ERR_INVALID_ARG;
  if (!y_perm && !topk_w) return MOE_ERR_INVALID_ARG;
  if (d.S && !h_shared) return MOE_ERR_INVALID_ARG;
  if (d.S && !d.packed && !ws_down) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_mx(d, mx, false, true));
  (void)ws;
  (void)ws_bytes;
  return do_down(cfg, d, h, w_down, h_shared, ws_down, mx, expert_offsets, sorted_rows, topk_w,
                 acc, y_perm, (hipStream_t)stream);
}

moe_status moe_combine(const moe_config* cfg, int64_t T, const float* acc, const void* y_perm,
                       const int32_t* row_pos, const float* topk_w, void* out,
                       moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (T == 0) return MOE_OK;
  if (!acc || !out) return MOE_ERR_INVALID_ARG;
  if (y_perm && (!row_pos || !topk_w)) return MOE_ERR_INVALID_ARG;
  return hip_ok(launch_combine(acc, y_perm, row_pos, topk_w, out, (int)T, d.H, d.k, d.dtype,
                               (hipStream_t)stream));
}

moe_status moe_expert_ffn_size(const moe_config* cfg, int64_t T, size_t* bytes) {
  Dims d;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (!ffn_supported(d)) return MOE_ERR_UNSUPPORTED;
  *bytes = ffn_planes_bytes(d, T);
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const void* w_gate,
                          const void* w_up, const void* w_down, const void* ws_gate,
                          const void* ws_up, const void* ws_down, const moe_mx_scales* mx,
                          const int32_t* topk_idx, float* parts, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (!ffn_supported(d)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !w_up || !w_down || !topk_idx || !parts) return MOE_ERR_INVALID_ARG;
  if (d.S && !d.packed && (!ws_gate || !ws_up || !ws_down)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_mx(d, mx, true, true));
  PartsSrc src;
  return do_ffn(cfg, d, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, mx, topk_idx, parts,
                (hipStream_t)stream, &src);
}

moe_status moe_combine_partials(const moe_config* cfg, int64_t T, const float* parts,
                                const float* topk_w, void* out, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (!ffn_supported(d)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!parts || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  const int slice = ffn_decode_slice();
  const PartsSrc src{parts, d.I / slice, d.S ? d.S * d.Is / slice : 0, (int)(T * d.k)};
  return hip_ok(launch_combine_parts(src, topk_w, out, (int)T, d.H, d.k, d.dtype,
                                     (hipStream_t)stream));
}

moe_status moe_layer_forward(const moe_config* cfg, int64_t T, const void* x,
                             const void* w_router, const float* expert_bias, const void* w_gate,
                             const void* w_up, const void* w_down, const void* ws_gate,
                             const void* ws_up, const void* ws_down, const moe_mx_scales* mx,
                             const float* router_logits_in, float* router_logits_out,
                             int32_t* topk_idx_out, float* topk_w_out, void* out,
                             int32_t deterministic, void* ws, size_t ws_bytes,
                             moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  if (T == 0) return MOE_OK;
  if (!out) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_layer_args(d, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                           router_logits_in, deterministic, mx));
  MOE_TRY(check_mx(d, mx, true, true));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  hipStream_t st = (hipStream_t)stream;
  Ws w = carve(d, ws);
  LayerOut lo;
  MOE_TRY(run_layer(cfg, d, x, w_router, expert_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                    ws_down, mx, router_logits_in, router_logits_out, topk_idx_out, topk_w_out,
                    deterministic, w, st, &lo));
  if (lo.parts.p)
    return hip_ok(launch_combine_parts(lo.parts, lo.topk_w, out, (int)T, d.H, d.k, d.dtype, st));
  return hip_ok(launch_combine(w.acc, lo.y_perm, w.row_pos, lo.topk_w, out, (int)T, d.H, d.k,
                               d.dtype, st));
}

moe_status moe_rms_norm(const moe_config* cfg, const moe_norm_config* norm, int64_t T,
                        const void* x, const float* weight, void* y, moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  MOE_TRY(check_norm(d, norm));
  if (T == 0) return MOE_OK;
  if (!x || !weight || !y) return MOE_ERR_INVALID_ARG;
  return hip_ok(launch_rmsnorm(x, weight, norm->add_one, norm->rms_norm_eps, y, (int)T, d.H,
                               d.dtype, (hipStream_t)stream));
}

moe_status moe_combine_norm_residual(const moe_config* cfg, const moe_norm_config* norm,
                                     int64_t T, const float* acc, const void* y_perm,
                                     const int32_t* row_pos, const float* topk_w,
                                     const float* post_norm_w, const void* residual, void* out,
                                     moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  MOE_TRY(check_norm(d, norm));
  if (T == 0) return MOE_OK;
  if (!acc || !post_norm_w || !residual || !out) return MOE_ERR_INVALID_ARG;
  if (y_perm && (!row_pos || !topk_w)) return MOE_ERR_INVALID_ARG;
  return hip_ok(launch_combine_norm(acc, y_perm, row_pos, topk_w, post_norm_w, norm->add_one,
                                    norm->rms_norm_eps, residual, out, (int)T, d.H, d.k, d.dtype,
                                    (hipStream_t)stream));
}

moe_status moe_block_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes) {
  Dims d;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_cfg(cfg, T, &d));
  *bytes = block_ws_bytes(d);
  return MOE_OK;
}

moe_status moe_block_forward(const moe_config* cfg, const moe_norm_config* norm, int64_t T,
                             const void* h, const float* pre_norm_w, const float* post_norm_w,
                             const void* w_router, const float* expert_bias, const void* w_gate,
                             const void* w_up, const void* w_down, const void* ws_gate,
                             const void* ws_up, const void* ws_down, const moe_mx_scales* mx,
                             float* router_logits_out,
                             int32_t* topk_idx_out, float* topk_w_out, void* out,
                             int32_t deterministic, void* ws, size_t ws_bytes,
                             moe_stream_t stream) {
  Dims d;
  MOE_TRY(check_cfg(cfg, T, &d));
  MOE_TRY(check_norm(d, norm));
  if (T == 0) return MOE_OK;
  if (!pre_norm_w || !post_norm_w || !out) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_layer_args(d, h, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                           nullptr, deterministic, mx));
  MOE_TRY(check_mx(d, mx, true, true));
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < block_ws_bytes(d)) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  Ws w = carve(d, ws);
  void* xn = static_cast<char*>(ws) + w.total;  // normalised rows after the layer's segments
  MOE_TRY(hip_ok(launch_rmsnorm(h, pre_norm_w, norm->add_one, norm->rms_norm_eps, xn, (int)T, d.H,
                                d.dtype, st)));
  LayerOut lo;
  MOE_TRY(run_layer(cfg, d, xn, w_router, expert_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                    ws_down, mx, nullptr, router_logits_out, topk_idx_out, topk_w_out,
                    deterministic, w, st, &lo));
  if (lo.parts.p)
    return hip_ok(launch_combine_norm_parts(lo.parts, lo.topk_w, post_norm_w, norm->add_one,
                                            norm->rms_norm_eps, h, out, (int)T, d.H, d.k,
                                            d.dtype, st));
  return hip_ok(launch_combine_norm(w.acc, lo.y_perm, w.row_pos, lo.topk_w, post_norm_w,
                                    norm->add_one, norm->rms_norm_eps, h, out, (int)T, d.H, d.k,
                                    d.dtype, st));
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: configuration not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
  }
  return "unknown moe_status";
}

const char* moe_build_info(void) { return "libmoe 0.1 gfx950 (bf16/fp32 MFMA, MXFP8 and MXFP4 weights)"; }

}  // extern "C"
