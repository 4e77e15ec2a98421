// Routing: one wavefront per token.
//
// The rule (mlxcel #845 "Routing detail"; mlxcel #763 "Architecture
// specification", MoE bullet): sigmoid scores; a per-expert bias is added for
// SELECTION only; the k chosen weights are gathered from the unbiased
// scores, renormalised to sum to one (route_norm) and multiplied by
// route_scale. Softmax scoring (HF "AFMoE" doc, key features: sigmoid or
// softmax scores) replaces the sigmoid by exp(L - max L) / sum over the E
// routed experts; the rest of the rule is the same.
//
// The selection key s + b is formed in fp64 from the fp32 logit, so that the
// order of two keys is decided exactly the same way as by a float64
// reference fed the same logits (exactly equal logits give exactly equal
// keys; distinct keys would have to lie within ~1e-16 of each other for the
// last-ulp differences of two exp implementations to matter). Ties go to the
// lower expert index, and the k indices are emitted in selection order.
//
// Lane l holds experts l, l+64, ... (NPL per lane). Each of the k rounds
// takes the lane-local best live candidate, reduces (key desc, index asc)
// within rows of 16 lanes by DPP exchanges (xor 1, xor 2, half-row mirror,
// row mirror: each pairs lanes symmetrically, so every lane ends with its
// row's best), then combines the four row winners read with readlane. The
// winner's lane retires it. No LDS round trip is involved.
//
// Group-limited selection (n_group > 1; mlxcel #845 "Routing detail" names
// group routing, the rule read from the DeepSeek MoE family): the wave
// writes its token's keys to LDS, lane g finds the two largest keys of group
// g (experts g*gs .. g*gs+gs-1) and adds them in fp64 (largest first), the
// topk_group best groups are picked by the same argmax rounds (ties: lower
// group), and experts outside them drop out of the top-k rounds.
#include <float.h>
#include <limits.h>

#include <cstdlib>
#include <cstring>

#include "moe_common.h"
#include "moe_kernels.h"

namespace {

// fp64 -> uint64 with the same order (finite values; -0 is never formed:
// keys are normalised with + 0.0)
__device__ __forceinline__ uint64_t ordered_bits(double d) {
  const uint64_t u = __double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

struct Cand {
  uint64_t k;  // ordered key; 0 = no candidate
  int i;       // expert index; INT_MAX = no candidate
};

__device__ __forceinline__ bool better(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

template <int CTRL>
__device__ __forceinline__ void dpp_step(Cand& c) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)c.k, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(c.k >> 32), CTRL, 0xF, 0xF, false);
  const int pi = __builtin_amdgcn_update_dpp(0, c.i, CTRL, 0xF, 0xF, false);
  const uint64_t pk = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
  if (better(pk, pi, c.k, c.i)) {
    c.k = pk;
    c.i = pi;
  }
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wave-wide max / sum of a double by a fixed butterfly (every lane ends with
// the same value; the order is the same on every call).
__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// The wave's best (key desc, index asc) of the lanes' candidates c, as
// uniform values: DPP exchanges within rows of 16 lanes, then the four row
// winners by readlane.
__device__ __forceinline__ void wave_best(Cand c, uint64_t& wk, int& wi) {
  dpp_step<0xB1>(c);   // quad_perm [1,0,3,2]: lane ^ 1
  dpp_step<0x4E>(c);   // quad_perm [2,3,0,1]: lane ^ 2
  dpp_step<0x141>(c);  // row_half_mirror: i <-> 7 - i within 8 lanes
  dpp_step<0x140>(c);  // row_mirror: i <-> 15 - i within 16 lanes
  wk = 0;
  wi = INT_MAX;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)c.k, 16 * row);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(c.k >> 32), 16 * row);
    const int ri = __builtin_amdgcn_readlane(c.i, 16 * row);
    const uint64_t rk = ((uint64_t)hi << 32) | lo;
    if (better(rk, ri, wk, wi)) {
      wk = rk;
      wi = ri;
    }
  }
}

// Where a token's logits come from: the row Lrow, or (planes != nullptr) the
// sum of np partial planes (plane stride pstride floats, summed in plane
// order in fp32), which is then also stored to out.
struct LogitSrc {
  const float* planes;
  int np;
  size_t pstride;
  float* out;
};

__device__ __forceinline__ float token_logit(const float* Lrow, const LogitSrc& src, int e) {
  if (!src.planes) return Lrow[e];
  // every plane's load issued before the first add (np <= ROUTER_MAX_PLANES)
  float p[ROUTER_MAX_PLANES];
#pragma unroll
  for (int g = 0; g < ROUTER_MAX_PLANES; ++g)
    p[g] = g < src.np ? src.planes[(size_t)g * src.pstride + e] : 0.f;
  float v = p[0];
#pragma unroll
  for (int g = 1; g < ROUTER_MAX_PLANES; ++g)
    if (g < src.np) v += p[g];
  src.out[e] = v;
  return v;
}

// Routes token row Lrow (one wavefront): writes its k indices and weights
// (lanes < k, in selection order) and, if ex_row is given, the indices there.
// gk: E doubles of LDS for this wave when n_group > 1 (else unused).
template <int NPL>
__device__ __forceinline__ void route_token(const float* Lrow,
                                            const float* __restrict__ bias, int E, int k,
                                            int score_func, int route_norm, float route_scale,
                                            int32_t* __restrict__ idx_row,
                                            float* __restrict__ w_row, int* ex_row,
                                            int32_t* __restrict__ counts, int n_group = 1,
                                            int topk_group = 1, double* gk = nullptr,
                                            LogitSrc src = LogitSrc{nullptr, 0, 0, nullptr}) {
  const int lane = threadIdx.x & 63;
  double key[NPL], sc[NPL];
  bool live[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < E;
    sc[i] = live[i] ? (double)token_logit(Lrow, src, e) : 0.0;
  }
  if (score_func == MOE_SCORE_SOFTMAX) {
    double m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (live[i]) m = fmax(m, sc[i]);
    m = wave_max_f64(m);
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      sc[i] = live[i] ? exp(sc[i] - m) : 0.0;
      part += sc[i];
    }
    const double den = wave_sum_f64(part);
#pragma unroll
    for (int i = 0; i < NPL; ++i) sc[i] = sc[i] / den;
  } else {
#pragma unroll
    for (int i = 0; i < NPL; ++i) sc[i] = 1.0 / (1.0 + exp(-sc[i]));
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = live[i] ? (sc[i] + (bias ? (double)bias[e] : 0.0)) + 0.0 : 0.0;
    if (!live[i]) sc[i] = 0.0;
  }
  if (n_group > 1 && gk) {
    const int gs = E / n_group;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (live[i]) gk[lane + 64 * i] = key[i];
    // this wave's LDS writes complete before its reads (and stay in order)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __asm__ __volatile__("" ::: "memory");
    bool gcand = lane < n_group;
    double gsc = 0.0;
    if (gcand) {
      double m1 = -INFINITY, m2 = -INFINITY;
      for (int i = 0; i < gs; ++i) {
        const double v = gk[lane * gs + i];
        if (v > m1) {
          m2 = m1;
          m1 = v;
        } else if (v > m2) {
          m2 = v;
        }
      }
      gsc = m1 + m2;
    }
    uint64_t kept = 0;
    for (int j = 0; j < topk_group; ++j) {
      Cand c{0ull, INT_MAX};
      if (gcand) {
        c.k = ordered_bits(gsc + 0.0);
        c.i = lane;
      }
      uint64_t wk;
      int wi;
      wave_best(c, wk, wi);
      kept |= 1ull << wi;
      if (lane == wi) gcand = false;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (live[i] && !((kept >> ((lane + 64 * i) / gs)) & 1)) live[i] = false;
  }
  double gsum = 0.0, my_g = 0.0;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    Cand c{0ull, INT_MAX};
    // candidates are visited in ascending index, so '>' keeps the lowest
    // index among equal keys
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      if (live[i]) {
        const uint64_t o = ordered_bits(key[i]);
        if (c.i == INT_MAX || o > c.k) {
          c.k = o;
          c.i = lane + 64 * i;
        }
      }
    }
    uint64_t wk;
    int wi;
    wave_best(c, wk, wi);
    const int wl = wi & 63, wslot = wi >> 6;
    double s_sel = 0.0;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i == wslot) {
        s_sel = sc[i];
        if (lane == wl) live[i] = false;
      }
    const double bs = readlane_f64(s_sel, wl);
    gsum += bs;  // same order (j = 0..k-1) in every lane
    if (lane == j) {
      my_g = bs;
      my_idx = wi;
    }
  }
  if (lane < k) {
    double w = my_g;
    if (route_norm) w = gsum != 0.0 ? w / gsum : 0.0;
    w *= (double)route_scale;
    idx_row[lane] = my_idx;
    w_row[lane] = (float)w;
    if (ex_row) ex_row[lane] = my_idx;
    if (counts) atomicAdd(counts + my_idx, 1);
  }
}

template <int NPL, bool GROUPED>
__global__ void __launch_bounds__(256) route_kernel(const float* logits,
                                                    const float* __restrict__ planes, int np,
                                                    float* logits_out,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int score_func, int route_norm,
                                                    float route_scale,
                                                    int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out,
                                                    int32_t* __restrict__ counts, int n_group,
                                                    int topk_group) {
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave leaves together
  const LogitSrc src{planes ? planes + (size_t)t * E : nullptr, np, (size_t)T * E,
                     planes ? logits_out + (size_t)t * E : nullptr};
  if constexpr (GROUPED) {
    __shared__ double gk[4][64 * NPL];
    route_token<NPL>(logits + (size_t)t * E, bias, E, k, score_func, route_norm, route_scale,
                     idx_out + (size_t)t * k, w_out + (size_t)t * k, nullptr, counts, n_group,
                     topk_group, gk[threadIdx.x >> 6], src);
  } else {
    route_token<NPL>(logits + (size_t)t * E, bias, E, k, score_func, route_norm, route_scale,
                     idx_out + (size_t)t * k, w_out + (size_t)t * k, nullptr, counts, 1, 1,
                     nullptr, src);
  }
}

// Sigmoid scores without a group limit, E <= 256: one workgroup of 256
// threads per token. Thread e forms expert e's score and selection key as
// route_token does. The rank of expert e is the number of experts whose key
// is larger, or equal with a lower index; 256 / E2 threads per expert (E2:
// E rounded up to a power of two) count it over equal shares of the keys in
// LDS. Ranks are distinct, so the experts of rank < k are the selection in
// selection order: the same experts, order, weights and weight arithmetic
// as the k arg-max rounds of route_token, found in parallel.
constexpr int RANK_MAX_E = 256;

__global__ void __launch_bounds__(256) route_rank_kernel(
    const float* logits, const float* __restrict__ planes, int np, float* logits_out,
    const float* __restrict__ bias, int T, int E, int E2, int k, int route_norm,
    float route_scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts) {
  __shared__ uint64_t keys[RANK_MAX_E];
  __shared__ int part[256];
  __shared__ double sel_s[32];
  __shared__ int sel_e[32];
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  double sc = 0.0;
  if (e < E) {
    const LogitSrc src{planes ? planes + (size_t)t * E : nullptr, np, (size_t)T * E,
                       planes ? logits_out + (size_t)t * E : nullptr};
    sc = 1.0 / (1.0 + exp(-(double)token_logit(logits + (size_t)t * E, src, e)));
    keys[e] = ordered_bits((sc + (bias ? (double)bias[e] : 0.0)) + 0.0);
  }
  __syncthreads();
  // thread i counts for expert i % E2 over share i / E2 of the keys
  const int tpc = 256 / E2;
  const int ei = threadIdx.x & (E2 - 1), pi = threadIdx.x / E2;
  const int cs = (E + tpc - 1) / tpc;
  int cnt = 0;
  if (ei < E) {
    const uint64_t mine = keys[ei];
    const int lo = pi * cs, hi = min(E, lo + cs);
#pragma unroll 4
    for (int j = lo; j < hi; ++j) {
      const uint64_t o = keys[j];
      cnt += (o > mine || (o == mine && j < ei)) ? 1 : 0;
    }
  }
  part[threadIdx.x] = cnt;
  __syncthreads();
  if (e < E) {
    int rank = 0;
    for (int q = 0; q < tpc; ++q) rank += part[e + E2 * q];
    if (rank < k) {
      sel_e[rank] = e;
      sel_s[rank] = sc;
    }
  }
  __syncthreads();
  if (e < k) {
    double gsum = 0.0;
    for (int j = 0; j < k; ++j) gsum += sel_s[j];  // selection order, as route_token
    double w = sel_s[e];
    if (route_norm) w = gsum != 0.0 ? w / gsum : 0.0;
    w *= (double)route_scale;
    idx_out[(size_t)t * k + e] = sel_e[e];
    w_out[(size_t)t * k + e] = (float)w;
    if (counts) atomicAdd(counts + sel_e[e], 1);
  }
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int score_func, int route_norm, float route_scale, int32_t* idx,
                        float* w, int32_t* counts, hipStream_t st, int n_group,
                        int topk_group, const float* planes, int np, float* logits_out) {
  // decode-sized batches with sigmoid scores, no group limit, E <= 256: the
  // rank selection, whose parallel counting shortens each token's chain
  // (measured: 13.5 vs 14.5 us alone at T = 32, equal at T = 64; for large
  // batches it is the more work, 44 vs 21 us at T = 8192). MOE_ROUTE_RANK=0
  // / =1 force the arg-max rounds / the ranks (testing knobs).
  const char* knob = std::getenv("MOE_ROUTE_RANK");
  const bool rank_ok = score_func == MOE_SCORE_SIGMOID && n_group <= 1 && E <= RANK_MAX_E;
  const bool rank = rank_ok && (knob && std::strcmp(knob, "1") == 0   ? true
                                : knob && std::strcmp(knob, "0") == 0 ? false
                                                                       : T <= 64);
  if (rank) {
    int E2 = 1;
    while (E2 < E) E2 <<= 1;
    hipLaunchKernelGGL(route_rank_kernel, dim3(T), dim3(256), 0, st, logits, planes, np,
                       logits_out, bias, T, E, E2, k, route_norm, route_scale, idx, w, counts);
    return hipGetLastError();
  }
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  const int npl = (E + 63) / 64;
#define MOE_ROUTE(N)                                                                       \
  do {                                                                                     \
    if (n_group > 1)                                                                       \
      hipLaunchKernelGGL((route_kernel<N, true>), grid, block, 0, st, logits, planes, np,  \
                         logits_out, bias, T, E, k, score_func, route_norm, route_scale,   \
                         idx, w, counts, n_group, topk_group);                             \
    else                                                                                   \
      hipLaunchKernelGGL((route_kernel<N, false>), grid, block, 0, st, logits, planes, np, \
                         logits_out, bias, T, E, k, score_func, route_norm, route_scale,   \
                         idx, w, counts, 1, 1);                                            \
  } while (0)
  if (npl <= 1) MOE_ROUTE(1);
  else if (npl <= 2) MOE_ROUTE(2);
  else if (npl <= 4) MOE_ROUTE(4);
  else if (npl <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}
