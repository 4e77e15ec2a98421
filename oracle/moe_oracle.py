"""Float64 CPU oracle of the sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only the tests, the package's smoke check and the CPU-baseline
leg of the benchmark do. It shares no code with the HIP path.

It is the plain definition of the layer, written in float64 numpy from the
pages, one step per function, in the pages' order:

  1. router logits  L = x . W_r^T                     (mlxcel #845 "Checkpoint
     weight layout": the router is mlp.router.gate; HF "AFMoE" doc,
     AfmoeForCausalLM outputs: router_logits are raw, one row per token)
  2. scores         s = sigmoid(L)  (or softmax)      (mlxcel #845 "Routing
     detail": score_func sigmoid; HF "AFMoE" doc, key features / expert
     routing: sigmoid or softmax scoring)
  3. selection key  key = s + expert_bias             (mlxcel #845 "Routing
     detail": bias added for selection only; mlxcel #763 "Architecture
     specification", MoE bullet: e_score_correction_bias, selection only)
  4. top-k          first k experts in the order (key desc, index asc);
                    with n_group > 1 only experts of the topk_group groups
                    with the largest sums of their two best keys
                    (group_limit; mlxcel #845 "Routing detail" names group
                    routing, the rule read from the DeepSeek MoE family)
  5. gather         g = s[idx]   (unbiased scores, mlxcel #845 "Routing detail")
  6. route_norm     w = g / sum(g)                    (mlxcel #845 "Routing detail")
  7. route_scale    w *= route_scale                  (mlxcel #845 "Routing
     detail"; HF "AFMoE" doc, route_scale: scaling for the routed experts)
  8. experts        y = W_d[e] . act(W_g[e] . x, W_u[e] . x)
     silu:      act(g,u) = g*sigmoid(g)*u              (HF "AFMoE" doc, hidden_act)
     swigluoai: act(g,u) = g'*sigmoid(alpha*g')*(u'+beta), g'=min(g,limit),
                u'=clip(u,-limit,limit)                (mlxcel #763, Activation)
  9. shared experts y_s = W_sd . act(W_sg . x, W_su . x), always on, weight 1
     (HF "AFMoE" doc, shared experts; mlxcel #763 MoE bullet: a shared expert
     packed as slot E participates with a fixed score of 1.0)
 10. combine        out = sum_j w_j * y_{idx_j} + sum_s y_s

The MoE block around the layer (mlxcel #845 "What the original body missed",
the sandwich norm layout): out = h + post_mlp_norm(layer(pre_mlp_norm(h))),
with RMSNorm y = x / sqrt(mean(x^2) + eps) * w (HF "AFMoE" doc: rms_norm_eps),
or * (w + 1) for the Gemma-style norms of MiniMax-M3 (mlxcel #763
"Architecture specification", Norms bullet).

Expert weights may also arrive as MXFP8 (mlxcel #763 "Validation": the
checkpoint's MXFP8 export), read as the OCP Microscaling (MX) v1.0 format:
every 32 consecutive inputs of a weight row share one E8M0 scale 2^(e-127)
and each element is an OCP FP8 E4M3 code; a weight is code value x scale.
The layer then runs unchanged on those exact values (mx_dequantize).
The 4-bit weights of the Trinity checkpoints (mlxcel #845 "Checkpoint
confirmed" and "Checkpoint weight layout": 4 bits per weight, the router at
8) have no format on the pages; they are read as OCP MXFP4: E2M1 elements,
two per byte, with the same E8M0 scales; the 8-bit router as MXFP8. The
layer runs on the exact dequantised values (mx_dequantize).

Readings where the pages are silent are listed in the design notes: the bias
is added to the post-sigmoid scores; normalise then scale; no epsilon in the
norm; ties go to the lower expert index and the k indices are emitted in the
selection order; the selection key is formed in float64 from fp32 logits.

Inputs are the exact stored values: bf16 tensors arrive as uint16 bit arrays
and are widened exactly to float64 here.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# storage decoding (exact)

def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored tensor (uint16 = bf16 bits). MX codes
    (uint8) have no value without their scales: dequantise them first
    (mx_dequantize, MxStacked)."""
    a = np.asarray(a)
    if a.dtype == np.uint8:
        raise ValueError("uint8 MX codes: dequantise them with their scales first")
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(F64)
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------
# MX weights (OCP MX v1.0: E4M3 or E2M1 elements, one E8M0 scale per 32 inputs)

MX_BLOCK = 32


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 codes: sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and
    0xFF are NaN; there are no infinities (largest finite 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = (c & 0x7).astype(F64)
    mag = np.where(ef == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(ef.astype(F64) - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def e8m0_value(e: np.ndarray) -> np.ndarray:
    """Exact value of E8M0 scale bytes: 2^(e - 127); 0xFF is NaN."""
    e = np.asarray(e, dtype=np.uint8).astype(F64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP4 E2M1 codes (the low four bits): sign bit 3, two
    exponent bits (bias 1), one mantissa bit; exponent field 0 is subnormal
    (m/2); no infinities or NaN (largest 6)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    ef = (c >> 1) & 0x3
    m = (c & 0x1).astype(F64)
    mag = np.where(ef == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(ef.astype(F64) - 1.0))
    return sign * mag


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] 4-bit codes: input 2j is the low nibble of
    byte j, input 2j+1 the high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, elem: str = "e4m3") -> np.ndarray:
    """Weight values of one MX matrix -> float64 [N, K], with scales [K/32, N]
    (uint8, block-major: the scales of all N rows for each block of 32
    inputs): w[n, k] = element(n, k) * 2^(s[k/32, n] - 127).
    elem "e4m3" (MXFP8): codes [N, K], one byte per input;
    elem "e2m1" (MXFP4): codes [N, K/2], two inputs per byte (unpack_fp4)."""
    # each element value is a function of its code alone: evaluated once per
    # possible code, then looked up (the same numbers, without re-deriving
    # them for every one of the N*K inputs)
    if elem == "e2m1":
        vals = e2m1_value(np.arange(16, dtype=np.uint8))[unpack_fp4(codes)]
    elif elem == "e4m3":
        vals = e4m3_value(np.arange(256, dtype=np.uint8))[np.asarray(codes, dtype=np.uint8)]
    else:
        raise ValueError(f"unknown MX element format {elem!r}")
    K = vals.shape[1]
    sc = e8m0_value(scales).T                                   # [N, K/32]
    return vals * np.repeat(sc, MX_BLOCK, axis=1)[:, :K]


class MxStacked:
    """Stacked MX matrices ([E, N, K] MXFP8 codes or [E, N, K/2] packed MXFP4
    codes, [E, K/32, N] scales) whose item e is the float64 dequantised
    matrix of expert e (computed on access, one expert at a time)."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, elem: str = "e4m3"):
        self.codes, self.scales, self.elem = codes, scales, elem
        E, N, Kc = codes.shape
        self.shape = (E, N, 2 * Kc if elem == "e2m1" else Kc)

    def __len__(self):
        return self.codes.shape[0]

    def __getitem__(self, e):
        return mx_dequantize(self.codes[e], self.scales[e], self.elem)


# ----------------------------------------------------------------------------
# routing

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """L[t, e] = sum_h x[t, h] * W_r[e, h]   (router.gate, a bias-free linear)."""
    return as_f64(x) @ as_f64(w_router).T


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=F64)
    return 1.0 / (1.0 + np.exp(-z))


def scores(logits: np.ndarray, score_func: str = "sigmoid") -> np.ndarray:
    """Per-expert scores from the router logits (float64)."""
    L = np.asarray(logits, dtype=F64)
    if score_func == "sigmoid":
        return sigmoid(L)
    if score_func == "softmax":
        m = L.max(axis=-1, keepdims=True)
        ez = np.exp(L - m)
        return ez / ez.sum(axis=-1, keepdims=True)
    raise ValueError(score_func)


def selection_keys(s: np.ndarray, expert_bias: np.ndarray | None) -> np.ndarray:
    """key = s + b: the bias only ever enters the selection."""
    if expert_bias is None:
        return np.array(s, dtype=F64, copy=True)
    return np.asarray(s, dtype=F64) + as_f64(expert_bias)[None, :]


def select_topk(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, in the total order
    (key descending, expert index ascending); emitted in that order.

    A stable sort on -key keeps equal keys in ascending index order."""
    order = np.argsort(-np.asarray(keys, dtype=F64), axis=-1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_weights(s: np.ndarray, idx: np.ndarray, route_norm: bool,
                  route_scale: float) -> np.ndarray:
    """Gather the UNBIASED scores of the chosen experts, renormalise them to
    sum to one (route_norm), then multiply by route_scale."""
    g = np.take_along_axis(np.asarray(s, dtype=F64), idx.astype(np.int64), axis=-1)
    if route_norm:
        den = g.sum(axis=-1, keepdims=True)
        w = np.divide(g, den, out=np.zeros_like(g), where=den != 0.0)
    else:
        w = g
    return w * F64(route_scale)


def group_limit(keys: np.ndarray, n_group: int, topk_group: int) -> np.ndarray:
    """Group-limited selection (mlxcel #845 "Routing detail" names group
    routing and n_group; read as the rule of the DeepSeek MoE family the page
    derives AFMoE from): the E experts form n_group contiguous groups; a
    group's score is the sum of its two largest selection keys; the
    topk_group best groups (ties: lower group index) stay eligible and every
    other expert's key becomes -inf, out of the top-k."""
    if n_group <= 1:
        return keys
    T, E = keys.shape
    gs = E // n_group
    grp = np.asarray(keys, dtype=F64).reshape(T, n_group, gs)
    top2 = -np.sort(-grp, axis=-1)[:, :, :2]
    gscore = top2[:, :, 0] + top2[:, :, 1]
    keep = np.argsort(-gscore, axis=-1, kind="stable")[:, :topk_group]
    mask = np.zeros((T, n_group), bool)
    np.put_along_axis(mask, keep, True, axis=-1)
    return np.where(np.repeat(mask, gs, axis=1), keys, -np.inf)


def route(logits: np.ndarray, expert_bias: np.ndarray | None, k: int,
          score_func: str = "sigmoid", route_norm: bool = True,
          route_scale: float = 1.0, n_group: int = 1, topk_group: int = 1):
    """Steps 2-7: returns (s, keys, idx [T,k] int32, w [T,k] float64). With
    n_group > 1 the keys of experts outside the kept groups are -inf."""
    s = scores(logits, score_func)
    keys = group_limit(selection_keys(s, expert_bias), n_group, topk_group)
    idx = select_topk(keys, k)
    w = route_weights(s, idx, route_norm, route_scale)
    return s, keys, idx, w


def boundary_gap(keys: np.ndarray, k: int) -> float:
    """Smallest gap between the k-th and (k+1)-th key over all rows (0 means
    an exact tie straddles the boundary somewhere)."""
    E = keys.shape[-1]
    if k >= E:
        return float("inf")
    srt = -np.sort(-np.asarray(keys, dtype=F64), axis=-1)
    return float(np.min(srt[:, k - 1] - srt[:, k]))


# ----------------------------------------------------------------------------
# grouping of the (token, slot) rows by expert

def permute(idx: np.ndarray, num_experts: int):
    """Stable counting sort of the rows r = t*k + j by expert.

    Returns counts[E], offsets[E+1] (exclusive scan), sorted_rows[T*k]
    (rows of expert 0 in ascending r, then expert 1, ...) and row_pos, the
    inverse permutation (row_pos[sorted_rows[p]] = p)."""
    e_of_row = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(e_of_row, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.argsort(e_of_row, kind="stable").astype(np.int32)
    row_pos = np.empty_like(sorted_rows)
    row_pos[sorted_rows] = np.arange(sorted_rows.size, dtype=np.int32)
    return counts, offsets, sorted_rows, row_pos


# ----------------------------------------------------------------------------
# expert MLPs

def act_silu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SwiGLU with SiLU: silu(gate) * up."""
    return g * sigmoid(g) * u


def act_swigluoai(g: np.ndarray, u: np.ndarray, alpha: float, limit: float,
                  beta: float) -> np.ndarray:
    """clamp-SwiGLU: x_glu (gate) clamped from above at limit, x_linear (up)
    clamped to [-limit, limit]; x_glu * sigmoid(alpha*x_glu) * (x_linear+beta)."""
    gc = np.minimum(g, F64(limit))
    uc = np.clip(u, -F64(limit), F64(limit))
    return gc * sigmoid(F64(alpha) * gc) * (uc + F64(beta))


def activation(cfg: dict):
    if cfg["hidden_act"] == "silu":
        return act_silu
    if cfg["hidden_act"] == "swigluoai":
        a, l, b = cfg["act_alpha"], cfg["act_limit"], cfg["act_beta"]
        return lambda g, u: act_swigluoai(g, u, a, l, b)
    raise ValueError(cfg["hidden_act"])


def mlp_hidden(xr: np.ndarray, wg: np.ndarray, wu: np.ndarray, act) -> np.ndarray:
    """act(x . W_g^T, x . W_u^T) for rows xr [n,H], W [I,H] (float64)."""
    return act(xr @ wg.T, xr @ wu.T)


def mlp_out(h: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """h . W_d^T for h [n,I], W_d [H,I]."""
    return h @ wd.T


# ----------------------------------------------------------------------------
# the whole layer

def _shared_weights(inp, cfg):
    """List of (W_g, W_u, W_d) float64 triples of the always-on experts."""
    S = cfg["num_shared_experts"]
    if S == 0:
        return []
    if cfg["shared_packed"]:
        E = cfg["num_experts"]
        return [(as_f64(inp.w_gate[E]), as_f64(inp.w_up[E]), as_f64(inp.w_down[E]))]
    return [(as_f64(inp.ws_gate[s]), as_f64(inp.ws_up[s]), as_f64(inp.ws_down[s]))
            for s in range(S)]


def moe_forward(inp, cfg: dict, logits: np.ndarray | None = None,
                want_hidden: bool = False) -> dict:
    """Full layer over all T tokens. `logits` (fp32 values) replaces step 1
    when given. Expert weights are widened to float64 one expert at a time."""
    T = inp.x.shape[0]
    E, k = cfg["num_experts"], cfg["num_experts_per_tok"]
    x = as_f64(inp.x)
    L = router_logits(inp.x, inp.w_router) if logits is None else as_f64(logits)
    s, keys, idx, w = route(L, inp.expert_bias, k, cfg["score_func"],
                            bool(cfg["route_norm"]), cfg["route_scale"],
                            cfg.get("n_group", 1), cfg.get("topk_group", 1))
    counts, offsets, sorted_rows, row_pos = permute(idx, E)
    act = activation(cfg)
    out = np.zeros((T, x.shape[1]), F64)
    I = cfg["moe_intermediate_size"]
    h = np.zeros((T * k, I), F64) if want_hidden else None
    for e in range(E):
        rows = sorted_rows[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        toks = rows // k
        he = mlp_hidden(x[toks], as_f64(inp.w_gate[e]), as_f64(inp.w_up[e]), act)
        if want_hidden:
            h[offsets[e]:offsets[e + 1]] = he
        ye = mlp_out(he, as_f64(inp.w_down[e]))
        wr = w.reshape(-1)[rows]
        # a token selects an expert at most once, so `toks` has no repeats
        out[toks] += wr[:, None] * ye
    hs_all = []
    for (wg, wu, wd) in _shared_weights(inp, cfg):
        hs = mlp_hidden(x, wg, wu, act)
        hs_all.append(hs)
        out += mlp_out(hs, wd)
    res = dict(logits=L, scores=s, keys=keys, idx=idx, w=w, counts=counts,
               offsets=offsets, sorted_rows=sorted_rows, row_pos=row_pos, out=out)
    if want_hidden:
        res["h"] = h
        res["h_shared"] = np.concatenate(hs_all, axis=1) if hs_all else None
    return res


def moe_forward_tokens(inp, cfg: dict, tokens, logits_rows: np.ndarray | None = None) -> dict:
    """The layer's output rows for a subset of tokens only (routing is per
    token, so each row is computed independently). logits_rows [n,E] (fp32
    values) replaces step 1 for those tokens when given."""
    tokens = np.asarray(tokens, dtype=np.int64)
    k = cfg["num_experts_per_tok"]
    x = as_f64(inp.x[tokens])
    L = (as_f64(inp.x[tokens]) @ as_f64(inp.w_router).T if logits_rows is None
         else as_f64(logits_rows))
    s, keys, idx, w = route(L, inp.expert_bias, k, cfg["score_func"],
                            bool(cfg["route_norm"]), cfg["route_scale"],
                            cfg.get("n_group", 1), cfg.get("topk_group", 1))
    act = activation(cfg)
    out = np.zeros((tokens.size, x.shape[1]), F64)
    for e in np.unique(idx):
        sel_t, sel_j = np.nonzero(idx == e)
        he = mlp_hidden(x[sel_t], as_f64(inp.w_gate[e]), as_f64(inp.w_up[e]), act)
        ye = mlp_out(he, as_f64(inp.w_down[e]))
        out[sel_t] += w[sel_t, sel_j][:, None] * ye
    for (wg, wu, wd) in _shared_weights(inp, cfg):
        out += mlp_out(mlp_hidden(x, wg, wu, act), wd)
    return dict(logits=L, idx=idx, w=w, out=out)


# ----------------------------------------------------------------------------
# the MoE block: pre-norm, layer, post-norm, residual

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float, add_one: bool) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * (w (+ 1))."""
    x = as_f64(x)
    scale = as_f64(w) + (1.0 if add_one else 0.0)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + F64(eps))
    return x * r * scale


def block_forward(inp, cfg: dict, pre_w: np.ndarray, post_w: np.ndarray, eps: float,
                  add_one: bool, logits: np.ndarray | None = None) -> dict:
    """out = h + post_norm(layer(pre_norm(h))), h = inp.x. The layer runs on the
    float64 pre-normed rows; `logits` (fp32 values) replaces its router GEMM
    when given."""
    h = as_f64(inp.x)
    xn = rms_norm(h, pre_w, eps, add_one)
    sub = type(inp)(**{**inp.__dict__, "x": xn})
    res = moe_forward(sub, cfg, logits=logits)
    moe_out = res["out"]
    y = rms_norm(moe_out, post_w, eps, add_one)
    return dict(res, xn=xn, moe_out=moe_out, out=h + y)

