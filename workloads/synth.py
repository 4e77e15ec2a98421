"""Seeded synthetic inputs for the sparse-MoE feed-forward layer.

This module is shared by the float64 oracle side (tests) and the GPU side
(tests, bench). It holds NONE of the layer's arithmetic: it only draws random
numbers, scales them, rounds them to the storage dtype and applies stored
workload parameters (a bias offset on a hot expert set, a copied router row).

Shapes and value ranges follow the pages:
  * AFMoE defaults (hidden 2048, moe_intermediate 1408, 64 experts, top-6,
    2 shared experts, route_scale 1.0, initializer range 0.02): Hugging Face
    Transformers doc "AFMoE", AfmoeConfig parameter list.
  * Trinity routing (route_scale 2.826) and Trinity-Nano shape (hidden 1024,
    128 experts): mlxcel issue #845 "add Arcee AFMoE", "Checkpoint confirmed"
    and "Routing detail".
  * MiniMax-M3 MoE (hidden 6144, 128 experts top-4, routed_scaling_factor 2.0,
    one shared expert of width 3072 packed as slot 128, clamp-SwiGLU with
    alpha 1.702 / limit 7.0 / beta 1.0): mlxcel issue #763 "add MiniMax-M3",
    "Architecture specification", MoE and Activation bullets.
  * The RMSNorms either side of the layer: rms_norm_eps 1e-5 (HF "AFMoE"
    doc, AfmoeConfig); Gemma-style w + 1 scales for MiniMax-M3 (mlxcel #763,
    Norms bullet), whose eps the pages do not print (1e-5 is used).

Seeding: every tensor, and every expert (or token block) within a tensor, has
its own stream np.random.default_rng(SeedSequence([seed, tensor_id, block])).
Draws are float32; bf16 tensors are rounded to nearest-even and kept as raw
uint16 bits, so that both sides consume the same stored values.
"""
from __future__ import annotations

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids of the seeding scheme
TID_X, TID_ROUTER, TID_BIAS = 0, 1, 2
TID_GATE, TID_UP, TID_DOWN = 3, 4, 5
TID_SGATE, TID_SUP, TID_SDOWN = 6, 7, 8
TID_HOTSET = 9
TID_PRE_NORM, TID_POST_NORM = 10, 11

X_BLOCK_ROWS = 256          # rows of x drawn from one stream
_CHUNK = 1 << 20            # elements drawn per call (buffers are reused)

_GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "tests", "golden")


def _cfg(**kw):
    base = dict(
        seed=0, shared_packed=0, score_func="sigmoid", route_norm=1,
        route_scale=1.0, hidden_act="silu", act_alpha=1.702, act_limit=7.0,
        act_beta=1.0, x_scale=1.0, w_std=0.02, router_bf16_values=True,
        skew=None, rms_norm_eps=1e-5, norm_add_one=0, norm_w_std=0.1,
        weight_format="dtype", n_group=1, topk_group=1, router_format="f32",
    )
    base.update(kw)
    if base.get("shared_intermediate_size", 0) == 0:
        base["shared_intermediate_size"] = base["moe_intermediate_size"]
    return base


# The five workloads. Names say what each one is; sizes are in the fields.
CONFIGS: dict[str, dict] = {
    # tiny fp32 layer that the oracle finishes in well under a second
    "tiny_fp32_T64": _cfg(
        T=64, hidden_size=256, num_experts=8, num_experts_per_tok=2,
        moe_intermediate_size=128, num_shared_experts=1,
        shared_intermediate_size=128, dtype="f32", bias_limit=0.1,
        router_bf16_values=False),
    # AFMoE config defaults, input scaled by sqrt(hidden) as the muP option does
    "afmoe_default_T4096": _cfg(
        T=4096, hidden_size=2048, num_experts=64, num_experts_per_tok=6,
        moe_intermediate_size=1408, num_shared_experts=2,
        shared_intermediate_size=1408, dtype="bf16", bias_limit=0.05,
        x_scale=math.sqrt(2048.0)),
    # Trinity-Nano-like layer (top-8, width 256 and one shared expert are
    # assumptions of the workload, not page values); router kept in fp32
    "trinity_nano_decode_T32": _cfg(
        T=32, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False),
    "trinity_nano_prefill_T8192": _cfg(
        T=8192, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False),
    # AFMoE-default shapes with a hot expert set (60% of assignments on 10% of
    # experts) and one exactly tied expert pair
    "skewed_afmoe_T8192": _cfg(
        T=8192, hidden_size=2048, num_experts=64, num_experts_per_tok=6,
        moe_intermediate_size=1408, num_shared_experts=2,
        shared_intermediate_size=1408, dtype="bf16", bias_limit=0.05,
        x_scale=math.sqrt(2048.0), skew="skewed_afmoe_T8192.json"),
    # MiniMax-M3-shaped layer, shared expert packed as slot 128
    "minimax_m3_prefill_T8192": _cfg(
        T=8192, hidden_size=6144, num_experts=128, num_experts_per_tok=4,
        moe_intermediate_size=3072, num_shared_experts=1,
        shared_intermediate_size=3072, shared_packed=1, dtype="bf16",
        bias_limit=0.05, w_std=0.01, route_scale=2.0, hidden_act="swigluoai",
        norm_add_one=1),
    "minimax_m3_decode_T64": _cfg(
        T=64, hidden_size=6144, num_experts=128, num_experts_per_tok=4,
        moe_intermediate_size=3072, num_shared_experts=1,
        shared_intermediate_size=3072, shared_packed=1, dtype="bf16",
        bias_limit=0.05, w_std=0.01, route_scale=2.0, hidden_act="swigluoai",
        norm_add_one=1),
    # the same layers with MXFP8 expert weights (the M3 checkpoint's MXFP8
    # export): the same fp32 draws, quantised instead of rounded to bf16
    "minimax_m3_decode_T64_mxfp8": _cfg(
        T=64, hidden_size=6144, num_experts=128, num_experts_per_tok=4,
        moe_intermediate_size=3072, num_shared_experts=1,
        shared_intermediate_size=3072, shared_packed=1, dtype="bf16",
        bias_limit=0.05, w_std=0.01, route_scale=2.0, hidden_act="swigluoai",
        norm_add_one=1, weight_format="mxfp8"),
    "minimax_m3_prefill_T8192_mxfp8": _cfg(
        T=8192, hidden_size=6144, num_experts=128, num_experts_per_tok=4,
        moe_intermediate_size=3072, num_shared_experts=1,
        shared_intermediate_size=3072, shared_packed=1, dtype="bf16",
        bias_limit=0.05, w_std=0.01, route_scale=2.0, hidden_act="swigluoai",
        norm_add_one=1, weight_format="mxfp8"),
    "trinity_nano_decode_T32_mxfp8": _cfg(
        T=32, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False, weight_format="mxfp8"),
    # 4-bit expert weights (the Trinity checkpoints are 4-bit, router at 8
    # bits; read as MXFP4 and MXFP8), and the M3 decode layer with the same
    # expert format
    "trinity_nano_decode_T32_mxfp4": _cfg(
        T=32, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False, weight_format="mxfp4"),
    "trinity_nano_prefill_T8192_mxfp4": _cfg(
        T=8192, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False, weight_format="mxfp4"),
    "trinity_nano_decode_T32_q4r8": _cfg(
        T=32, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False, weight_format="mxfp4",
        router_format="mxfp8"),
    "trinity_nano_prefill_T8192_q4r8": _cfg(
        T=8192, hidden_size=1024, num_experts=128, num_experts_per_tok=8,
        moe_intermediate_size=256, num_shared_experts=1,
        shared_intermediate_size=256, dtype="bf16", bias_limit=0.05,
        route_scale=2.826, router_bf16_values=False, weight_format="mxfp4",
        router_format="mxfp8"),
    "minimax_m3_decode_T64_mxfp4": _cfg(
        T=64, hidden_size=6144, num_experts=128, num_experts_per_tok=4,
        moe_intermediate_size=3072, num_shared_experts=1,
        shared_intermediate_size=3072, shared_packed=1, dtype="bf16",
        bias_limit=0.05, w_std=0.01, route_scale=2.0, hidden_act="swigluoai",
        norm_add_one=1, weight_format="mxfp4"),
}


def config(name: str, **override) -> dict:
    c = dict(CONFIGS[name])
    c.update(override)
    c["name"] = name
    return c


def layer_keys(cfg: dict) -> dict:
    """The config keys of the layer itself (no workload fields)."""
    keys = ("hidden_size", "num_experts", "num_experts_per_tok",
            "num_shared_experts", "moe_intermediate_size",
            "shared_intermediate_size", "shared_packed", "score_func",
            "route_norm", "route_scale", "hidden_act", "act_alpha",
            "act_limit", "act_beta", "dtype", "weight_format", "n_group", "topk_group",
            "router_format")
    return {k: cfg[k] for k in keys}


# ----------------------------------------------------------------------------
# low-level draws

def _stream(seed: int, tid: int, block: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tid, block]))


def f32_to_bf16_bits(a: np.ndarray, out: np.ndarray | None = None,
                     tmp: np.ndarray | None = None) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if tmp is None:
        tmp = np.empty(u.shape, np.uint32)
    np.right_shift(u, 16, out=tmp)
    np.bitwise_and(tmp, 1, out=tmp)
    np.add(tmp, 0x7FFF, out=tmp)
    np.add(tmp, u, out=tmp)
    np.right_shift(tmp, 16, out=tmp)
    if out is None:
        out = np.empty(u.shape, np.uint16)
    out[...] = tmp
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _fill_normal(dst: np.ndarray, rng: np.random.Generator, std: float,
                 bf16: bool) -> None:
    """dst (flat, float32 or uint16 bits) <- std * N(0,1) draws, in chunks."""
    n = dst.size
    flat = dst.reshape(-1)
    buf = np.empty(min(n, _CHUNK), np.float32)
    tmp = np.empty(buf.size, np.uint32) if bf16 else None
    s = np.float32(std)
    for lo in range(0, n, _CHUNK):
        m = min(_CHUNK, n - lo)
        b = buf[:m]
        rng.standard_normal(out=b, dtype=np.float32)
        if s != np.float32(1.0):
            b *= s
        if bf16:
            f32_to_bf16_bits(b, out=flat[lo:lo + m], tmp=tmp[:m])
        else:
            flat[lo:lo + m] = b


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------

@dataclass
class MoeInputs:
    """Stored input values. bf16 tensors are uint16 bit arrays."""
    cfg: dict
    x: np.ndarray                      # [T, H]
    w_router: np.ndarray               # [E, H] float32
    expert_bias: np.ndarray            # [E] float32
    w_gate: np.ndarray | None = None   # [E_tot, I, H]
    w_up: np.ndarray | None = None     # [E_tot, I, H]
    w_down: np.ndarray | None = None   # [E_tot, H, I]
    ws_gate: np.ndarray | None = None  # [S, I_s, H] (separate shared experts)
    ws_up: np.ndarray | None = None
    ws_down: np.ndarray | None = None  # [S, H, I_s]
    meta: dict = field(default_factory=dict)
    # MXFP8 router (router_format "mxfp8"): w_router holds E4M3 codes [E, H]
    # and mx["router"] their scales [H/32, E].
    # MX expert weights: the w_* / ws_* arrays hold E4M3 codes (MXFP8, uint8
    # [., N, K]) or packed E2M1 codes (MXFP4, uint8 [., N, K/2], input 2j in
    # the low nibble of byte j) and mx holds their E8M0 scales, block-major:
    # [E_tot or S, K/32, N] for a stack of [N, K] matrices (keys gate, up,
    # down, shared_gate, shared_up, shared_down)
    mx: dict | None = None


def load_skew(name: str) -> dict:
    with open(os.path.join(_GOLDEN, name)) as f:
        return json.load(f)


def generate(cfg: dict, T: int | None = None, experts: bool = True,
             apply_skew: bool = True) -> MoeInputs:
    """Draw the inputs of one workload.

    T overrides the token count (x rows are drawn in blocks of 256 from
    per-block streams, so a smaller T gives a prefix of the larger x).
    experts=False skips the expert weights (router-only uses).
    apply_skew=False returns the base draw of a skewed workload.
    """
    seed = cfg["seed"]
    T = cfg["T"] if T is None else T
    H, E = cfg["hidden_size"], cfg["num_experts"]
    I, S, Is = (cfg["moe_intermediate_size"], cfg["num_shared_experts"],
                cfg["shared_intermediate_size"])
    bf16 = cfg["dtype"] == "bf16"
    wdt = np.uint16 if bf16 else np.float32
    wf = cfg.get("weight_format", "dtype")
    if wf not in ("dtype", "mxfp8", "mxfp4"):
        raise ValueError(f"unknown weight_format {wf!r}")
    mx = wf != "dtype"
    kdiv = 2 if wf == "mxfp4" else 1      # MXFP4: two inputs per byte
    xdt = wdt
    std = cfg["w_std"]

    # x: N(0,1) * x_scale, per 256-row block streams
    x = np.empty((T, H), xdt)
    nblk = (T + X_BLOCK_ROWS - 1) // X_BLOCK_ROWS

    def _xblock(b):
        r0 = b * X_BLOCK_ROWS
        r1 = min(T, r0 + X_BLOCK_ROWS)
        full = np.empty((X_BLOCK_ROWS, H), np.float32)
        _fill_normal(full, _stream(seed, TID_X, b), 1.0, False)
        blk = full[: r1 - r0]
        if cfg["x_scale"] != 1.0:
            blk *= np.float32(cfg["x_scale"])
        if bf16:
            f32_to_bf16_bits(blk, out=x[r0:r1])
        else:
            x[r0:r1] = blk

    # router: N(0, std) float32, optionally rounded to bf16 values (stored fp32)
    wr = np.empty((E, H), np.float32)
    _fill_normal(wr, _stream(seed, TID_ROUTER, 0), std, False)
    if cfg["router_bf16_values"]:
        wr = bf16_bits_to_f32(f32_to_bf16_bits(wr)).reshape(E, H)

    # selection bias: U[-lim, lim) float32
    u = _stream(seed, TID_BIAS, 0).random(E, dtype=np.float32)
    lim = np.float32(cfg["bias_limit"])
    bias = ((u * np.float32(2.0) - np.float32(1.0)) * lim).astype(np.float32)

    inp = MoeInputs(cfg=dict(cfg, T=T), x=x, w_router=wr, expert_bias=bias)
    rf = cfg.get("router_format", "f32")
    if rf not in ("f32", "mxfp8"):
        raise ValueError(f"unknown router_format {rf!r}")
    if rf == "mxfp8":
        # the 8-bit router: the same fp32 draw, quantised (codes [E, H],
        # scales [H/32, E])
        inp.w_router, rsc = quantize_mxfp8(wr)
        inp.mx = {"router": rsc}

    jobs = [(_xblock, b) for b in range(nblk)]

    def _matrix(arr, sc, tid, e):
        # one expert's matrix: fp32 draws, then bf16 rounding or MX quantisation
        if sc is None:
            _fill_normal(arr[e], _stream(seed, tid, e), std, bf16)
            return
        n, kc = arr.shape[1:]
        tmp = np.empty((n, kc * kdiv), np.float32)
        _fill_normal(tmp, _stream(seed, tid, e), std, False)
        arr[e], sc[e] = (quantize_mxfp4 if kdiv == 2 else quantize_mxfp8)(tmp)

    if experts:
        Etot = E + (1 if cfg["shared_packed"] else 0)
        edt = np.uint8 if mx else wdt
        inp.w_gate = np.empty((Etot, I, H // kdiv), edt)
        inp.w_up = np.empty((Etot, I, H // kdiv), edt)
        inp.w_down = np.empty((Etot, H, I // kdiv), edt)
        if mx:
            inp.mx = dict(inp.mx or {},
                          gate=np.empty((Etot, H // 32, I), np.uint8),
                          up=np.empty((Etot, H // 32, I), np.uint8),
                          down=np.empty((Etot, I // 32, H), np.uint8))
        scl = (lambda key: inp.mx[key]) if mx else (lambda key: None)
        for arr, key, tid in ((inp.w_gate, "gate", TID_GATE), (inp.w_up, "up", TID_UP),
                              (inp.w_down, "down", TID_DOWN)):
            for e in range(Etot):
                jobs.append((lambda e, arr=arr, sc=scl(key), tid=tid: _matrix(arr, sc, tid, e), e))
        if S > 0 and not cfg["shared_packed"]:
            inp.ws_gate = np.empty((S, Is, H // kdiv), edt)
            inp.ws_up = np.empty((S, Is, H // kdiv), edt)
            inp.ws_down = np.empty((S, H, Is // kdiv), edt)
            if mx:
                inp.mx.update({"shared_gate": np.empty((S, H // 32, Is), np.uint8),
                               "shared_up": np.empty((S, H // 32, Is), np.uint8),
                               "shared_down": np.empty((S, Is // 32, H), np.uint8)})
            for arr, key, tid in ((inp.ws_gate, "shared_gate", TID_SGATE),
                                  (inp.ws_up, "shared_up", TID_SUP),
                                  (inp.ws_down, "shared_down", TID_SDOWN)):
                for s in range(S):
                    jobs.append((lambda s, arr=arr, sc=scl(key), tid=tid: _matrix(arr, sc, tid, s), s))
    nthr = _threads()
    if nthr > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(lambda j: j[0](j[1]), jobs))
    else:
        for fn, a in jobs:
            fn(a)

    if cfg.get("skew") and apply_skew:
        sk = load_skew(cfg["skew"])
        apply_skew_params(inp, sk)
    return inp


# ----------------------------------------------------------------------------
# MXFP8 (OCP Microscaling v1.0: E4M3 elements, one E8M0 scale per 32 inputs)

def quantize_mxfp8(w: np.ndarray):
    """float32 [N, K] -> (codes uint8 [N, K], scales uint8 [K/32, N]).

    Per block of 32 inputs of a row: scale 2^(floor(log2 amax) - 8) (8 is
    E4M3's largest exponent); each element, divided by the scale (exact) and
    clamped to +-448, is rounded to the nearest E4M3 value, ties to the even
    code: from 2^-6 up by rounding the float32 significand to 3 bits (the
    carry moves into the exponent), below it to a multiple of 2^-9 (codes
    0..8, where 8 is 2^-6)."""
    N, K = w.shape
    blk = np.ascontiguousarray(w, dtype=np.float32).reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    ex = np.where(amax > 0, ex - 1, -119)        # floor(log2 amax); zero block: scale byte 0
    sbyte = np.clip(ex - 8 + 127, 0, 254).astype(np.uint8)
    v = blk * np.ldexp(np.float32(1.0), 127 - sbyte.astype(np.int32))[:, :, None]
    a = np.minimum(np.abs(v), np.float32(448.0))
    u = a.view(np.uint32)
    # (u + 0x7FFFF + lsb) >> 20 is (exponent << 3 | mantissa) rounded to
    # nearest even; minus (127 - 7) << 3 rebiases the exponent (wraps below
    # 2^-6, where the subnormal branch is taken instead)
    normal = ((u + np.uint32(0x7FFFF) + ((u >> 20) & np.uint32(1))) >> 20) - np.uint32(120 << 3)
    sub = np.rint(a * np.float32(512.0)).astype(np.uint32)
    code = np.where(a >= np.float32(2.0 ** -6), normal, sub)
    code |= (v.view(np.uint32) >> 24) & np.uint32(0x80)
    return code.astype(np.uint8).reshape(N, K), np.ascontiguousarray(sbyte.T)


# MXFP4 (OCP Microscaling v1.0: E2M1 elements, one E8M0 scale per 32 inputs)

# midpoints between neighbouring E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


def quantize_mxfp4(w: np.ndarray):
    """float32 [N, K] -> (packed codes uint8 [N, K/2], scales uint8 [K/32, N]).

    Per block of 32 inputs of a row: scale 2^(floor(log2 amax) - 2) (2 is
    E2M1's largest exponent); each element, divided by the scale (exact) and
    clamped to +-6, goes to the nearest E2M1 magnitude, ties to the even code
    (code i + 1 past midpoint i; at the midpoint only when i + 1 is even); the
    sign is bit 3. Input 2j is the low nibble of byte j, input 2j+1 the high."""
    N, K = w.shape
    blk = np.ascontiguousarray(w, dtype=np.float32).reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    ex = np.where(amax > 0, ex - 1, -125)        # floor(log2 amax); zero block: scale byte 0
    sbyte = np.clip(ex - 2 + 127, 0, 254).astype(np.uint8)
    v = blk * np.ldexp(np.float32(1.0), 127 - sbyte.astype(np.int32))[:, :, None]
    a = np.minimum(np.abs(v), np.float32(6.0))
    code = np.zeros(a.shape, np.uint8)
    for i, m in enumerate(_E2M1_MID):
        code += (a > m) | ((a == m) & ((i + 1) % 2 == 0))
    code |= ((v.view(np.uint32) >> 28) & np.uint32(0x8)).astype(np.uint8)
    code = code.reshape(N, K)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return np.ascontiguousarray(packed, dtype=np.uint8), np.ascontiguousarray(sbyte.T)


def norm_weights(cfg: dict) -> dict:
    """Weights of the RMSNorms either side of the layer (pre_mlp_norm,
    post_mlp_norm), float32 [H] holding bf16 values, plus eps and the
    Gemma-style offset flag.

    Trained values are not available; the draw centres on the initial value
    of each style (1 for a plain norm scale, 0 for a Gemma-style weight that
    is used as w + 1) with spread norm_w_std."""
    H = cfg["hidden_size"]
    centre = np.float32(0.0 if cfg["norm_add_one"] else 1.0)
    out = {}
    for name, tid in (("pre", TID_PRE_NORM), ("post", TID_POST_NORM)):
        w = np.empty(H, np.float32)
        _fill_normal(w, _stream(cfg["seed"], tid, 0), cfg["norm_w_std"], False)
        w += centre
        out[name] = bf16_bits_to_f32(f32_to_bf16_bits(w))
    out["eps"] = float(cfg["rms_norm_eps"])
    out["add_one"] = int(cfg["norm_add_one"])
    return out


def hot_set(cfg: dict) -> np.ndarray:
    """Seeded choice of floor(0.1*E) hot experts (sorted)."""
    E = cfg["num_experts"]
    n = int(math.floor(0.1 * E))
    rng = _stream(cfg["seed"], TID_HOTSET, 0)
    return np.sort(rng.choice(E, size=n, replace=False)).astype(np.int64)


def apply_skew_params(inp: MoeInputs, sk: dict) -> None:
    """Apply the stored skew parameters: +delta on the hot experts' selection
    bias, and a copy of expert a's router row and bias onto expert c so that
    the two keys tie exactly."""
    hot = np.asarray(sk["hot_experts"], dtype=np.int64)
    delta = np.float32(sk["delta"])
    inp.expert_bias[hot] = (inp.expert_bias[hot] + delta).astype(np.float32)
    a, c = sk["tie_pair"]
    inp.w_router[c] = inp.w_router[a]
    inp.expert_bias[c] = inp.expert_bias[a]
    inp.meta["skew"] = sk
