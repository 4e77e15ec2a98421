"""Python binding of libmoe.so: the sparse mixture-of-experts feed-forward
layer of AFMoE / MiniMax-M3 on one MI355X.

The functions here carry the names of the C entry points in include/moe.h and
only marshal arguments (device pointers of torch tensors, the stream handle);
every step of the layer runs in the library's HIP kernels. PyTorch provides
device memory and streams. The library must be built first
(`python -m sparse_moe_transformer_amd.build`); nothing falls back to another
implementation when it is missing.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX = 0, 1
MOE_ACT_SILU, MOE_ACT_SWIGLUOAI = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_WEIGHTS_DTYPE, MOE_WEIGHTS_MXFP8, MOE_WEIGHTS_MXFP4 = 0, 1, 2
MOE_ROUTER_F32, MOE_ROUTER_MXFP8 = 0, 1

ENTRY_POINTS = (
    "moe_workspace_size", "moe_router_logits", "moe_route", "moe_permute",
    "moe_grouped_gate_up_swiglu", "moe_grouped_down", "moe_combine",
    "moe_expert_ffn_size", "moe_expert_ffn", "moe_combine_partials",
    "moe_layer_forward", "moe_rms_norm", "moe_combine_norm_residual",
    "moe_block_workspace_size", "moe_block_forward", "moe_status_string",
    "moe_build_info",
)


class MoeConfig(ctypes.Structure):
    """Mirror of moe_config (include/moe.h)."""
    _fields_ = [
        ("hidden_size", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_experts_per_tok", ctypes.c_int32),
        ("num_shared_experts", ctypes.c_int32),
        ("moe_intermediate_size", ctypes.c_int32),
        ("shared_intermediate_size", ctypes.c_int32),
        ("shared_packed", ctypes.c_int32),
        ("score_func", ctypes.c_int32),
        ("route_norm", ctypes.c_int32),
        ("route_scale", ctypes.c_float),
        ("hidden_act", ctypes.c_int32),
        ("act_alpha", ctypes.c_float),
        ("act_limit", ctypes.c_float),
        ("act_beta", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("weight_format", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("router_format", ctypes.c_int32),
    ]


class MoeMxScales(ctypes.Structure):
    """Mirror of moe_mx_scales (include/moe.h): device pointers of the E8M0
    scale tensors of MX (MXFP8, MXFP4) expert weights and of an MXFP8
    router."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate", "up", "down", "shared_gate", "shared_up", "shared_down", "router")]


def make_mx_scales(mx):
    """MoeMxScales from a dict of device tensors (keys as the struct fields),
    or None."""
    if mx is None or isinstance(mx, MoeMxScales):
        return mx
    m = MoeMxScales()
    for n, _ in MoeMxScales._fields_:
        setattr(m, n, _p(mx.get(n)))
    return m


def _mxp(m):
    return ctypes.byref(m) if m is not None else None


class MoeNormConfig(ctypes.Structure):
    """Mirror of moe_norm_config (include/moe.h)."""
    _fields_ = [("rms_norm_eps", ctypes.c_float), ("add_one", ctypes.c_int32)]


def make_norm_config(norm) -> MoeNormConfig:
    """MoeNormConfig from a dict with keys eps / add_one (or pass-through)."""
    if isinstance(norm, MoeNormConfig):
        return norm
    n = MoeNormConfig()
    n.rms_norm_eps = float(norm.get("eps", norm.get("rms_norm_eps", 1e-5)))
    n.add_one = int(norm.get("add_one", 0))
    return n


_SCORE = {"sigmoid": MOE_SCORE_SIGMOID, "softmax": MOE_SCORE_SOFTMAX}
_ACT = {"silu": MOE_ACT_SILU, "swigluoai": MOE_ACT_SWIGLUOAI}
_DT = {"f32": MOE_F32, "bf16": MOE_BF16}
_WF = {"dtype": MOE_WEIGHTS_DTYPE, "mxfp8": MOE_WEIGHTS_MXFP8, "mxfp4": MOE_WEIGHTS_MXFP4}
_RF = {"f32": MOE_ROUTER_F32, "mxfp8": MOE_ROUTER_MXFP8}


def make_config(cfg) -> MoeConfig:
    """MoeConfig from a dict of the layer's config keys (or pass-through)."""
    if isinstance(cfg, MoeConfig):
        return cfg
    c = MoeConfig()
    c.hidden_size = cfg["hidden_size"]
    c.num_experts = cfg["num_experts"]
    c.num_experts_per_tok = cfg["num_experts_per_tok"]
    c.num_shared_experts = cfg.get("num_shared_experts", 0)
    c.moe_intermediate_size = cfg["moe_intermediate_size"]
    c.shared_intermediate_size = cfg.get("shared_intermediate_size", 0)
    c.shared_packed = int(cfg.get("shared_packed", 0))
    sf = cfg.get("score_func", "sigmoid")
    c.score_func = _SCORE.get(sf, sf) if isinstance(sf, str) else sf
    c.route_norm = int(cfg.get("route_norm", 1))
    c.route_scale = float(cfg.get("route_scale", 1.0))
    act = cfg.get("hidden_act", "silu")
    c.hidden_act = _ACT.get(act, act) if isinstance(act, str) else act
    c.act_alpha = float(cfg.get("act_alpha", 1.702))
    c.act_limit = float(cfg.get("act_limit", 7.0))
    c.act_beta = float(cfg.get("act_beta", 1.0))
    dt = cfg.get("dtype", "bf16")
    c.dtype = _DT.get(dt, dt) if isinstance(dt, str) else dt
    wf = cfg.get("weight_format", "dtype")
    c.weight_format = _WF.get(wf, wf) if isinstance(wf, str) else wf
    c.n_group = int(cfg.get("n_group", 1))
    c.topk_group = int(cfg.get("topk_group", 1))
    rf = cfg.get("router_format", "f32")
    c.router_format = _RF.get(rf, rf) if isinstance(rf, str) else rf
    return c


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


_lib = None
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_moe_transformer_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        cp = ctypes.POINTER(MoeConfig)
        ncp = ctypes.POINTER(MoeNormConfig)
        i64, sz, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32
        sig = {
            "moe_workspace_size": [cp, i64, ctypes.POINTER(sz)],
            "moe_router_logits": [cp, i64, _vp, _vp, _vp, _vp, _vp, sz, _vp],
            "moe_route": [cp, i64, _vp, _vp, _vp, _vp, _vp, _vp],
            "moe_permute": [cp, i64, _vp, _vp, _vp, _vp, _vp, sz, _vp],
            "moe_grouped_gate_up_swiglu": [cp, i64] + [_vp] * 10 + [_vp, sz, _vp],
            "moe_grouped_down": [cp, i64] + [_vp] * 10 + [_vp, sz, _vp],
            "moe_combine": [cp, i64, _vp, _vp, _vp, _vp, _vp, _vp],
            "moe_expert_ffn_size": [cp, i64, ctypes.POINTER(sz)],
            "moe_expert_ffn": [cp, i64] + [_vp] * 10 + [_vp],
            "moe_combine_partials": [cp, i64, _vp, _vp, _vp, _vp],
            "moe_layer_forward": [cp, i64] + [_vp] * 15 + [i32, _vp, sz, _vp],
            "moe_rms_norm": [cp, ncp, i64, _vp, _vp, _vp, _vp],
            "moe_combine_norm_residual": [cp, ncp, i64] + [_vp] * 7 + [_vp],
            "moe_block_workspace_size": [cp, i64, ctypes.POINTER(sz)],
            "moe_block_forward": [cp, ncp, i64] + [_vp] * 16 + [i32, _vp, sz, _vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_build_info.argtypes = []
        L.moe_build_info.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(code).decode()


moe_status_string = status_string


def moe_build_info() -> str:
    return lib().moe_build_info().decode()


# ---------------------------------------------------------------------------
# marshalling helpers

def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoeError(st, name)


def _need(t, numel, what):
    if t is not None and not isinstance(t, int) and t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, need {numel}")


# ---------------------------------------------------------------------------
# entry points (same names and argument order as include/moe.h)

def moe_workspace_size(cfg, T: int) -> int:
    c = make_config(cfg)
    n = ctypes.c_size_t(0)
    _call("moe_workspace_size", ctypes.byref(c), int(T), ctypes.byref(n))
    return n.value


def moe_router_logits(cfg, T, x, w_router, logits, ws, stream=None, mx=None):
    """mx: MX scales (an MXFP8 router's in mx["router"]), in the C argument
    list after w_router."""
    c = make_config(cfg)
    m = make_mx_scales(mx)
    _need(logits, T * c.num_experts, "logits")
    _need(x, T * c.hidden_size, "x")
    _call("moe_router_logits", ctypes.byref(c), int(T), _p(x), _p(w_router), _mxp(m), _p(logits),
          _p(ws), ws.numel() if ws is not None else 0, _stream(stream))


def moe_route(cfg, T, logits, expert_bias, topk_idx, topk_w, expert_counts=None, stream=None):
    c = make_config(cfg)
    k = c.num_experts_per_tok
    _need(logits, T * c.num_experts, "logits")
    _need(topk_idx, T * k, "topk_idx")
    _need(topk_w, T * k, "topk_w")
    _need(expert_bias, c.num_experts, "expert_bias")
    _need(expert_counts, c.num_experts, "expert_counts")
    _call("moe_route", ctypes.byref(c), int(T), _p(logits), _p(expert_bias), _p(topk_idx),
          _p(topk_w), _p(expert_counts), _stream(stream))


def moe_permute(cfg, T, topk_idx, expert_offsets, sorted_rows, row_pos, ws, stream=None):
    c = make_config(cfg)
    rows = T * c.num_experts_per_tok
    _need(topk_idx, rows, "topk_idx")
    _need(expert_offsets, c.num_experts + 1, "expert_offsets")
    _need(sorted_rows, rows, "sorted_rows")
    _need(row_pos, rows, "row_pos")
    _call("moe_permute", ctypes.byref(c), int(T), _p(topk_idx), _p(expert_offsets),
          _p(sorted_rows), _p(row_pos), _p(ws), ws.numel() if ws is not None else 0,
          _stream(stream))


def moe_grouped_gate_up_swiglu(cfg, T, x, w_gate, w_up, ws_gate, ws_up, expert_offsets,
                               sorted_rows, h, h_shared, ws, stream=None, mx=None):
    """mx: MX scales (dict of device tensors or MoeMxScales), in the C
    argument list after ws_up."""
    c = make_config(cfg)
    m = make_mx_scales(mx)
    _need(h, T * c.num_experts_per_tok * c.moe_intermediate_size, "h")
    _call("moe_grouped_gate_up_swiglu", ctypes.byref(c), int(T), _p(x), _p(w_gate), _p(w_up),
          _p(ws_gate), _p(ws_up), _mxp(m), _p(expert_offsets), _p(sorted_rows), _p(h),
          _p(h_shared), _p(ws), ws.numel() if ws is not None else 0, _stream(stream))


def moe_grouped_down(cfg, T, h, w_down, h_shared, ws_down, expert_offsets, sorted_rows, topk_w,
                     acc, y_perm, ws, stream=None, mx=None):
    """mx: MX scales, in the C argument list after ws_down."""
    c = make_config(cfg)
    m = make_mx_scales(mx)
    _need(acc, T * c.hidden_size, "acc")
    _need(y_perm, T * c.num_experts_per_tok * c.hidden_size, "y_perm")
    _call("moe_grouped_down", ctypes.byref(c), int(T), _p(h), _p(w_down), _p(h_shared),
          _p(ws_down), _mxp(m), _p(expert_offsets), _p(sorted_rows), _p(topk_w), _p(acc),
          _p(y_perm), _p(ws), ws.numel() if ws is not None else 0, _stream(stream))


def moe_combine(cfg, T, acc, y_perm, row_pos, topk_w, out, stream=None):
    c = make_config(cfg)
    _need(out, T * c.hidden_size, "out")
    _call("moe_combine", ctypes.byref(c), int(T), _p(acc), _p(y_perm), _p(row_pos), _p(topk_w),
          _p(out), _stream(stream))


def moe_expert_ffn_size(cfg, T: int):
    """Bytes of the fused FFN's partial planes, or None where it does not
    apply (MOE_ERR_UNSUPPORTED)."""
    c = make_config(cfg)
    n = ctypes.c_size_t(0)
    st = lib().moe_expert_ffn_size(ctypes.byref(c), int(T), ctypes.byref(n))
    if st == MOE_ERR_UNSUPPORTED:
        return None
    if st != MOE_OK:
        raise MoeError(st, "moe_expert_ffn_size")
    return n.value


def moe_expert_ffn(cfg, T, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, topk_idx, parts,
                   stream=None, mx=None):
    """mx: MX scales, in the C argument list after ws_down."""
    c = make_config(cfg)
    m = make_mx_scales(mx)
    need = moe_expert_ffn_size(cfg, T)
    if need is not None:
        _need(parts, need // 4, "parts")
    _call("moe_expert_ffn", ctypes.byref(c), int(T), _p(x), _p(w_gate), _p(w_up), _p(w_down),
          _p(ws_gate), _p(ws_up), _p(ws_down), _mxp(m), _p(topk_idx), _p(parts), _stream(stream))


def moe_combine_partials(cfg, T, parts, topk_w, out, stream=None):
    c = make_config(cfg)
    _need(out, T * c.hidden_size, "out")
    _call("moe_combine_partials", ctypes.byref(c), int(T), _p(parts), _p(topk_w), _p(out),
          _stream(stream))


def moe_layer_forward(cfg, T, x, w_router, expert_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, router_logits_in, router_logits_out, topk_idx_out, topk_w_out,
                      out, deterministic, ws, stream=None, mx=None):
    """mx: MX scales, in the C argument list after ws_down."""
    c = make_config(cfg)
    m = make_mx_scales(mx)
    k = c.num_experts_per_tok
    _need(x, T * c.hidden_size, "x")
    _need(out, T * c.hidden_size, "out")
    _need(router_logits_in, T * c.num_experts, "router_logits_in")
    _need(router_logits_out, T * c.num_experts, "router_logits_out")
    _need(topk_idx_out, T * k, "topk_idx_out")
    _need(topk_w_out, T * k, "topk_w_out")
    _call("moe_layer_forward", ctypes.byref(c), int(T), _p(x), _p(w_router), _p(expert_bias),
          _p(w_gate), _p(w_up), _p(w_down), _p(ws_gate), _p(ws_up), _p(ws_down), _mxp(m),
          _p(router_logits_in), _p(router_logits_out), _p(topk_idx_out), _p(topk_w_out),
          _p(out), int(deterministic), _p(ws), ws.numel() if ws is not None else 0,
          _stream(stream))


def moe_rms_norm(cfg, norm, T, x, weight, y, stream=None):
    c = make_config(cfg)
    n = make_norm_config(norm)
    _need(x, T * c.hidden_size, "x")
    _need(y, T * c.hidden_size, "y")
    _need(weight, c.hidden_size, "weight")
    _call("moe_rms_norm", ctypes.byref(c), ctypes.byref(n), int(T), _p(x), _p(weight), _p(y),
          _stream(stream))


def moe_combine_norm_residual(cfg, norm, T, acc, y_perm, row_pos, topk_w, post_norm_w,
                              residual, out, stream=None):
    c = make_config(cfg)
    n = make_norm_config(norm)
    _need(acc, T * c.hidden_size, "acc")
    _need(residual, T * c.hidden_size, "residual")
    _need(out, T * c.hidden_size, "out")
    _need(post_norm_w, c.hidden_size, "post_norm_w")
    _call("moe_combine_norm_residual", ctypes.byref(c), ctypes.byref(n), int(T), _p(acc),
          _p(y_perm), _p(row_pos), _p(topk_w), _p(post_norm_w), _p(residual), _p(out),
          _stream(stream))


def moe_block_workspace_size(cfg, T: int) -> int:
    c = make_config(cfg)
    nb = ctypes.c_size_t(0)
    _call("moe_block_workspace_size", ctypes.byref(c), int(T), ctypes.byref(nb))
    return nb.value


def moe_block_forward(cfg, norm, T, h, pre_norm_w, post_norm_w, w_router, expert_bias, w_gate,
                      w_up, w_down, ws_gate, ws_up, ws_down, router_logits_out, topk_idx_out,
                      topk_w_out, out, deterministic, ws, stream=None, mx=None):
    """mx: MX scales, in the C argument list after ws_down."""
    c = make_config(cfg)
    m = make_mx_scales(mx)
    n = make_norm_config(norm)
    k = c.num_experts_per_tok
    _need(h, T * c.hidden_size, "h")
    _need(out, T * c.hidden_size, "out")
    _need(pre_norm_w, c.hidden_size, "pre_norm_w")
    _need(post_norm_w, c.hidden_size, "post_norm_w")
    _need(router_logits_out, T * c.num_experts, "router_logits_out")
    _need(topk_idx_out, T * k, "topk_idx_out")
    _need(topk_w_out, T * k, "topk_w_out")
    _call("moe_block_forward", ctypes.byref(c), ctypes.byref(n), int(T), _p(h), _p(pre_norm_w),
          _p(post_norm_w), _p(w_router), _p(expert_bias), _p(w_gate), _p(w_up), _p(w_down),
          _p(ws_gate), _p(ws_up), _p(ws_down), _mxp(m), _p(router_logits_out), _p(topk_idx_out),
          _p(topk_w_out), _p(out), int(deterministic), _p(ws),
          ws.numel() if ws is not None else 0, _stream(stream))


# ---------------------------------------------------------------------------
# device plumbing for callers (torch memory only)

def torch_dtype(cfg):
    import torch
    c = make_config(cfg)
    return torch.bfloat16 if c.dtype == MOE_BF16 else torch.float32


def alloc_workspace(cfg, T, device="cuda"):
    import torch
    return torch.empty(moe_workspace_size(cfg, T), dtype=torch.uint8, device=device)


def alloc_block_workspace(cfg, T, device="cuda"):
    import torch
    return torch.empty(moe_block_workspace_size(cfg, T), dtype=torch.uint8, device=device)


def to_device(arr, device="cuda"):
    """numpy array -> torch tensor on device (uint16 arrays are bf16 bits)."""
    import numpy as np
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
