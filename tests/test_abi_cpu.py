"""CPU-only checks of the C ABI: the library loads, exports every function
that include/moe.h declares, and rejects bad arguments on the host before any
launch (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import sparse_moe_transformer_amd as moe
from workloads import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert "moe_layer_forward" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.ENTRY_POINTS)
    assert "gfx950" in moe.moe_build_info()


def _cfg(**kw):
    c = synth.layer_keys(synth.config("afmoe_default_T4096"))
    c.update(kw)
    return c


@pytest.mark.parametrize("bad", [
    dict(hidden_size=100), dict(hidden_size=0), dict(num_experts=0), dict(num_experts=2000),
    dict(num_experts_per_tok=0), dict(num_experts_per_tok=65), dict(num_experts=8, num_experts_per_tok=9),
    dict(moe_intermediate_size=1400), dict(shared_intermediate_size=100),
    dict(shared_packed=1),                       # needs S == 1 and I_s == I
    dict(shared_packed=2), dict(route_norm=3), dict(hidden_act=7), dict(dtype=5),
    dict(route_scale=float("nan")),
])
def test_invalid_config_rejected(bad):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(_cfg(**bad), 16)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_softmax_is_accepted():
    """Softmax scoring is a supported score_func: the workspace query succeeds
    (the query runs every argument check of the entry points)."""
    assert moe.moe_workspace_size(_cfg(score_func="softmax"), 16) > 0


def test_workspace_grows_with_tokens():
    c = _cfg()
    sizes = [moe.moe_workspace_size(c, t) for t in (1, 64, 4096, 8192)]
    assert all(b > a for a, b in zip(sizes, sizes[1:]))
    assert all(s % 256 == 0 for s in sizes)


def _raw_forward(cfg, T, ptr=0x1000, ws=0x100000, ws_bytes=1 << 40, x=True, mx=None):
    """moe_layer_forward with fake (never dereferenced) device addresses."""
    L = moe.lib()
    c = moe.make_config(cfg)
    p = ptr if x else None
    return L.moe_layer_forward(ctypes.byref(c), T, p, ptr, None, ptr, ptr, ptr, ptr, ptr, ptr,
                               mx, None, None, None, None, ptr, 0, ws, ws_bytes, None)


def test_host_checks_run_before_any_launch():
    c = _cfg()
    assert _raw_forward(c, 0) == moe.MOE_OK                      # T == 0: nothing to do
    assert _raw_forward(c, 8, x=False) == moe.MOE_ERR_INVALID_ARG
    assert _raw_forward(c, 8, ws_bytes=1024) == moe.MOE_ERR_WORKSPACE
    assert _raw_forward(c, 8, ws=0x100010) == moe.MOE_ERR_INVALID_ARG   # misaligned
    assert _raw_forward(c, -1) == moe.MOE_ERR_INVALID_ARG


def test_status_strings():
    for code in range(5):
        assert moe.status_string(code).startswith("MOE_")


def _raw_block(cfg, T, norm=None, H_ok=True, ptr=0x1000, ws=0x100000, ws_bytes=1 << 40):
    """moe_block_forward with fake (never dereferenced) device addresses."""
    L = moe.lib()
    c = moe.make_config(cfg)
    n = moe.make_norm_config(norm or {"eps": 1e-5, "add_one": 0})
    return L.moe_block_forward(ctypes.byref(c), ctypes.byref(n), T, ptr, ptr, ptr, ptr, None,
                               ptr, ptr, ptr, ptr, ptr, ptr, None, None, None, None, ptr, 0, ws,
                               ws_bytes, None)


def test_block_host_checks():
    c = _cfg()
    assert _raw_block(c, 0) == moe.MOE_OK
    assert _raw_block(c, 8, ws_bytes=moe.moe_workspace_size(c, 8)) == moe.MOE_ERR_WORKSPACE
    for bad in ({"eps": float("nan")}, {"eps": -1.0}, {"eps": 1e-5, "add_one": 2}):
        assert _raw_block(c, 8, norm=bad) == moe.MOE_ERR_INVALID_ARG
    # a row of more than 8192 columns does not fit one workgroup
    assert _raw_block(_cfg(hidden_size=8256), 8) == moe.MOE_ERR_UNSUPPORTED


def test_block_workspace_adds_the_normalised_rows():
    c = _cfg()
    for T in (1, 64, 4096):
        extra = moe.moe_block_workspace_size(c, T) - moe.moe_workspace_size(c, T)
        assert extra == -(-(T * 2048 * 2) // 256) * 256


def _mx_cfg(**kw):
    c = synth.layer_keys(synth.config("minimax_m3_decode_T64_mxfp8"))
    c.update(kw)
    return c


def test_mxfp8_config_checks():
    """MXFP8 weights need bf16 activations; the scales must be given."""
    assert moe.moe_workspace_size(_mx_cfg(), 64) > 0
    assert moe.moe_workspace_size(_mx_cfg(hidden_size=6208, moe_intermediate_size=1408,
                                          shared_intermediate_size=1408), 64) > 0
    for bad, status in ((dict(weight_format=3), moe.MOE_ERR_INVALID_ARG),
                        (dict(weight_format=-1), moe.MOE_ERR_INVALID_ARG),
                        (dict(dtype="f32"), moe.MOE_ERR_UNSUPPORTED),
                        (dict(dtype="f32", weight_format="mxfp4"), moe.MOE_ERR_UNSUPPORTED)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_workspace_size(_mx_cfg(**bad), 64)
        assert ei.value.status == status, bad
    # missing scales: rejected on the host before any launch
    assert _raw_forward(_mx_cfg(), 8) == moe.MOE_ERR_INVALID_ARG
    m = moe.MoeMxScales(gate=0x2000, up=0x2000, down=None)
    assert _raw_forward(_mx_cfg(), 8, mx=ctypes.byref(m)) == moe.MOE_ERR_INVALID_ARG


def test_mxfp4_config_checks():
    """MXFP4 weights: accepted with bf16 activations, scales required; the
    weights are half a byte each, so the workspace (no weights in it) is the
    same as for MXFP8."""
    c4 = synth.layer_keys(synth.config("minimax_m3_decode_T64_mxfp4"))
    assert c4["weight_format"] == "mxfp4"
    assert moe.moe_workspace_size(c4, 64) == moe.moe_workspace_size(_mx_cfg(), 64)
    assert _raw_forward(c4, 8) == moe.MOE_ERR_INVALID_ARG
    m = moe.MoeMxScales(gate=0x2000, up=0x2000, down=None)
    assert _raw_forward(c4, 8, mx=ctypes.byref(m)) == moe.MOE_ERR_INVALID_ARG


def test_mxfp8_router_checks():
    """An MXFP8 router (the 8-bit router of the 4-bit checkpoints): its scales
    are required unless router logits are passed in, the format is validated,
    and the workspace grows by the dequantised fp32 router (E*H*4, aligned)."""
    c = synth.layer_keys(synth.config("trinity_nano_decode_T32_q4r8"))
    assert c["router_format"] == "mxfp8"
    base = moe.moe_workspace_size(dict(c, router_format="f32"), 32)
    assert moe.moe_workspace_size(c, 32) - base == -(-(128 * 1024 * 4) // 256) * 256
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(dict(c, router_format=2), 32)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    # expert scales present, router scales missing: rejected before any launch
    m = moe.MoeMxScales(gate=0x2000, up=0x2000, down=0x2000, router=None)
    assert _raw_forward(c, 8, mx=ctypes.byref(m)) == moe.MOE_ERR_INVALID_ARG
    cr = dict(c, weight_format="dtype")
    assert _raw_forward(cr, 8) == moe.MOE_ERR_INVALID_ARG
    L = moe.lib()
    cc = moe.make_config(cr)
    assert L.moe_router_logits(ctypes.byref(cc), 8, 0x1000, 0x1000, None, 0x1000, 0x100000,
                               1 << 40, None) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(n_group=3), dict(n_group=65), dict(n_group=8, topk_group=0),
                                 dict(n_group=8, topk_group=9), dict(n_group=64),
                                 dict(n_group=32, topk_group=2), dict(n_group=-1)])
def test_group_routing_config_checks(bad):
    """64 experts, top-6: groups must divide E into groups of at least two
    experts, keep 1..n_group groups, and leave room for k experts."""
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(_cfg(**bad), 16)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_group_routing_accepted():
    assert moe.moe_workspace_size(_cfg(n_group=8, topk_group=3), 16) > 0
    assert moe.moe_workspace_size(_cfg(n_group=1, topk_group=0), 16) > 0   # off



def _tri(**kw):
    c = synth.layer_keys(synth.config("trinity_nano_decode_T32"))
    c.update(kw)
    return c


def test_expert_ffn_applies_where_documented():
    """moe_expert_ffn_size: the partial planes' bytes where the fused decode
    FFN applies (bf16 weights, H 512 or 1024, widths in 128-column slices,
    E <= 256, T <= 32 and T*k <= 256), MOE_ERR_UNSUPPORTED (None) elsewhere."""
    H, I, k = 1024, 256, 8
    for T in (0, 1, 7, 32):
        assert moe.moe_expert_ffn_size(_tri(), T) == (I // 128 * T * k + 256 // 128 * T) * H * 4
    assert moe.moe_expert_ffn_size(_tri(hidden_size=512, num_shared_experts=0), 5) == \
        I // 128 * 5 * k * 512 * 4
    for bad, T in [({}, 33), ({"num_experts_per_tok": 9}, 32), ({"hidden_size": 768}, 8),
                   ({"hidden_size": 2048}, 8), ({"moe_intermediate_size": 192}, 8),
                   ({"shared_intermediate_size": 320}, 8), ({"num_experts": 300}, 8),
                   ({"dtype": "f32"}, 8), ({"weight_format": "mxfp4", "hidden_size": 512}, 8)]:
        assert moe.moe_expert_ffn_size(_tri(**bad), T) is None, bad
    # MX weights: MXFP8 at hidden 512 and 1024, MXFP4 at 1024
    for wf, H in (("mxfp8", 512), ("mxfp8", 1024), ("mxfp4", 1024)):
        assert moe.moe_expert_ffn_size(_tri(weight_format=wf, hidden_size=H), 4) == \
            (I // 128 * 4 * k + 256 // 128 * 4) * H * 4


def test_expert_ffn_host_checks():
    """Null arguments and unsupported shapes are refused before any launch."""
    L = moe.lib()
    p = 0x1000
    c = moe.make_config(_tri())
    ffn = lambda T, parts=p, idx=p, cc=c: L.moe_expert_ffn(ctypes.byref(cc), T, p, p, p, p, p, p, p,
                                                          None, idx, parts, None)
    assert ffn(0) == moe.MOE_OK
    assert ffn(8, parts=None) == moe.MOE_ERR_INVALID_ARG
    assert ffn(8, idx=None) == moe.MOE_ERR_INVALID_ARG
    assert ffn(33) == moe.MOE_ERR_UNSUPPORTED
    assert ffn(8, cc=moe.make_config(_tri(hidden_size=768))) == moe.MOE_ERR_UNSUPPORTED
    # MX weights need their scales
    assert ffn(8, cc=moe.make_config(_tri(weight_format="mxfp4"))) == moe.MOE_ERR_INVALID_ARG
    comb = lambda T, parts=p: L.moe_combine_partials(ctypes.byref(c), T, parts, p, p, None)
    assert comb(0) == moe.MOE_OK
    assert comb(8, parts=None) == moe.MOE_ERR_INVALID_ARG
    assert comb(40) == moe.MOE_ERR_UNSUPPORTED


def test_workspace_covers_smaller_batches_with_the_fused_ffn():
    """The layer's workspace reserves the fused FFN's planes for min(T, 32)
    tokens, so a workspace sized for T tokens serves every smaller batch."""
    c = _tri()
    sizes = [moe.moe_workspace_size(c, t) for t in (1, 8, 31, 32, 33, 64, 8192)]
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))
