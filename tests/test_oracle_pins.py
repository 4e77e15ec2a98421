"""Pins of the float64 oracle against facts fixed outside the oracle itself:
hand-worked examples of the routing rule, closed forms, brute-force top-k,
invariants of the selection-only bias and of route_norm, and degenerate
layers that reduce to a textbook MLP or a dense mixture.

Pages: mlxcel issue #845 (Arcee AFMoE) "Routing detail"; HF Transformers doc
"AFMoE" (AfmoeConfig, expert routing, shared experts); mlxcel issue #763
(MiniMax-M3) "Architecture specification" (MoE and Activation bullets) and
"Implementation plan" (tests of router selection with bias and of the packed
shared expert).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
ULP1 = np.finfo(np.float64).eps


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _logit(s):
    return {"0": 0.0, "ln2": math.log(2.0), "ln3": math.log(3.0), "-ln3": -math.log(3.0),
            "ln4": math.log(4.0), "-ln4": -math.log(4.0)}[s]


# --------------------------------------------------------------------------
# sigmoid

def test_sigmoid_closed_forms():
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(O.sigmoid(np.array([math.log(3.0)]))[0] - 0.75) <= 2 * ULP1
    assert abs(O.sigmoid(np.array([-math.log(4.0)]))[0] - 0.2) <= 2 * ULP1
    z = np.linspace(-30, 30, 2001)
    assert np.max(np.abs(O.sigmoid(z) + O.sigmoid(-z) - 1.0)) <= 2 * ULP1
    # saturation: exactly 1.0 far right; monotone
    assert O.sigmoid(np.array([40.0]))[0] == 1.0
    assert np.all(np.diff(O.sigmoid(z)) >= 0)


def test_softmax_scores():
    L = np.random.default_rng(1).standard_normal((5, 7))
    s = O.scores(L, "softmax")
    assert np.allclose(s.sum(-1), 1.0, rtol=0, atol=4 * ULP1)
    assert np.allclose(O.scores(np.zeros((1, 4)), "softmax"), 0.25, rtol=0, atol=0)


def test_softmax_two_experts_is_sigmoid_of_the_difference():
    """softmax(a, b)_0 = 1 / (1 + e^(b - a)) = sigmoid(a - b): the oracle's
    softmax against its (separately pinned) sigmoid, a closed-form identity."""
    rng = np.random.default_rng(3)
    a, b = rng.normal(0, 4, 200), rng.normal(0, 4, 200)
    s = O.scores(np.stack([a, b], axis=1), "softmax")
    assert np.max(np.abs(s[:, 0] - O.sigmoid(a - b))) <= 4 * ULP1


def test_softmax_shift_invariant_and_finite_for_large_logits():
    """Subtracting the row maximum keeps large logits finite; adding a
    constant to every logit leaves the scores unchanged."""
    L = np.random.default_rng(4).normal(0, 3, (6, 9))
    s = O.scores(L, "softmax")
    s_big = O.scores(L + 800.0, "softmax")
    assert np.all(np.isfinite(s_big))
    assert np.max(np.abs(s_big - s)) <= 1e-12
    # a planted mistake (no max subtraction) overflows at these logits
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(L + 800.0) / np.exp(L + 800.0).sum(-1, keepdims=True)
    assert not np.all(np.isfinite(naive))


def test_softmax_route_norm_cancels_the_full_normaliser():
    """With route_norm on, softmax weights equal route_scale times the softmax
    over the k chosen logits alone (the sum over all E experts cancels)."""
    rng = np.random.default_rng(5)
    L = rng.normal(0, 2, (40, 16))
    b = rng.uniform(-0.05, 0.05, 16)
    _, _, idx, w = O.route(L, b, 4, "softmax", True, 2.5)
    Ls = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    ez = np.exp(Ls - Ls.max(axis=1, keepdims=True))
    assert np.max(np.abs(w - 2.5 * ez / ez.sum(axis=1, keepdims=True))) <= 1e-14


def test_route_softmax_hand_example():
    g = _gold("route_softmax_hand_example.json")
    for case in g["cases"]:
        L = np.array([[_logit(v) for v in case["logits"]]])
        b = np.array(case["bias"], dtype=np.float64)
        s, keys, idx, w = O.route(L, b, g["k"], "softmax", case["route_norm"], g["route_scale"])
        assert np.allclose(s[0], case["scores"], rtol=0, atol=4 * ULP1), case["what"]
        assert idx[0].tolist() == case["idx"], case["what"]
        assert np.allclose(w[0], case["w"], rtol=8 * ULP1, atol=0), case["what"]
        if "idx_without_bias" in case:
            _, _, idx0, _ = O.route(L, None, g["k"], "softmax", True, g["route_scale"])
            assert idx0[0].tolist() == case["idx_without_bias"]


# --------------------------------------------------------------------------
# routing rule: hand-worked example

def test_route_hand_example():
    g = _gold("route_hand_example.json")
    for case in g["cases"]:
        L = np.array([[_logit(v) for v in case["logits"]]])
        b = np.array(case["bias"], dtype=np.float64)
        s, keys, idx, w = O.route(L, b, g["k"], "sigmoid", g["route_norm"], g["route_scale"])
        assert np.allclose(s[0], case["scores"], rtol=0, atol=4 * ULP1)
        assert idx[0].tolist() == case["idx"], case["what"]
        assert np.allclose(w[0], case["w"], rtol=4 * ULP1, atol=0), case["what"]
        if "idx_without_bias" in case:
            _, _, idx0, _ = O.route(L, None, g["k"], "sigmoid", True, g["route_scale"])
            assert idx0[0].tolist() == case["idx_without_bias"]


def test_route_hand_example_catches_bias_on_logits():
    """A plausible mistake (bias added to the logits) changes the selection."""
    case = _gold("route_hand_example.json")["cases"][0]
    L = np.array([[_logit(v) for v in case["logits"]]])
    b = np.array(case["bias"])
    wrong = O.select_topk(O.sigmoid(L + b), 2)
    assert wrong[0].tolist() != case["idx"]


# --------------------------------------------------------------------------
# top-k: brute force over all subsets

def _brute_topk(key_row, k):
    """All k-subsets where every chosen key beats every unchosen one (greater,
    or equal with a lower index)."""
    E = key_row.size
    good = []
    for sub in itertools.combinations(range(E), k):
        chosen = set(sub)
        ok = True
        for a in chosen:
            for c in range(E):
                if c in chosen:
                    continue
                if not (key_row[a] > key_row[c] or (key_row[a] == key_row[c] and a < c)):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            good.append(sub)
    return good


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (8, 3), (12, 4), (6, 6)])
def test_topk_bruteforce(E, k):
    rng = np.random.default_rng(E * 100 + k)
    for trial in range(40):
        if trial % 2:
            keys = rng.choice(np.array([0.1, 0.5, 0.5, 0.9, 1.0]), size=(1, E))  # many exact ties
        else:
            keys = rng.random((1, E))
        idx = O.select_topk(keys, k)[0]
        subs = _brute_topk(keys[0], k)
        assert len(subs) == 1
        assert sorted(idx.tolist()) == list(subs[0])
        # emitted in the total order: key desc, then index asc
        for a, c in zip(idx[:-1], idx[1:]):
            assert keys[0, a] > keys[0, c] or (keys[0, a] == keys[0, c] and a < c)


# --------------------------------------------------------------------------
# bias and norm invariants

def _rand_route_inputs(T=300, E=16, seed=3):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)) * 2.0
    b = rng.uniform(-0.3, 0.3, E)
    return L, b


def test_weights_come_from_unbiased_scores():
    L, b = _rand_route_inputs()
    s, keys, idx, w = O.route(L, b, 4, "sigmoid", True, 2.5)
    g = np.take_along_axis(O.sigmoid(L), idx.astype(np.int64), 1)
    assert np.array_equal(w, g / g.sum(1, keepdims=True) * 2.5)


def test_bias_shift_invariance():
    L, b = _rand_route_inputs()
    _, _, i1, w1 = O.route(L, b, 4, "sigmoid", True, 1.7)
    _, _, i2, w2 = O.route(L, b + 0.25, 4, "sigmoid", True, 1.7)  # exact in fp64 here
    keep = np.all(i1 == i2, axis=1)
    assert keep.mean() > 0.95
    assert np.array_equal(w1[keep], w2[keep])


def test_bias_changes_selection_never_weights():
    L, b = _rand_route_inputs()
    _, _, ib, wb = O.route(L, b, 4, "sigmoid", True, 1.0)
    _, _, i0, w0 = O.route(L, None, 4, "sigmoid", True, 1.0)
    same = np.all(ib == i0, axis=1)
    assert 0 < same.sum() < same.size      # the bias does change some selections
    assert np.array_equal(wb[same], w0[same])


@pytest.mark.parametrize("k,scale", [(1, 2.826), (3, 1.0), (6, 2.0), (8, 2.826)])
def test_norm_sums_to_route_scale(k, scale):
    L, b = _rand_route_inputs(E=16)
    _, _, _, w = O.route(L, b, k, "sigmoid", True, scale)
    assert np.max(np.abs(w.sum(1) - scale)) <= 4 * ULP1 * k * scale
    if k == 1:
        assert np.all(w == scale)


def test_norm_off_gives_scaled_scores():
    L, b = _rand_route_inputs()
    s, _, idx, w = O.route(L, b, 3, "sigmoid", False, 2.0)
    assert np.array_equal(w, 2.0 * np.take_along_axis(s, idx.astype(np.int64), 1))


# --------------------------------------------------------------------------
# activations: closed-form points

def test_activation_points():
    g = _gold("activation_points.json")
    for p in g["swigluoai"]:
        v = O.act_swigluoai(np.float64(p["g"]), np.float64(p["u"]), g["alpha"], g["limit"], g["beta"])
        assert abs(v - p["value"]) <= 1e-13 * max(1.0, abs(p["value"])), p
    for p in g["silu"]:
        v = O.act_silu(np.float64(p["g"]), np.float64(p["u"]))
        assert abs(v - p["value"]) <= 1e-15, p


# --------------------------------------------------------------------------
# permutation

def test_permute_properties():
    rng = np.random.default_rng(5)
    T, E, k = 97, 11, 3
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[:, :] = np.where(rng.random((T, k)) < 0.0, 0, idx)
    counts, offsets, sr, rp = O.permute(idx, E)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(sr), np.arange(T * k))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = sr[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)        # stable: ascending row order
    assert np.array_equal(rp[sr], np.arange(T * k))


# --------------------------------------------------------------------------
# degenerate layers

def _tiny_cfg(**kw):
    c = dict(hidden_size=8, num_experts=3, num_experts_per_tok=2,
             moe_intermediate_size=4, num_shared_experts=1,
             shared_intermediate_size=4, shared_packed=0, score_func="sigmoid",
             route_norm=1, route_scale=1.0, hidden_act="silu", act_alpha=1.702,
             act_limit=7.0, act_beta=1.0, dtype="f32")
    c.update(kw)
    return c


def _tiny_inputs(cfg, T=5, seed=11):
    rng = np.random.default_rng(seed)
    H, E, I = cfg["hidden_size"], cfg["num_experts"], cfg["moe_intermediate_size"]
    S, Is = cfg["num_shared_experts"], cfg["shared_intermediate_size"]
    Et = E + (1 if cfg["shared_packed"] else 0)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    inp = synth.MoeInputs(cfg=cfg, x=f(T, H), w_router=f(E, H) * np.float32(0.5),
                          expert_bias=(rng.uniform(-0.2, 0.2, E)).astype(np.float32),
                          w_gate=f(Et, I, H) * np.float32(0.3), w_up=f(Et, I, H) * np.float32(0.3),
                          w_down=f(Et, H, I) * np.float32(0.3))
    if S and not cfg["shared_packed"]:
        inp.ws_gate, inp.ws_up, inp.ws_down = (f(S, Is, H) * np.float32(0.3),
                                               f(S, Is, H) * np.float32(0.3),
                                               f(S, H, Is) * np.float32(0.3))
    return inp


def _loop_swiglu_mlp(x, wg, wu, wd, act):
    """Textbook SwiGLU MLP with explicit loops over the [out, in] layout."""
    I, H = wg.shape
    y = np.zeros(H)
    hid = np.zeros(I)
    for i in range(I):
        gs = 0.0
        us = 0.0
        for h in range(H):
            gs += float(wg[i, h]) * float(x[h])
            us += float(wu[i, h]) * float(x[h])
        hid[i] = act(gs, us)
    for o in range(H):
        acc = 0.0
        for i in range(I):
            acc += float(wd[o, i]) * hid[i]
        y[o] = acc
    return y


def _py_silu(g, u):
    return g / (1.0 + math.exp(-g)) * u


def test_single_expert_is_scaled_mlp():
    cfg = _tiny_cfg(num_experts=1, num_experts_per_tok=1, num_shared_experts=0,
                    route_scale=2.826)
    inp = _tiny_inputs(cfg)
    res = O.moe_forward(inp, cfg)
    for t in range(inp.x.shape[0]):
        ref = 2.826 * _loop_swiglu_mlp(inp.x[t], inp.w_gate[0], inp.w_up[0], inp.w_down[0], _py_silu)
        assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


def test_all_experts_unnormalised_is_dense_mixture():
    cfg = _tiny_cfg(num_experts_per_tok=3, route_norm=0)
    inp = _tiny_inputs(cfg)
    inp.expert_bias[:] = 0
    res = O.moe_forward(inp, cfg)
    for t in range(inp.x.shape[0]):
        ref = _loop_swiglu_mlp(inp.x[t], inp.ws_gate[0], inp.ws_up[0], inp.ws_down[0], _py_silu)
        for e in range(3):
            logit = sum(float(inp.x[t, h]) * float(inp.w_router[e, h]) for h in range(8))
            ref = ref + (1.0 / (1.0 + math.exp(-logit))) * _loop_swiglu_mlp(
                inp.x[t], inp.w_gate[e], inp.w_up[e], inp.w_down[e], _py_silu)
        assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


def test_packed_shared_equals_separate():
    cfg_p = _tiny_cfg(shared_packed=1, route_scale=2.0, hidden_act="swigluoai")
    inp_p = _tiny_inputs(cfg_p)
    cfg_s = dict(cfg_p, shared_packed=0)
    E = cfg_p["num_experts"]
    inp_s = synth.MoeInputs(cfg=cfg_s, x=inp_p.x, w_router=inp_p.w_router,
                            expert_bias=inp_p.expert_bias,
                            w_gate=inp_p.w_gate[:E], w_up=inp_p.w_up[:E], w_down=inp_p.w_down[:E],
                            ws_gate=inp_p.w_gate[E:], ws_up=inp_p.w_up[E:], ws_down=inp_p.w_down[E:])
    a = O.moe_forward(inp_p, cfg_p)
    b = O.moe_forward(inp_s, cfg_s)
    assert np.array_equal(a["idx"], b["idx"]) and np.all(a["idx"] < E)
    assert np.allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)


def test_two_shared_equal_one_concatenated():
    cfg2 = _tiny_cfg(num_shared_experts=2)
    inp2 = _tiny_inputs(cfg2)
    cfg1 = dict(cfg2, num_shared_experts=1, shared_intermediate_size=8)
    inp1 = synth.MoeInputs(cfg=cfg1, x=inp2.x, w_router=inp2.w_router,
                           expert_bias=inp2.expert_bias, w_gate=inp2.w_gate,
                           w_up=inp2.w_up, w_down=inp2.w_down,
                           ws_gate=inp2.ws_gate.reshape(1, 8, 8),
                           ws_up=inp2.ws_up.reshape(1, 8, 8),
                           ws_down=np.concatenate([inp2.ws_down[0], inp2.ws_down[1]], axis=1)[None])
    a = O.moe_forward(inp2, cfg2)
    b = O.moe_forward(inp1, cfg1)
    assert np.allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)


def test_tokens_subset_matches_full():
    cfg = _tiny_cfg(num_experts=6, num_experts_per_tok=2, hidden_act="swigluoai")
    inp = _tiny_inputs(cfg, T=9)
    full = O.moe_forward(inp, cfg, want_hidden=True)
    sub = O.moe_forward_tokens(inp, cfg, [0, 4, 8])
    assert np.array_equal(sub["idx"], full["idx"][[0, 4, 8]])
    assert np.allclose(sub["out"], full["out"][[0, 4, 8]], rtol=1e-13, atol=1e-13)


def test_loop_layer_matches_vectorised():
    """Whole tiny layer through explicit per-token loops."""
    cfg = _tiny_cfg(num_experts=5, num_experts_per_tok=2, route_scale=1.5)
    inp = _tiny_inputs(cfg, T=6)
    res = O.moe_forward(inp, cfg)
    for t in range(6):
        logits = [sum(float(inp.x[t, h]) * float(inp.w_router[e, h]) for h in range(8)) for e in range(5)]
        s = [1.0 / (1.0 + math.exp(-v)) for v in logits]
        key = [s[e] + float(inp.expert_bias[e]) for e in range(5)]
        chosen = sorted(range(5), key=lambda e: (-key[e], e))[:2]
        den = sum(s[e] for e in chosen)
        y = _loop_swiglu_mlp(inp.x[t], inp.ws_gate[0], inp.ws_up[0], inp.ws_down[0], _py_silu)
        for e in chosen:
            y = y + 1.5 * s[e] / den * _loop_swiglu_mlp(inp.x[t], inp.w_gate[e], inp.w_up[e], inp.w_down[e], _py_silu)
        assert res["idx"][t].tolist() == chosen
        assert np.allclose(res["out"][t], y, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# the workload table agrees with the values the pages print

def test_workloads_use_page_constants():
    pc = _gold("page_constants.json")
    c2 = synth.CONFIGS["afmoe_default_T4096"]
    d = pc["afmoe_defaults"]
    for key in ("hidden_size", "moe_intermediate_size", "num_experts",
                "num_experts_per_tok", "num_shared_experts", "route_scale", "hidden_act"):
        assert c2[key] == d[key], key
    assert c2["w_std"] == d["initializer_range"]
    c3 = synth.CONFIGS["trinity_nano_prefill_T8192"]
    for key in ("hidden_size", "num_experts", "route_scale", "score_func"):
        assert c3[key] == pc["trinity"][key], key
    c5 = synth.CONFIGS["minimax_m3_prefill_T8192"]
    m3 = pc["minimax_m3"]
    assert (c5["hidden_size"], c5["num_experts"], c5["num_experts_per_tok"]) == (
        m3["hidden_size"], m3["num_experts"], m3["num_experts_per_tok"])
    assert c5["route_scale"] == m3["routed_scaling_factor"]
    assert c5["shared_intermediate_size"] == m3["shared_intermediate_size"]
    assert c5["shared_packed"] == 1 and c5["num_experts"] == m3["shared_slot"]
    assert (c5["act_alpha"], c5["act_limit"], c5["act_beta"]) == (m3["alpha"], m3["limit"], m3["beta"])
    assert c2["rms_norm_eps"] == d["rms_norm_eps"]
    assert c5["norm_add_one"] == 1 and c2["norm_add_one"] == 0


# --------------------------------------------------------------------------
# RMSNorm and the block around the layer (mlxcel #845 "What the original body
# missed": out = h + post_mlp_norm(mlp(pre_mlp_norm(h))); mlxcel #763 Norms
# bullet: Gemma-style w + 1)

def test_rms_norm_hand_example():
    for c in _gold("rms_norm_hand_example.json")["cases"]:
        y = O.rms_norm(np.array([c["x"]]), np.array(c["w"]), c["eps"], bool(c["add_one"]))[0]
        assert np.allclose(y, c["y"], rtol=4 * ULP1, atol=0), c["why"]


def test_rms_norm_rows_by_loops():
    """Each row is normalised on its own, over the hidden axis: explicit
    per-element loops on rows of very different scales."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 9)) * np.array([1e-3, 1.0, 7.0, 1e3, 0.5, 40.0])[:, None]
    w = rng.standard_normal(9)
    for add_one in (False, True):
        y = O.rms_norm(x, w, 1e-5, add_one)
        for t in range(6):
            ms = sum(float(v) * float(v) for v in x[t]) / 9
            r = 1.0 / math.sqrt(ms + 1e-5)
            for i in range(9):
                ref = float(x[t, i]) * r * (float(w[i]) + (1.0 if add_one else 0.0))
                assert abs(y[t, i] - ref) <= 8 * ULP1 * max(1.0, abs(ref))


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 64)) * np.array([1e-2, 1.0, 3.0, 1e4])[:, None]
    ones = np.ones(64)
    y = O.rms_norm(x, ones, 0.0, False)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=8 * ULP1)
    for a in (0.25, 3.0, 1e3):
        assert np.allclose(O.rms_norm(a * x, ones, 0.0, False), y, rtol=8 * ULP1, atol=0)
    assert np.array_equal(O.rms_norm(-x, ones, 0.0, False), -y)
    # eps dominates a tiny row: y -> x / sqrt(eps)
    tiny = np.full((1, 8), 1e-9)
    assert np.allclose(O.rms_norm(tiny, np.ones(8), 1.0, False), tiny, rtol=1e-12, atol=0)


def _block_inputs(cfg, T=5, seed=11):
    inp = _tiny_inputs(cfg, T=T, seed=seed)
    rng = np.random.default_rng(seed + 100)
    H = cfg["hidden_size"]
    return inp, rng.uniform(0.5, 1.5, H), rng.uniform(0.5, 1.5, H)


def test_block_zero_expert_outputs_give_the_residual():
    """With every down projection zero the layer output is zero, its RMSNorm
    (eps > 0) is zero, and the block returns its input unchanged."""
    cfg = _tiny_cfg()
    inp, pre, post = _block_inputs(cfg)
    inp.w_down[:] = 0
    inp.ws_down[:] = 0
    res = O.block_forward(inp, cfg, pre, post, 1e-5, False)
    assert np.array_equal(res["out"], O.as_f64(inp.x))


def test_block_branch_has_the_post_norm_scale():
    """eps = 0 and a unit post-norm weight: every row of out - h has RMS 1;
    with post weight w the row RMS of (out - h) / w is 1."""
    cfg = _tiny_cfg(hidden_act="swigluoai")
    inp, pre, post = _block_inputs(cfg, T=7)
    for w, add_one in ((np.ones(8), False), (post, False), (post - 1.0, True)):
        res = O.block_forward(inp, cfg, pre, w, 0.0, add_one)
        scale = w + (1.0 if add_one else 0.0)
        br = (res["out"] - O.as_f64(inp.x)) / scale
        assert np.allclose(np.sqrt(np.mean(br * br, axis=-1)), 1.0, rtol=0, atol=1e-12)


def test_block_ignores_the_input_scale():
    """eps = 0: the pre-norm removes a positive scale of h, so routing and
    out - h are unchanged while the residual scales."""
    cfg = _tiny_cfg(num_experts=5, num_experts_per_tok=2)
    inp, pre, post = _block_inputs(cfg, T=6)
    a = O.block_forward(inp, cfg, pre, post, 0.0, False)
    big = synth.MoeInputs(**{**inp.__dict__, "x": (inp.x * np.float32(16.0)).astype(np.float32)})
    b = O.block_forward(big, cfg, pre, post, 0.0, False)
    assert np.array_equal(a["idx"], b["idx"])
    da = a["out"] - O.as_f64(inp.x)
    db = b["out"] - O.as_f64(big.x)
    assert np.allclose(da, db, rtol=1e-12, atol=1e-12)


def test_block_by_loops():
    """The whole block through explicit per-token loops: pre-norm, router,
    selection, experts, post-norm, residual (Gemma-style and plain scales)."""
    cfg = _tiny_cfg(num_experts=5, num_experts_per_tok=2, route_scale=1.5)
    inp, pre, post = _block_inputs(cfg, T=4)
    for add_one in (False, True):
        res = O.block_forward(inp, cfg, pre, post, 1e-5, add_one)
        off = 1.0 if add_one else 0.0
        for t in range(4):
            h = [float(v) for v in inp.x[t]]
            r = 1.0 / math.sqrt(sum(v * v for v in h) / 8 + 1e-5)
            xn = np.array([h[i] * r * (pre[i] + off) for i in range(8)])
            logits = [sum(xn[i] * float(inp.w_router[e, i]) for i in range(8)) for e in range(5)]
            s = [1.0 / (1.0 + math.exp(-v)) for v in logits]
            key = [s[e] + float(inp.expert_bias[e]) for e in range(5)]
            chosen = sorted(range(5), key=lambda e: (-key[e], e))[:2]
            den = sum(s[e] for e in chosen)
            y = _loop_swiglu_mlp(xn, inp.ws_gate[0], inp.ws_up[0], inp.ws_down[0], _py_silu)
            for e in chosen:
                y = y + 1.5 * s[e] / den * _loop_swiglu_mlp(xn, inp.w_gate[e], inp.w_up[e],
                                                            inp.w_down[e], _py_silu)
            r2 = 1.0 / math.sqrt(sum(float(v) * float(v) for v in y) / 8 + 1e-5)
            ref = [h[i] + float(y[i]) * r2 * (post[i] + off) for i in range(8)]
            assert res["idx"][t].tolist() == chosen
            assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# MXFP8 expert weights (OCP MX v1.0 format; the MXFP8 export of mlxcel #763
# "Validation")

def test_e4m3_hand_values():
    g = _gold("mxfp8_hand_example.json")
    for code, val in g["e4m3"]:
        got = O.e4m3_value(np.array([int(code, 16)], np.uint8))[0]
        assert got == val, code
    for code in g["e4m3_nan"]:
        assert np.isnan(O.e4m3_value(np.array([int(code, 16)], np.uint8))[0])


def test_e4m3_all_codes_match_torch():
    """Every code against an independent decoder (torch's float8_e4m3fn)."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e8m0_hand_values_and_torch():
    g = _gold("mxfp8_hand_example.json")
    for e, val in g["e8m0"]:
        assert O.e8m0_value(np.array([e], np.uint8))[0] == val
    assert np.isnan(O.e8m0_value(np.array([255], np.uint8))[0])
    torch = pytest.importorskip("torch")
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(O.e8m0_value(codes), ref)


def test_mx_dequantize_block_major_scales():
    """Scales are [K/32, N]: a transposed read gives row 1's first block the
    wrong scale and fails here."""
    d = _gold("mxfp8_hand_example.json")["dequant"]
    codes = np.full((2, 64), int(d["codes_fill"], 16), np.uint8)
    for r, k, c in d["codes_set"]:
        codes[r, k] = int(c, 16)
    w = O.mx_dequantize(codes, np.array(d["scales"], np.uint8))
    for row in d["rows"]:
        r = row["row"]
        first = np.delete(w[r, :32], [])
        last = w[r, 32:].copy()
        if "at40" in row:
            assert w[r, 40] == row["at40"]
            last = np.delete(last, 8)
        assert np.all(first == row["first32"]) and np.all(last == row["last32"])


def test_mx_layer_runs_on_the_dequantised_values():
    """The layer with stacked MXFP8 experts (lazy per-expert dequantisation,
    packed shared slot included) equals the layer given the dequantised
    matrices as plain float64 tensors."""
    cfg = _tiny_cfg(hidden_size=64, moe_intermediate_size=64, shared_packed=1,
                    hidden_act="swigluoai", route_scale=2.0)
    rng = np.random.default_rng(4)
    T, H, E, I = 6, 64, 3, 64
    codes = {k: rng.integers(0, 256, (E + 1, n, kk), dtype=np.uint8)
             for k, (n, kk) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))}
    for c in codes.values():
        c[(c & 0x7F) == 0x7F] = 0x38               # no NaN codes
    scales = {k: rng.integers(118, 124, (E + 1, c.shape[2] // 32, c.shape[1]), dtype=np.uint8)
              for k, c in codes.items()}
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    b = np.zeros(E, np.float32)
    mx = synth.MoeInputs(cfg=cfg, x=x, w_router=wr, expert_bias=b,
                         w_gate=O.MxStacked(codes["gate"], scales["gate"]),
                         w_up=O.MxStacked(codes["up"], scales["up"]),
                         w_down=O.MxStacked(codes["down"], scales["down"]))
    dense = synth.MoeInputs(cfg=cfg, x=x, w_router=wr, expert_bias=b,
                            w_gate=np.stack([mx.w_gate[e] for e in range(E + 1)]),
                            w_up=np.stack([mx.w_up[e] for e in range(E + 1)]),
                            w_down=np.stack([mx.w_down[e] for e in range(E + 1)]))
    a, d = O.moe_forward(mx, cfg), O.moe_forward(dense, cfg)
    assert np.array_equal(a["idx"], d["idx"]) and np.array_equal(a["out"], d["out"])


# --------------------------------------------------------------------------
# MXFP4 expert weights (OCP MX v1.0 E2M1; the 4-bit Trinity checkpoints of
# mlxcel #845 "Checkpoint confirmed")

def test_e2m1_hand_values():
    g = _gold("mxfp4_hand_example.json")
    for code, val in g["e2m1"]:
        got = O.e2m1_value(np.array([int(code, 16)], np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), code
    # only the low nibble is a code
    assert O.e2m1_value(np.array([0xF7], np.uint8))[0] == 6.0


def test_e2m1_values_are_exact_in_e4m3():
    """Every E2M1 value is an E4M3 value (both OCP minifloats): decoding the
    E4M3 code with the same sign, exponent (rebiased 1 -> 7) and mantissa
    (shifted into the top bit) gives the same number for the normal codes."""
    for c in range(16):
        ef, m, sgn = (c >> 1) & 3, c & 1, c >> 3
        if ef == 0:
            continue
        e4 = (sgn << 7) | ((ef - 1 + 7) << 3) | (m << 2)
        assert O.e2m1_value(np.array([c], np.uint8))[0] == O.e4m3_value(np.array([e4], np.uint8))[0]


def test_mxfp4_dequantize_nibble_order_and_block_major_scales():
    d = _gold("mxfp4_hand_example.json")["dequant"]
    packed = np.full((2, 32), int(d["bytes_fill"], 16), np.uint8)
    for r, j, c in d["bytes_set"]:
        packed[r, j] = int(c, 16)
    w = O.mx_dequantize(packed, np.array(d["scales"], np.uint8), "e2m1")
    assert w.shape == (2, 64)
    for row in d["rows"]:
        r = row["row"]
        expect = np.concatenate([np.full(32, row["first32"]), np.full(32, row["last32"])])
        for k, v in row.get("at", []):
            expect[k] = v
        assert np.array_equal(w[r], expect), r


def test_mxfp4_stacked_layer_equals_dense():
    """The layer with stacked MXFP4 experts (two inputs per byte, lazy
    per-expert dequantisation, packed shared slot included) equals the layer
    given the dequantised matrices as plain float64 tensors."""
    cfg = _tiny_cfg(hidden_size=64, moe_intermediate_size=64, shared_packed=1,
                    hidden_act="swigluoai", route_scale=2.0)
    rng = np.random.default_rng(5)
    T, H, E, I = 6, 64, 3, 64
    codes = {k: rng.integers(0, 256, (E + 1, n, kk // 2), dtype=np.uint8)
             for k, (n, kk) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))}
    scales = {k: rng.integers(122, 128, (E + 1, 2 * c.shape[2] // 32, c.shape[1]), dtype=np.uint8)
              for k, c in codes.items()}
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    b = np.zeros(E, np.float32)
    st = {k: O.MxStacked(codes[k], scales[k], "e2m1") for k in codes}
    assert st["gate"].shape == (E + 1, I, H) and st["down"].shape == (E + 1, H, I)
    mx = synth.MoeInputs(cfg=cfg, x=x, w_router=wr, expert_bias=b,
                         w_gate=st["gate"], w_up=st["up"], w_down=st["down"])
    dense = synth.MoeInputs(cfg=cfg, x=x, w_router=wr, expert_bias=b,
                            w_gate=np.stack([st["gate"][e] for e in range(E + 1)]),
                            w_up=np.stack([st["up"][e] for e in range(E + 1)]),
                            w_down=np.stack([st["down"][e] for e in range(E + 1)]))
    a, d = O.moe_forward(mx, cfg), O.moe_forward(dense, cfg)
    assert np.array_equal(a["idx"], d["idx"]) and np.array_equal(a["out"], d["out"])
    # element (n, k) of expert e by hand from its byte and scale
    e, n, k = 2, 5, 37
    byte = int(codes["gate"][e, n, k // 2])
    nib = byte & 0xF if k % 2 == 0 else byte >> 4
    val = O.e2m1_value(np.array([nib], np.uint8))[0] * 2.0 ** (int(scales["gate"][e, k // 32, n]) - 127)
    assert st["gate"][e][n, k] == val


# --------------------------------------------------------------------------
# group-limited routing (mlxcel #845 "Routing detail": group routing, n_group;
# the rule read from the DeepSeek MoE family the page derives AFMoE from)

def test_route_group_hand_example():
    for c in _gold("route_group_hand_example.json")["cases"]:
        L = np.array([[_logit(v) for v in c["logits"]]])
        _, keys, idx, w = O.route(L, np.array(c["bias"], dtype=np.float32), c["k"], "sigmoid",
                                  bool(c["route_norm"]), c["route_scale"], c["n_group"],
                                  c["topk_group"])
        assert idx[0].tolist() == c["idx"], c["why"]
        assert np.allclose(w[0], c["w"], rtol=1e-12, atol=0), c["why"]
        kept = sorted({int(e) // 2 for e in np.nonzero(np.isfinite(keys[0]))[0]})
        assert kept == c["kept_groups"], c["why"]


def _brute_group_route(key_row, n_group, topk_group, k):
    """The rule by enumeration: the set of kept groups is the topk_group-subset
    of groups ranked first by (score desc, index asc); top-k inside it by
    (key desc, index asc)."""
    E = key_row.size
    gs = E // n_group
    gscore = []
    for g in range(n_group):
        vals = sorted((float(v) for v in key_row[g * gs:(g + 1) * gs]), reverse=True)
        gscore.append(vals[0] + vals[1])
    ranked = sorted(range(n_group), key=lambda g: (-gscore[g], g))
    kept = set(ranked[:topk_group])
    cand = [e for e in range(E) if e // gs in kept]
    return sorted(cand, key=lambda e: (-float(key_row[e]), e))[:k]


@pytest.mark.parametrize("E,n_group,topk_group,k", [(8, 4, 2, 3), (12, 3, 1, 2), (16, 4, 3, 5),
                                                    (256, 8, 4, 8), (10, 5, 5, 4)])
def test_route_group_bruteforce(E, n_group, topk_group, k):
    rng = np.random.default_rng(E + k)
    L = rng.standard_normal((40, E))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    L[3, :] = 0.0                             # every key equal: ties everywhere
    L[5, : E // 2] = L[5, E // 2:]            # mirrored halves: tied groups
    _, keys, idx, w = O.route(L, bias, k, "sigmoid", True, 1.0, n_group, topk_group)
    s = O.sigmoid(L)
    raw = s + bias.astype(np.float64)[None, :]
    for t in range(L.shape[0]):
        assert idx[t].tolist() == _brute_group_route(raw[t], n_group, topk_group, k), t
        assert len({int(e) // (E // n_group) for e in idx[t]}) <= topk_group
    # weights are still the unbiased scores of the chosen experts, normalised
    g = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    assert np.allclose(w, g / g.sum(1, keepdims=True), rtol=1e-14, atol=0)


def test_route_all_groups_kept_is_plain_topk():
    rng = np.random.default_rng(9)
    L = rng.standard_normal((30, 32))
    bias = rng.uniform(-0.05, 0.05, 32).astype(np.float32)
    a = O.route(L, bias, 6, "softmax", True, 2.0)
    b = O.route(L, bias, 6, "softmax", True, 2.0, n_group=8, topk_group=8)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])



# --------------------------------------------------------------------------
# storage decoding and the routing report's boundary gap

def _hand_value(s):
    """A hand-written exact value: "1", "-0", "inf", "2^-133", "127*2^-133"."""
    if s in ("inf", "-inf"):
        return float(s)
    sign = -1.0 if s.startswith("-") else 1.0
    s = s.lstrip("-")
    mult = 1.0
    if "*" in s:
        m, s = s.split("*")
        mult = float(int(m))
    if s.startswith("2^"):
        return sign * mult * math.ldexp(1.0, int(s[2:]))
    return sign * mult * float(s)


def test_as_f64_bf16_bits_hand_values():
    """bf16 bit patterns through the oracle's storage decoder, against values
    worked by hand from the format (the path every bf16 workload value takes
    into the oracle)."""
    g = _gold("bf16_hand_example.json")
    bits = np.array([int(b, 16) for b, _ in g["values"]], dtype=np.uint16)
    want = np.array([_hand_value(v) for _, v in g["values"]], dtype=np.float64)
    got = O.as_f64(bits)
    assert got.dtype == np.float64
    assert np.array_equal(got, want)
    # the sign of zero is kept (0x8000 is -0)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    nan = O.as_f64(np.array([int(b, 16) for b in g["nan"]], dtype=np.uint16))
    assert np.all(np.isnan(nan))
    # shape is kept; a 2-D array decodes element by element
    two = O.as_f64(bits[:4].reshape(2, 2))
    assert two.shape == (2, 2) and np.array_equal(two.reshape(-1), want[:4])


def test_as_f64_bf16_catches_a_shift_before_widening():
    """A plausible slip, shifting the 16-bit array before widening it, loses
    every bit: the hand values reject it (planted on the CPU, in a copy)."""
    g = _gold("bf16_hand_example.json")
    bits = np.array([int(b, 16) for b, _ in g["values"]], dtype=np.uint16)
    want = np.array([_hand_value(v) for _, v in g["values"]], dtype=np.float64)

    def shifted_first(a):
        return (a << 16).astype(np.uint32).view(np.float32).astype(np.float64)

    def low_half(a):  # the bits placed in the low half of the binary32
        return a.astype(np.uint32).view(np.float32).astype(np.float64)

    for bad in (shifted_first, low_half):
        with np.errstate(all="ignore"):
            assert not np.array_equal(bad(bits), want)


def test_as_f64_other_dtypes():
    """fp32 values widen exactly; MX codes without scales are refused."""
    v = np.array([1.0, -3.5, 2.0 ** -140, 3.4e38], dtype=np.float32)
    assert np.array_equal(O.as_f64(v), v.astype(np.float64))
    with pytest.raises(ValueError):
        O.as_f64(np.zeros(4, np.uint8))


def test_boundary_gap_hand_examples():
    """The smallest k-th minus (k+1)-th key, worked by hand on dyadic keys
    (exact tie -> 0, no boundary -> inf)."""
    for c in _gold("boundary_gap_hand_example.json")["cases"]:
        keys = np.array([[float(v) for v in row] for row in c["keys"]], dtype=np.float64)
        want = float(c["gap"])
        assert O.boundary_gap(keys, c["k"]) == want, c["why"]
