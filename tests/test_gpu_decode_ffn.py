"""GPU parity of the fused decode FFN (bf16 weights, at most 32 tokens and 256
routed rows, hidden 512 or 1024): one kernel runs the gate/up GEMM of a
128-column slice of an expert's intermediate width, keeps the activated
slice in LDS and multiplies it by the matching columns of the down matrix
into fp32 partial planes, which the combine sums per row in slice order
before weighting (the expert FFN down(act(gate x, up x)) of mlxcel #845
"Routing detail" is a sum over the columns of h, so the slices add up to
it).

Every case runs through moe_layer_forward against the float64 oracle fed the
GPU's own router logits: routing exactly, the output at the layer's bf16 bar
(max|err| <= 2e-2 max|ref|). The cases cover one and four slices per expert,
no shared expert, two separate shared experts (one slice each) and a shared
width of three slices, the packed shared slot with clamp-SwiGLU, one token,
256 experts (the kernel's limit), 256 routed rows with every expert full
(k = E), hidden 512 and 1024 (two and four down n-tiles), and MXFP8 and
MXFP4 expert weights (the oracle on their exact values). The same layer
with the fused kernel switched off (MOE_DECODE_FFN=0: separate gate/up and
down kernels) is held to the same bar, and the two differ in rounding only
(the fused path never rounds an expert's output to bf16), which also shows
that the fused kernel ran. Repeats are bitwise equal; the block forward takes
the fused path too."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, generated, rel_err, say
from tests.test_gpu_block import check_block, run_block
from tests.test_gpu_mxfp8 import oracle_view
from tests.test_gpu_parity import check_routing
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


FFN = {
    "no_shared_one_slice_h512": custom(T=32, hidden_size=512, num_experts=16,
                                       num_experts_per_tok=8, moe_intermediate_size=128,
                                       num_shared_experts=0),
    "two_shared_four_slices": custom(T=7, hidden_size=1024, num_experts=32, num_experts_per_tok=4,
                                     moe_intermediate_size=512, num_shared_experts=2,
                                     shared_intermediate_size=128),
    "packed_clamp_h512": custom(T=24, hidden_size=512, num_experts=64, num_experts_per_tok=6,
                                moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                                hidden_act="swigluoai", route_scale=2.0, w_std=0.2,
                                x_scale=20.0),
    "one_token_256_experts": custom(T=1, hidden_size=1024, num_experts=256,
                                    num_experts_per_tok=8, moe_intermediate_size=256,
                                    num_shared_experts=1, shared_intermediate_size=256),
    "k_eq_E_full_tiles": custom(T=32, hidden_size=512, num_experts=8, num_experts_per_tok=8,
                                moe_intermediate_size=128, num_shared_experts=1,
                                shared_intermediate_size=384),
    # MX expert weights (the gate/up and down K-steps of 128 inputs)
    "mxfp8_h512_two_shared": custom(T=7, hidden_size=512, num_experts=32, num_experts_per_tok=4,
                                    moe_intermediate_size=256, num_shared_experts=2,
                                    shared_intermediate_size=128, weight_format="mxfp8"),
    "mxfp4_packed_clamp": custom(T=24, hidden_size=1024, num_experts=64, num_experts_per_tok=6,
                                 moe_intermediate_size=256, num_shared_experts=1,
                                 shared_packed=1, hidden_act="swigluoai", route_scale=2.0,
                                 weight_format="mxfp4"),
    "mxfp8_one_token_i512": custom(T=1, hidden_size=1024, num_experts=128,
                                   num_experts_per_tok=8, moe_intermediate_size=512,
                                   num_shared_experts=1, shared_intermediate_size=256,
                                   weight_format="mxfp8"),
}


def _layer(dev, det, monkeypatch, fused):
    if fused:
        monkeypatch.delenv("MOE_DECODE_FFN", raising=False)
    else:
        monkeypatch.setenv("MOE_DECODE_FFN", "0")
    return dev.forward(deterministic=det)


def _check(cfg, inp, res):
    check_routing(cfg, inp, res)
    ref = O.moe_forward(oracle_view(inp), cfg, logits=res["logits"])
    e = rel_err(res["out"], ref["out"])
    assert e <= TOL["bf16"], f"out rel err {e:.3e}"
    return e


@pytest.mark.parametrize("name", list(FFN) + ["trinity_nano_decode_T32",
                                              "trinity_nano_decode_T32_mxfp4",
                                              "trinity_nano_decode_T32_mxfp8"])
def test_fused_ffn_matches_oracle(name, monkeypatch):
    inp = generated(name) if name in synth.CONFIGS else synth.generate(FFN[name])
    cfg = inp.cfg
    dev = Dev(inp)
    fused = _layer(dev, 1, monkeypatch, True)
    ef = _check(cfg, inp, fused)
    again = _layer(dev, 0, monkeypatch, True)
    assert np.array_equal(again["out"], fused["out"]), "fused path not bitwise repeatable"
    split = _layer(dev, 1, monkeypatch, False)
    es = _check(cfg, inp, split)
    assert np.array_equal(split["idx"], fused["idx"])
    assert not np.array_equal(split["out"], fused["out"]), "the fused kernel did not run"
    assert rel_err(fused["out"], split["out"]) <= TOL["bf16"]
    say(f"[ffn] {name} fused {ef:.2e} split {es:.2e}")


@pytest.mark.parametrize("grid,name", [(1, "few_items"), (3, "few_items"), (3, "many_items"),
                                       (5, "many_items"), (3, "many_items_mxfp4")])
def test_fused_ffn_small_grids(grid, name, monkeypatch):
    """Fewer workgroups than work items (MOE_FFN_GRID caps the grid): the
    items beyond the grid go to the workgroups whose own item is not real,
    then round-robin, so workgroups run several items in a row and some
    start on a handed-over item instead of their own."""
    cfg = {"few_items": custom(T=6, hidden_size=512, num_experts=4, num_experts_per_tok=2,
                               moe_intermediate_size=128, num_shared_experts=1,
                               shared_intermediate_size=128),
           "many_items": custom(T=9, hidden_size=1024, num_experts=16, num_experts_per_tok=2,
                                moe_intermediate_size=128, num_shared_experts=2,
                                shared_intermediate_size=128),
           "many_items_mxfp4": custom(T=9, hidden_size=1024, num_experts=16,
                                      num_experts_per_tok=2, moe_intermediate_size=128,
                                      num_shared_experts=2, shared_intermediate_size=128,
                                      weight_format="mxfp4")}[name]
    inp = synth.generate(cfg)
    dev = Dev(inp)
    monkeypatch.setenv("MOE_FFN_GRID", str(grid))
    res = _layer(dev, 1, monkeypatch, True)
    e = _check(cfg, inp, res)
    monkeypatch.delenv("MOE_FFN_GRID")
    full = _layer(dev, 1, monkeypatch, True)
    assert np.array_equal(full["out"], res["out"]), "the schedule changed the result"
    say(f"[ffn] grid {grid} {name} out {e:.2e} experts chosen {len(np.unique(res['idx']))}")


def test_fused_ffn_batch_sizes_on_one_workspace(monkeypatch):
    """One workspace sized for 300 tokens (which take the separate kernels)
    serves every fused batch size after it, with nothing carried over: each
    output against the oracle, and T = 32 bitwise equal when it comes round
    again."""
    monkeypatch.delenv("MOE_DECODE_FFN", raising=False)
    cfg = custom(T=300, hidden_size=1024, num_experts=64, num_experts_per_tok=8,
                 moe_intermediate_size=256, num_shared_experts=1, route_scale=2.826)
    full = synth.generate(cfg)
    dev = Dev(full)
    first = None
    for T in (32, 300, 5, 17, 1, 32):
        sub = synth.MoeInputs(cfg=dict(cfg, T=T), x=full.x[:T], w_router=full.w_router,
                              expert_bias=full.expert_bias, w_gate=full.w_gate, w_up=full.w_up,
                              w_down=full.w_down, ws_gate=full.ws_gate, ws_up=full.ws_up,
                              ws_down=full.ws_down)
        d = Dev.__new__(Dev)
        d.__dict__.update(dev.__dict__)
        d.inp, d.cfg, d.T = sub, sub.cfg, T
        d.x = dev.x[: T * cfg["hidden_size"]] if dev.x.dim() == 1 else dev.x[:T]
        res = d.forward(deterministic=1)
        e = _check(sub.cfg, sub, res)
        say(f"[ffn] interleaved T={T} out {e:.2e}")
        if T == 32:
            if first is None:
                first = res["out"]
            else:
                assert np.array_equal(first, res["out"])


def test_fused_ffn_inside_the_block(monkeypatch):
    monkeypatch.delenv("MOE_DECODE_FFN", raising=False)
    cfg = custom(T=32, hidden_size=1024, num_experts=64, num_experts_per_tok=8,
                 moe_intermediate_size=256, num_shared_experts=1, shared_intermediate_size=256,
                 route_scale=2.826)
    inp = synth.generate(cfg)
    nw = synth.norm_weights(cfg)
    dev = Dev(inp)
    res = run_block(dev, nw, 1)
    worst = check_block(cfg, inp, nw, res)
    monkeypatch.setenv("MOE_DECODE_FFN", "0")
    split = run_block(dev, nw, 1)
    check_block(cfg, inp, nw, split)
    assert not np.array_equal(split["out"], res["out"]), "the fused kernel did not run"
    say(f"[ffn] block worst err/bound {worst:.3f}")


@pytest.mark.parametrize("name", ["trinity_nano_decode_T32", "two_shared_four_slices",
                                  "packed_clamp_h512", "trinity_nano_decode_T32_mxfp4",
                                  "mxfp8_h512_two_shared"])
def test_ffn_entry_points(name, monkeypatch):
    """moe_expert_ffn and moe_combine_partials called on their own: every
    partial plane against the oracle's expert FFN restricted to that slice of
    the intermediate width (routed rows and shared rows), and the combined
    output bitwise equal to the layer's."""
    monkeypatch.delenv("MOE_DECODE_FFN", raising=False)
    inp = generated(name) if name in synth.CONFIGS else synth.generate(FFN[name])
    cfg, c = inp.cfg, synth.layer_keys(inp.cfg)
    dev = Dev(inp)
    layer = dev.forward(deterministic=1)
    T, k, H = dev.T, cfg["num_experts_per_tok"], cfg["hidden_size"]
    I, S = cfg["moe_intermediate_size"], cfg["num_shared_experts"]
    Is = cfg["shared_intermediate_size"] or I
    idx = torch.from_numpy(layer["idx"].astype(np.int32)).cuda().reshape(-1)
    w = torch.from_numpy(layer["w"].astype(np.float32)).cuda().reshape(-1)
    n = moe.moe_expert_ffn_size(c, T)
    nr, ns = I // 128, S * Is // 128
    assert n == (nr * T * k + ns * T) * H * 4
    parts = torch.full((n // 4,), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(c, T, dev.x, dev.w_gate, dev.w_up, dev.w_down, dev.ws_gate, dev.ws_up,
                       dev.ws_down, idx, parts, mx=dev.mx)
    out = torch.empty(T * H, dtype=moe.torch_dtype(c), device="cuda")
    moe.moe_combine_partials(c, T, parts, w, out)
    torch.cuda.synchronize()
    got = out.view(T, H).float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, layer["out"]), "entry points differ from the layer"

    P = parts.cpu().numpy().astype(np.float64)
    routed = P[: nr * T * k * H].reshape(nr, T * k, H)
    shared = P[nr * T * k * H:].reshape(ns, T, H) if ns else None
    ov = oracle_view(inp)   # MX weights as their exact values
    x = O.as_f64(inp.x)
    act = O.activation(cfg)
    worst = 0.0
    for cs in range(nr):
        C = slice(128 * cs, 128 * cs + 128)
        ref = np.zeros((T * k, H))
        for r in range(T * k):
            e = int(layer["idx"].reshape(-1)[r])
            he = O.mlp_hidden(x[r // k][None], O.as_f64(ov.w_gate[e][C]), O.as_f64(ov.w_up[e][C]),
                              act)
            ref[r] = O.mlp_out(he, O.as_f64(ov.w_down[e][:, C]))[0]
        e_c = rel_err(routed[cs], ref)
        assert e_c <= TOL["bf16"], f"routed plane {cs}: {e_c:.3e}"
        worst = max(worst, e_c)
    sw = O._shared_weights(ov, cfg)
    for a in range(ns):
        s, off = divmod(128 * a, Is)
        wg, wu, wd = sw[s]
        C = slice(off, off + 128)
        ref = O.mlp_out(O.mlp_hidden(x, wg[C], wu[C], act), wd[:, C])
        e_a = rel_err(shared[a], ref)
        assert e_a <= TOL["bf16"], f"shared plane {a}: {e_a:.3e}"
        worst = max(worst, e_a)
    say(f"[ffn] entry points {name}: planes worst {worst:.2e}")
