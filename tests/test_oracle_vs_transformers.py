"""An independent pin of the oracle's AFMoE layer: the MoE block of the
Hugging Face Transformers AFMoE model (AfmoeSparseMoeBlock: token-choice
router with sigmoid scores, a selection-only expert bias, normalisation and
route_scale; stacked experts; the shared experts as one MLP of width
moe_intermediate_size x num_shared_experts), run on the CPU in float64 on
the same weights (HF Transformers doc "AFMoE": expert routing, shared
experts, AfmoeConfig).

That module casts the router logits to fp32 before the sigmoid, so its
scores and routing weights carry fp32 rounding; the oracle is given the same
fp32-rounded logits. The selected experts then agree exactly (tie-free
inputs), and the outputs to the fp32 rounding of the weights (relative
1e-6), far inside anything a plausible oracle slip (bias on the logits, a
missing route_scale, scale before the norm, a dropped shared expert, gate
and up swapped) would leave: each of those moves the output by more than
1e-2 of its scale."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import synth

torch = pytest.importorskip("torch")
afmoe = pytest.importorskip("transformers.models.afmoe.modeling_afmoe")
cfg_mod = pytest.importorskip("transformers.models.afmoe.configuration_afmoe")


def _case(seed=3):
    cfg = synth._cfg(T=48, hidden_size=64, num_experts=8, num_experts_per_tok=3,
                     moe_intermediate_size=32, num_shared_experts=2, shared_intermediate_size=0,
                     dtype="f32", bias_limit=0.05, route_scale=2.5, router_bf16_values=False,
                     w_std=0.2)
    cfg["name"] = "hf_afmoe_pin"
    cfg["seed"] = seed
    return cfg, synth.generate(cfg)


def _hf_block(cfg, inp):
    c = cfg_mod.AfmoeConfig(hidden_size=cfg["hidden_size"],
                            moe_intermediate_size=cfg["moe_intermediate_size"],
                            num_experts=cfg["num_experts"],
                            num_experts_per_tok=cfg["num_experts_per_tok"],
                            num_shared_experts=cfg["num_shared_experts"],
                            route_scale=cfg["route_scale"], hidden_act="silu",
                            num_hidden_layers=1, num_dense_layers=0, vocab_size=16)
    blk = afmoe.AfmoeSparseMoeBlock(c).to(torch.float64).eval()
    f = lambda a: torch.from_numpy(O.as_f64(a))
    I, S = cfg["moe_intermediate_size"], cfg["num_shared_experts"]
    with torch.no_grad():
        blk.router.gate.weight.copy_(f(inp.w_router))
        blk.expert_bias.copy_(f(inp.expert_bias))
        blk.experts.gate_up_proj.copy_(torch.cat([f(inp.w_gate), f(inp.w_up)], dim=1))
        blk.experts.down_proj.copy_(f(inp.w_down))
        # S shared experts of width I = one MLP of width S*I
        blk.shared_experts.gate_proj.weight.copy_(f(inp.ws_gate).reshape(S * I, -1))
        blk.shared_experts.up_proj.weight.copy_(f(inp.ws_up).reshape(S * I, -1))
        blk.shared_experts.down_proj.weight.copy_(
            torch.cat([f(inp.ws_down[s]) for s in range(S)], dim=1))
    return blk


def test_oracle_matches_transformers_afmoe_block():
    cfg, inp = _case()
    blk = _hf_block(cfg, inp)
    x = torch.from_numpy(O.as_f64(inp.x))
    with torch.no_grad():
        logits, w_hf, idx_hf = blk.router(x[None], blk.expert_bias)
        out_hf = blk(x[None])[0].numpy()
    # the same fp32 router logits on both sides
    L32 = logits.numpy().astype(np.float32)
    ref = O.moe_forward(inp, cfg, logits=L32)
    keys = ref["keys"]
    assert O.boundary_gap(keys, cfg["num_experts_per_tok"]) > 1e-4   # tie-free
    assert np.array_equal(ref["idx"], idx_hf.numpy())
    assert np.max(np.abs(ref["w"] - w_hf.numpy())) <= 1e-6 * cfg["route_scale"]
    scale = np.max(np.abs(ref["out"]))
    err = np.max(np.abs(out_hf - ref["out"])) / scale
    assert err <= 1e-6, err


@pytest.mark.parametrize("slip", ["bias_on_logits", "no_route_scale", "no_shared", "swap_gate_up"])
def test_planted_oracle_slips_are_caught(slip):
    """The same comparison fails for plausible mistakes planted in a copy of
    the oracle's inputs or rule (on the CPU)."""
    cfg, inp = _case()
    blk = _hf_block(cfg, inp)
    x = torch.from_numpy(O.as_f64(inp.x))
    with torch.no_grad():
        logits, _, _ = blk.router(x[None], blk.expert_bias)
        out_hf = blk(x[None])[0].numpy()
    L32 = logits.numpy().astype(np.float32)
    bad_cfg, bad_inp = dict(cfg), inp
    if slip == "bias_on_logits":
        # bias added to the logits instead of the scores: select on sigmoid(L + b)
        L32 = (L32.astype(np.float64) + O.as_f64(inp.expert_bias)[None, :]).astype(np.float32)
        bad_inp = synth.MoeInputs(**{**inp.__dict__, "expert_bias": np.zeros_like(inp.expert_bias)})
    elif slip == "no_route_scale":
        bad_cfg["route_scale"] = 1.0
    elif slip == "no_shared":
        bad_cfg["num_shared_experts"] = 0
    elif slip == "swap_gate_up":
        bad_inp = synth.MoeInputs(**{**inp.__dict__, "w_gate": inp.w_up, "w_up": inp.w_gate})
    ref = O.moe_forward(bad_inp, bad_cfg, logits=L32)
    err = np.max(np.abs(out_hf - ref["out"])) / np.max(np.abs(out_hf))
    assert err > 1e-2, (slip, err)
