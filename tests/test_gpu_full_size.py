"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (moe_layer_forward, one stream): routing and grouping are checked over
every token, and the layer output over every token too (the float64 oracle
runs the whole layer, one expert at a time, fed the GPU's own logits), so
every tile class of the grouped GEMMs (each expert's ragged last m-slot,
every row band of a full tile, every XCD's tile range) is compared."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, generated, rel_err, say
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _check(dev, name, deterministic=0):
    inp, cfg = dev.inp, dev.inp.cfg
    say(f"[full] {name} T={dev.T}")
    res = dev.forward(deterministic=deterministic)
    k = cfg["num_experts_per_tok"]
    Lref = O.router_logits(inp.x, inp.w_router)
    assert rel_err(res["logits"], Lref) <= 1e-5
    s, keys, idx, w = O.route(res["logits"], inp.expert_bias, k, cfg["score_func"],
                              bool(cfg["route_norm"]), cfg["route_scale"],
                              cfg.get("n_group", 1), cfg.get("topk_group", 1))
    assert np.array_equal(res["idx"], idx)
    assert np.max(np.abs(res["w"] - w) / np.maximum(np.abs(w), 1e-30)) <= 1e-6
    say(f"[full] {name} boundary key gap {O.boundary_gap(keys, k):.3e}")
    ref = O.moe_forward(inp, cfg, logits=res["logits"])
    assert np.array_equal(ref["idx"], res["idx"])
    e = rel_err(res["out"], ref["out"])
    say(f"[full] {name} all {dev.T} tokens compared, rel err {e:.3e}")
    assert e <= TOL[cfg["dtype"]]
    return res


def test_trinity_prefill_T8192():
    dev = Dev(generated("trinity_nano_prefill_T8192"))
    _check(dev, "trinity_nano_prefill_T8192")


def test_skewed_T8192_hot_experts_and_ties():
    inp = generated("skewed_afmoe_T8192")
    dev = Dev(inp)
    sk = inp.meta["skew"]
    a, c = sk["tie_pair"]
    res = dev.forward(deterministic=0)
    L = res["logits"]
    # identical router rows give bitwise identical logit columns
    assert np.array_equal(L[:, a], L[:, c])
    idx = res["idx"]
    straddle = np.nonzero((idx == a).any(1) ^ (idx == c).any(1))[0]
    assert straddle.size > 0
    assert not np.any((idx == c).any(1) & ~(idx == a).any(1))  # a (lower) always wins the tie
    hot_share = np.isin(idx, sk["hot_experts"]).mean()
    counts = np.bincount(idx.reshape(-1), minlength=inp.cfg["num_experts"])
    say(f"[full] skew: hot share {hot_share:.3f}, empty experts {(counts == 0).sum()}, "
        f"max load {counts.max()}, tie straddle {straddle.size / idx.shape[0]:.3f}")
    _check(dev, "skewed_afmoe_T8192")


@pytest.fixture(scope="module")
def m3():
    return Dev(generated("minimax_m3_prefill_T8192"))


def test_minimax_m3_prefill_T8192(m3):
    _check(m3, "minimax_m3_prefill_T8192", deterministic=1)


def test_minimax_m3_decode_T64(m3):
    inp = m3.inp
    sub = synth.MoeInputs(cfg=dict(inp.cfg, T=64), x=inp.x[:64], w_router=inp.w_router,
                          expert_bias=inp.expert_bias, w_gate=inp.w_gate, w_up=inp.w_up,
                          w_down=inp.w_down)
    dev = Dev.__new__(Dev)
    dev.__dict__.update(m3.__dict__)
    dev.inp, dev.T = sub, 64
    dev.x = m3.x[: 64 * inp.cfg["hidden_size"]] if m3.x.dim() == 1 else m3.x[:64]
    dev.ws = moe.alloc_workspace(dev.keys, 64)
    # same x rows as a T=64 draw of the decode workload
    assert np.array_equal(synth.generate(synth.config("minimax_m3_decode_T64"), experts=False).x,
                          inp.x[:64])
    _check(dev, "minimax_m3_decode_T64")


def _check_block(dev, name):
    """The block (pre-norm, layer, post-norm, residual) at full size: routing
    and the output over every token."""
    from tests.test_gpu_block import check_block, run_block
    cfg = dev.inp.cfg
    nw = synth.norm_weights(cfg)
    say(f"[full] block {name} T={dev.T} add_one={nw['add_one']}")
    res = run_block(dev, nw, 1)
    worst = check_block(cfg, dev.inp, nw, res)
    say(f"[full] block {name} all {dev.T} tokens compared, worst err/bound {worst:.3f}")


def test_minimax_m3_block_T8192(m3):
    _check_block(m3, "minimax_m3_prefill_T8192")


def test_afmoe_default_block_T4096():
    _check_block(Dev(generated("afmoe_default_T4096")), "afmoe_default_T4096")
