"""Batches large enough that every workgroup of the persistent grouped GEMMs
runs more tiles than it places up front: a workgroup stores the places of
its first tiles in LDS (256 for the 128-row kernels, 128 for the 32-row and
256-row ones) and computes the places of later ones on the fly.

* 128-row kernels: 600000 tokens, hidden 64, 4 experts top-2, intermediate
  1024 (8 gate/up column tiles): about 290 gate/up tiles per workgroup.
  Every token's output is compared with the float64 oracle (per token, in
  chunks).
* 32-row (decode) kernels, forced with MOE_GEMM_TILE=32 (they place 128 up
  front): 70000 tokens, hidden 256, 4 experts top-2, intermediate 1024: about
  137 gate/up tiles per workgroup, every token against the oracle.
* 256-row kernels: 600000 tokens, hidden and intermediate 1024, 4 experts
  top-2: about 146 gate/up tiles per workgroup. 24576 sampled tokens are
  compared (a 256-row tile holds none of their rows with probability about
  2e-5, (1 - 24576/600000)^256), the oracle's cost at full size being about
  7 TFLOP in float64.

Routing is checked over every token in both, at the layer's bf16 bar."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, say
from workloads import synth

import bench

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402

PLACED_UP_FRONT = 256  # tiles a workgroup of the 128-row kernels places in LDS before its loop
BM = 128               # activation rows per tile
GATE_UP_COLS = 128     # intermediate columns per gate/up tile


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def test_more_tiles_per_workgroup_than_placed_up_front():
    assert bench.gate_up_kernel(custom(T=600000, hidden_size=64, num_experts=4,
                                       num_experts_per_tok=2, moe_intermediate_size=1024,
                                       num_shared_experts=0), 600000) == "moe_gate_up_kernel"
    cfg = custom(T=600000, hidden_size=64, num_experts=4, num_experts_per_tok=2,
                 moe_intermediate_size=1024, num_shared_experts=0, name="many_tiles")
    inp = synth.generate(cfg)
    T, k, E, I = cfg["T"], cfg["num_experts_per_tok"], cfg["num_experts"], cfg["moe_intermediate_size"]
    dev = Dev(inp)
    say(f"[many tiles] T={T}")
    res = dev.forward(deterministic=1)
    s, keys, idx, w = O.route(res["logits"], inp.expert_bias, k, cfg["score_func"],
                              bool(cfg["route_norm"]), cfg["route_scale"])
    assert np.array_equal(res["idx"], idx)
    assert np.max(np.abs(res["w"] - w) / np.maximum(np.abs(w), 1e-30)) <= 1e-6
    # the launch really puts more tiles on each workgroup than it places up front
    counts = np.bincount(idx.reshape(-1), minlength=E)
    tiles = int(sum((n + BM - 1) // BM for n in counts)) * (I // GATE_UP_COLS)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"[many tiles] {tiles} gate/up tiles on {cus} compute units: {tiles / cus:.0f} each")
    assert tiles > PLACED_UP_FRONT * cus
    scale, err = 0.0, 0.0
    for c0 in range(0, T, 100000):
        tok = np.arange(c0, min(T, c0 + 100000))
        ref = O.moe_forward_tokens(inp, cfg, tok, logits_rows=res["logits"][tok])
        assert np.array_equal(ref["idx"], res["idx"][tok])
        scale = max(scale, float(np.max(np.abs(ref["out"]))))
        err = max(err, float(np.max(np.abs(res["out"][tok] - ref["out"]))))
    say(f"[many tiles] all {T} tokens compared, rel err {err / scale:.3e}")
    assert err / scale <= TOL[cfg["dtype"]]


WIDE_PLACED_UP_FRONT = 128
WIDE_BM = 256


def test_wide_tiles_more_per_workgroup_than_placed_up_front():
    cfg = custom(T=600000, hidden_size=1024, num_experts=4, num_experts_per_tok=2,
                 moe_intermediate_size=1024, num_shared_experts=0, name="many_wide_tiles")
    T, k, E, I = cfg["T"], cfg["num_experts_per_tok"], cfg["num_experts"], cfg["moe_intermediate_size"]
    assert bench.gate_up_kernel(cfg, T) == "moe_gate_up_wide_kernel"
    inp = synth.generate(cfg)
    dev = Dev(inp)
    say(f"[many wide tiles] T={T}")
    res = dev.forward(deterministic=1)
    s, keys, idx, w = O.route(res["logits"], inp.expert_bias, k, cfg["score_func"],
                              bool(cfg["route_norm"]), cfg["route_scale"])
    assert np.array_equal(res["idx"], idx)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    tiles = int(sum((n + WIDE_BM - 1) // WIDE_BM for n in counts)) * (2 * I // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"[many wide tiles] {tiles} gate/up tiles on {cus} compute units: {tiles / cus:.0f} each")
    assert tiles > WIDE_PLACED_UP_FRONT * cus
    tok = np.sort(np.random.default_rng(5).choice(T, 24576, replace=False))
    ref = O.moe_forward_tokens(inp, cfg, tok, logits_rows=res["logits"][tok])
    assert np.array_equal(ref["idx"], res["idx"][tok])
    e = float(np.max(np.abs(res["out"][tok] - ref["out"]))) / float(np.max(np.abs(ref["out"])))
    say(f"[many wide tiles] {tok.size} sampled tokens compared, rel err {e:.3e}")
    assert e <= TOL[cfg["dtype"]]


DECODE_PLACED_UP_FRONT = 128
DECODE_BM = 32


def test_decode_tiles_more_per_workgroup_than_placed_up_front(monkeypatch):
    monkeypatch.setenv("MOE_GEMM_TILE", "32")
    cfg = custom(T=70000, hidden_size=256, num_experts=4, num_experts_per_tok=2,
                 moe_intermediate_size=1024, num_shared_experts=0, name="many_decode_tiles")
    T, k, E, I = cfg["T"], cfg["num_experts_per_tok"], cfg["num_experts"], cfg["moe_intermediate_size"]
    inp = synth.generate(cfg)
    dev = Dev(inp)
    say(f"[many decode tiles] T={T}")
    res = dev.forward(deterministic=1)
    s, keys, idx, w = O.route(res["logits"], inp.expert_bias, k, cfg["score_func"],
                              bool(cfg["route_norm"]), cfg["route_scale"])
    assert np.array_equal(res["idx"], idx)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    tiles = int(sum((n + DECODE_BM - 1) // DECODE_BM for n in counts)) * (I // GATE_UP_COLS)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"[many decode tiles] {tiles} gate/up tiles on {cus} compute units: {tiles / cus:.0f} each")
    assert tiles > DECODE_PLACED_UP_FRONT * cus
    scale, err = 0.0, 0.0
    for c0 in range(0, T, 35000):
        tok = np.arange(c0, min(T, c0 + 35000))
        ref = O.moe_forward_tokens(inp, cfg, tok, logits_rows=res["logits"][tok])
        assert np.array_equal(ref["idx"], res["idx"][tok])
        scale = max(scale, float(np.max(np.abs(ref["out"]))))
        err = max(err, float(np.max(np.abs(res["out"][tok] - ref["out"]))))
    say(f"[many decode tiles] all {T} tokens compared, rel err {err / scale:.3e}")
    assert err / scale <= TOL[cfg["dtype"]]
