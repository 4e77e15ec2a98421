"""GPU parity of the 32-row tile GEMM kernels (decode-sized batches, bf16),
forced onto small seeded workloads so that every path runs: several tiles
per expert with a ragged last one, one row per expert, two shared experts
(the shared down projection's K segments), no shared expert, the packed
shared slot with clamp-SwiGLU, and both combine modes (fixed-order rows and
fp32 atomics).

Every stage is compared with the float64 oracle fed the GPU's own router
logits: routing and grouping exactly, h, h_shared and the output at the
layer's bf16 bar (max|err| <= 2e-2 max|ref|). Through the single entry
point, batches of at most 256 routed rows are grouped inside the gate/up
kernel (token masks up to 64 tokens, counted ranks above); its output is
held to the same bar."""
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, rel_err, say
from tests.test_gpu_parity import check_routing, run_stages
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


# hidden, intermediate and S*I_s are multiples of 256 (the 32-row kernel's
# K lengths are whole numbers of four 64-element steps)
DECODE = {
    "several_tiles": custom(T=300, hidden_size=256, num_experts=4, num_experts_per_tok=2,
                            moe_intermediate_size=256, num_shared_experts=1,
                            shared_intermediate_size=256),
    "two_shared": custom(T=33, hidden_size=512, num_experts=8, num_experts_per_tok=2,
                         moe_intermediate_size=256, num_shared_experts=2,
                         shared_intermediate_size=128),
    "no_shared_k_eq_E": custom(T=20, hidden_size=256, num_experts=4, num_experts_per_tok=4,
                               moe_intermediate_size=256, num_shared_experts=0),
    "packed_clamp": custom(T=64, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                           moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                           hidden_act="swigluoai", route_scale=2.0, w_std=0.2, x_scale=20.0),
    "one_token": custom(T=1, hidden_size=256, num_experts=8, num_experts_per_tok=3,
                        moe_intermediate_size=256, num_shared_experts=1,
                        shared_intermediate_size=256),
    "m3_like_128_experts": custom(T=48, hidden_size=768, num_experts=128, num_experts_per_tok=4,
                                  moe_intermediate_size=256, num_shared_experts=1,
                                  shared_packed=1, route_scale=2.0),
    # more than 64 tokens and at most 256 routed rows: the layer groups the
    # rows inside the gate/up kernel by counting earlier equal rows (64
    # tokens or fewer take the token-mask ranks; above 256 rows, a grouping
    # launch runs first)
    "t120_rows240": custom(T=120, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                           moe_intermediate_size=256, num_shared_experts=1),
}


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_tiles_match_oracle(name, monkeypatch):
    monkeypatch.setenv("MOE_GEMM_TILE", "32")
    cfg = DECODE[name]
    inp = synth.generate(cfg)
    dev = Dev(inp)
    for det in (True, False):
        st = run_stages(dev, deterministic=det)
        check_routing(cfg, inp, st)
        c, off, sr, rp = O.permute(st["idx"], cfg["num_experts"])
        assert np.array_equal(st["offsets"], off) and np.array_equal(st["sorted_rows"], sr)
        ref = O.moe_forward(inp, cfg, logits=st["logits"], want_hidden=True)
        tol = TOL["bf16"]
        eh = rel_err(st["h"], ref["h"])
        assert eh <= tol, f"h rel err {eh:.3e}"
        if ref["h_shared"] is not None:
            assert rel_err(st["h_shared"], ref["h_shared"]) <= tol
        e = rel_err(st["out"], ref["out"])
        say(f"[decode] {name} det={det} max rows/expert {c.max()} h {eh:.2e} out {e:.2e}")
        assert e <= tol
    for det in (1, 0):
        res = dev.forward(deterministic=det)
        check_routing(cfg, inp, res)
        ref = O.moe_forward(inp, cfg, logits=res["logits"])
        assert rel_err(res["out"], ref["out"]) <= TOL["bf16"]


def test_decode_and_128_row_tiles_agree():
    """The two GEMM kernels differ only in tiling: identical routing, outputs
    within the bf16 bar of each other, and each bitwise repeatable."""
    cfg = DECODE["several_tiles"]
    inp = synth.generate(cfg)
    dev = Dev(inp)
    outs = {}
    for tile in ("128", "32"):
        os.environ["MOE_GEMM_TILE"] = tile
        try:
            a, b = dev.forward(deterministic=1), dev.forward(deterministic=1)
        finally:
            del os.environ["MOE_GEMM_TILE"]
        assert np.array_equal(a["out"], b["out"])
        outs[tile] = a
    assert np.array_equal(outs["128"]["idx"], outs["32"]["idx"])
    assert rel_err(outs["32"]["out"], outs["128"]["out"]) <= TOL["bf16"]


def test_batch_sizes_interleaved_on_one_workspace():
    """One workspace, batch sizes that take every grouping path in turn
    (inside the gate/up kernel with token masks, the one-workgroup sort, the
    three-kernel sort) and both GEMM kernels, with no
    state carried from one call to the next: each output against the oracle,
    and the first batch size bitwise equal when it comes round again."""
    cfg = custom(T=300, hidden_size=512, num_experts=16, num_experts_per_tok=4,
                 moe_intermediate_size=256, num_shared_experts=1)
    full = synth.generate(cfg)
    dev = Dev(full)
    first = None
    for T in (32, 300, 7, 100, 64, 1, 32):
        sub = synth.MoeInputs(cfg=dict(cfg, T=T), x=full.x[:T], w_router=full.w_router,
                              expert_bias=full.expert_bias, w_gate=full.w_gate, w_up=full.w_up,
                              w_down=full.w_down, ws_gate=full.ws_gate, ws_up=full.ws_up,
                              ws_down=full.ws_down)
        d = Dev.__new__(Dev)
        d.__dict__.update(dev.__dict__)
        d.inp, d.cfg, d.T = sub, sub.cfg, T
        d.x = dev.x[: T * cfg["hidden_size"]] if dev.x.dim() == 1 else dev.x[:T]
        res = d.forward(deterministic=1)
        check_routing(sub.cfg, sub, res)
        ref = O.moe_forward(sub, sub.cfg, logits=res["logits"])
        e = rel_err(res["out"], ref["out"])
        say(f"[decode] interleaved T={T} rows={T * 4} out {e:.2e}")
        assert e <= TOL["bf16"]
        if T == 32:
            if first is None:
                first = res["out"]
            else:
                assert np.array_equal(first, res["out"])
