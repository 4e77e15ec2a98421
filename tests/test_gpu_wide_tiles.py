"""The 256-row tile kernels (prefill-sized bf16 batches), forced onto edge
cases with MOE_GEMM_TILE=256, through the C ABI against the float64 oracle:
odd K-step counts (a leading zero step), N tails of the gate/up and down
tiles, half tiles (an expert's last <= 128 rows) next to full and partly
filled tiles, several full tiles per expert, two shared experts (the shared
down projection's K segments), the packed shared slot with clamp-SwiGLU and
no route_norm, no shared expert, and both combine modes. Every stage is
also compared with the 128-row kernels on the same inputs: both run the
same MFMA sequence over K per output element, so h and the fixed-order
outputs agree bit for bit, and the atomic-combine outputs to the order of
the fp32 atomics (one bf16 rounding step)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, rel_err, say
from tests.test_gpu_parity import EDGE, check_routing, run_stages
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


WIDE = {
    # H=192: 3 K-steps (odd); I=64: gate/up and down N tails, 1-step down K;
    # two shared experts (shared down K = 2 segments); ~180 rows per expert
    "ragged_odd_k_two_shared": custom(T=300, hidden_size=192, num_experts=5,
                                      num_experts_per_tok=3, moe_intermediate_size=64,
                                      num_shared_experts=2, shared_intermediate_size=64),
    # packed shared slot, clamp-SwiGLU, route_norm off; 3 gate/up n-tiles;
    # shared m-slots 256, 256, 188 rows
    "packed_clamp_nonorm": custom(T=700, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                                  moe_intermediate_size=384, num_shared_experts=1,
                                  shared_packed=1, hidden_act="swigluoai", route_norm=0,
                                  route_scale=2.0, w_std=0.05),
    # ~512 rows per expert: several full tiles per expert, two down n-tiles
    "multi_tile_experts": custom(T=2048, hidden_size=512, num_experts=16, num_experts_per_tok=4,
                                 moe_intermediate_size=256, num_shared_experts=1),
    # no shared expert; H=320 (5 K-steps), I=192 (gate/up N tail of 64, 3-step down K)
    "no_shared_odd": custom(T=513, hidden_size=320, num_experts=4, num_experts_per_tok=2,
                            moe_intermediate_size=192, num_shared_experts=0),
    # clamp driven hard (most pre-activations past the limit); all half tiles
    "clamp_swigluoai": EDGE["clamp_swigluoai"],
}


def _stages(dev, det, tile, monkeypatch):
    monkeypatch.setenv("MOE_GEMM_TILE", tile)
    return run_stages(dev, deterministic=det)


@pytest.mark.parametrize("name", list(WIDE))
def test_wide_tiles_match_oracle_and_128_row_tiles(name, monkeypatch):
    cfg = WIDE[name]
    inp = synth.generate(cfg)
    dev = Dev(inp)
    tol = TOL[cfg["dtype"]]
    counts = None
    for det in (True, False):
        say(f"[wide] {name} det={det}")
        st = _stages(dev, det, "256", monkeypatch)
        ref128 = _stages(dev, det, "128", monkeypatch)
        check_routing(cfg, inp, st)
        counts = np.bincount(st["idx"].reshape(-1), minlength=cfg["num_experts"])
        ref = O.moe_forward(inp, cfg, logits=st["logits"], want_hidden=True)
        assert rel_err(st["h"], ref["h"]) <= tol
        if ref["h_shared"] is not None:
            assert rel_err(st["h_shared"], ref["h_shared"]) <= tol
        e = rel_err(st["out"], ref["out"])
        assert e <= tol
        # against the 128-row kernels on the same inputs
        assert np.array_equal(st["idx"], ref128["idx"])
        assert rel_err(st["h"], ref128["h"]) <= 1e-6
        # fixed-order combine: the same fp32 sums; atomic combine: the fp32
        # atomics' order varies from run to run, and the bf16 output rounding
        # then moves an element by up to one bf16 ulp (2^-8 relative)
        e128 = rel_err(st["out"], ref128["out"])
        assert e128 <= (1e-6 if det else 2.0 ** -8)
        bitwise = np.array_equal(st["h"], ref128["h"]) and np.array_equal(st["out"], ref128["out"])
        say(f"[wide] {name} det={det} out rel err {e:.3e}, vs 128-row {e128:.1e} "
            f"(bitwise {bitwise}), rows per expert {counts.tolist()}")


def test_wide_layer_forward_repeats_bitwise(monkeypatch):
    """The whole layer on the 256-row tiles, fixed-order combine: bitwise
    repeatable, and within the bar of the oracle."""
    monkeypatch.setenv("MOE_GEMM_TILE", "256")
    cfg = WIDE["multi_tile_experts"]
    inp = synth.generate(cfg)
    dev = Dev(inp)
    a, b = dev.forward(deterministic=1), dev.forward(deterministic=1)
    assert np.array_equal(a["out"], b["out"])
    ref = O.moe_forward(inp, cfg, logits=a["logits"])
    assert np.array_equal(a["idx"], ref["idx"])
    assert rel_err(a["out"], ref["out"]) <= TOL["bf16"]
