"""GPU parity of the layer with an MXFP8 router (the 8-bit router of the
4-bit Trinity checkpoints, mlxcel #845 "Checkpoint weight layout"): E4M3
codes [E, H] with E8M0 scales per 32 inputs, dequantised exactly to fp32 in
the workspace before the router GEMM, through the C ABI.

The oracle runs on the exact dequantised router (and experts): the GPU's
logits within 1e-5 of the oracle's, routing exactly from the GPU's logits,
the output at the layer's bar. Cases cover the four router GEMM paths (the
fp32-activation kernel, the one-launch small-batch kernel, the K-chunked
kernel with its reduce, the tiled kernel over split planes), bf16 and MXFP4 experts on both tile kernels, the stage
entry point moe_router_logits, and the Trinity-like q4r8 workloads (MXFP4
experts, MXFP8 router) at full size on sampled tokens."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, generated, rel_err, say
from tests.test_gpu_mxfp8 import oracle_view
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


CASES = {
    "fp32_tiny": custom(T=33, hidden_size=128, num_experts=6, num_experts_per_tok=2,
                        moe_intermediate_size=64, num_shared_experts=1, dtype="f32",
                        bias_limit=0.1, router_bf16_values=False, router_format="mxfp8"),
    "bf16_small_batch": custom(T=40, hidden_size=512, num_experts=16, num_experts_per_tok=4,
                               moe_intermediate_size=128, num_shared_experts=1,
                               router_format="mxfp8"),
    "bf16_partial_router": custom(T=16, hidden_size=2304, num_experts=8, num_experts_per_tok=2,
                                  moe_intermediate_size=128, num_shared_experts=1,
                                  router_format="mxfp8"),
    "bf16_tiled_router": custom(T=300, hidden_size=256, num_experts=16, num_experts_per_tok=4,
                                moe_intermediate_size=128, num_shared_experts=2,
                                shared_intermediate_size=64, x_scale=16.0,
                                router_format="mxfp8"),
    "softmax_grouped": custom(T=90, hidden_size=256, num_experts=64, num_experts_per_tok=6,
                              moe_intermediate_size=128, num_shared_experts=1, n_group=8,
                              topk_group=3, score_func="softmax", route_scale=2.5,
                              router_format="mxfp8"),
    "q4r8_decode": custom(T=32, hidden_size=1024, num_experts=64, num_experts_per_tok=8,
                          moe_intermediate_size=256, num_shared_experts=1,
                          shared_intermediate_size=256, route_scale=2.826,
                          router_bf16_values=False, weight_format="mxfp4",
                          router_format="mxfp8"),
    "q4r8_prefill": custom(T=600, hidden_size=384, num_experts=8, num_experts_per_tok=2,
                           moe_intermediate_size=320, num_shared_experts=1, shared_packed=1,
                           hidden_act="swigluoai", route_scale=2.0, weight_format="mxfp4",
                           router_format="mxfp8"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mx_router_layer_matches_oracle(name):
    cfg = CASES[name]
    inp = synth.generate(cfg)
    assert inp.w_router.dtype == np.uint8
    ov = oracle_view(inp)
    dev = Dev(inp)
    Lref = O.router_logits(ov.x, ov.w_router)
    for det in (True, False):
        st = run_stages(dev, deterministic=det)
        assert rel_err(st["logits"], Lref) <= 1e-5
        check_routing(cfg, inp, st)
        ref = O.moe_forward(ov, cfg, logits=st["logits"], want_hidden=True)
        e = rel_err(st["out"], ref["out"])
        say(f"[mx-router] {name} det={det} out {e:.2e}")
        assert e <= TOL[cfg["dtype"]]
    for det in (1, 0):
        res = dev.forward(deterministic=det)
        assert rel_err(res["logits"], Lref) <= 1e-5
        check_routing(cfg, inp, res)
        ref = O.moe_forward(ov, cfg, logits=res["logits"])
        assert rel_err(res["out"], ref["out"]) <= TOL[cfg["dtype"]]


def test_mx_router_equals_its_fp32_values():
    """The same layer with the MXFP8 router and with an fp32 router holding the
    dequantised values: the logits are bitwise equal (the router GEMM sees the
    same fp32 values), so routing and output are too."""
    cfg = CASES["bf16_small_batch"]
    inp = synth.generate(cfg)
    wr = O.mx_dequantize(inp.w_router, inp.mx["router"]).astype(np.float32)
    plain = synth.MoeInputs(**{**inp.__dict__, "cfg": dict(cfg, router_format="f32"),
                               "w_router": wr, "mx": None})
    a = Dev(inp).forward(deterministic=1)
    b = Dev(plain).forward(deterministic=1)
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("name", ["trinity_nano_decode_T32_q4r8", "trinity_nano_prefill_T8192_q4r8"])
def test_q4r8_full_size(name):
    """Every token: logits, routing and output of both combine modes against
    one oracle run on the exact dequantised router and expert values."""
    inp = generated(name)
    cfg = inp.cfg
    dev = Dev(inp)
    ov = oracle_view(inp)
    say(f"[q4r8-full] {name} T={dev.T}")
    runs = [dev.forward(deterministic=det) for det in (1, 0)]
    assert np.array_equal(runs[0]["logits"], runs[1]["logits"])
    Lref = O.router_logits(ov.x, ov.w_router)
    assert rel_err(runs[0]["logits"], Lref) <= 1e-5
    ref = O.moe_forward(ov, cfg, logits=runs[0]["logits"])
    for det, res in zip((1, 0), runs):
        check_routing(cfg, inp, res)
        assert np.array_equal(res["idx"], ref["idx"])
        e = rel_err(res["out"], ref["out"])
        say(f"[q4r8-full] {name} det={det} all {dev.T} tokens compared, rel err {e:.3e}")
        assert e <= TOL["bf16"]
