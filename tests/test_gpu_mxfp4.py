"""GPU parity of the layer with MXFP4 expert weights (OCP MX: E2M1 codes, two
per byte with input 2j in the low nibble of byte j, and one E8M0 scale per
32 inputs, scales block-major; read as the format of the 4-bit Trinity
checkpoints of mlxcel #845 "Checkpoint confirmed"), through the C ABI.

As for MXFP8: the oracle runs the layer on the exactly dequantised weights,
fed the GPU's own router logits; routing and grouping exactly, h, h_shared
and the output at the layer's bf16 bar (max|err| <= 2e-2 max|ref|). The GPU
turns codes into bf16 exactly (a power-of-two scale on a 2-bit significand).
Cases cover the 32-row kernel with four and two stages of 128-input K-steps
(and a launch mixing them: gate/up with four, down with two), several tiles
per expert, two separate shared experts (the shared down projection's K
segments), the packed shared slot with clamp-SwiGLU, no shared expert, one
token and 128 experts; the 128-row kernel on batches beyond the decode size,
on K lengths that are not multiples of 256, and on four shared experts of
width 64 (a 128-input K-step would straddle two of them, so the 128-row
kernel takes even a decode-sized batch); at full size the Trinity-like decode
and prefill layers and the M3-shaped decode layer, on every token."""
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


def _c(**kw):
    return custom(weight_format="mxfp4", **kw)


# the 32-row kernel (every K length a multiple of 256)
MX4 = {
    # K lengths of six 128-input steps (two stages), the packed shared slot;
    # three separate shared experts of width 256, whose down projection is
    # K-segmented
    "k768_packed": _c(T=40, hidden_size=768, num_experts=16, num_experts_per_tok=4,
                         moe_intermediate_size=768, num_shared_experts=1, shared_packed=1,
                         hidden_act="swigluoai", route_scale=2.0),
    "k768_three_shared": _c(T=33, hidden_size=768, num_experts=8, num_experts_per_tok=2,
                               moe_intermediate_size=768, num_shared_experts=3,
                               shared_intermediate_size=256),
    "k512_packed_four_stages": _c(T=40, hidden_size=1024, num_experts=16, num_experts_per_tok=4,
                                  moe_intermediate_size=512, num_shared_experts=1, shared_packed=1,
                                  hidden_act="swigluoai", route_scale=2.0),
    "mixed_stages": _c(T=48, hidden_size=1024, num_experts=16, num_experts_per_tok=4,
                       moe_intermediate_size=256, num_shared_experts=1,
                       shared_intermediate_size=256),
    "two_shared": _c(T=33, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                     moe_intermediate_size=256, num_shared_experts=2, shared_intermediate_size=128),
    "several_tiles": _c(T=300, hidden_size=256, num_experts=4, num_experts_per_tok=2,
                        moe_intermediate_size=256, num_shared_experts=1,
                        shared_intermediate_size=256),
    "no_shared_k_eq_E": _c(T=20, hidden_size=256, num_experts=4, num_experts_per_tok=4,
                           moe_intermediate_size=256, num_shared_experts=0),
    "packed_clamp": _c(T=64, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                       moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                       hidden_act="swigluoai", route_scale=2.0, w_std=0.2, x_scale=20.0),
    "one_token": _c(T=1, hidden_size=256, num_experts=8, num_experts_per_tok=3,
                    moe_intermediate_size=256, num_shared_experts=1, shared_intermediate_size=256),
    "m3_like_128_experts": _c(T=48, hidden_size=768, num_experts=128, num_experts_per_tok=4,
                              moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                              route_scale=2.0),
}

# the 128-row kernel
MX4_128 = {
    "afmoe_shape_two_shared": _c(T=700, hidden_size=512, num_experts=8, num_experts_per_tok=6,
                                 moe_intermediate_size=448, num_shared_experts=2,
                                 shared_intermediate_size=192, x_scale=22.6),
    "packed_clamp_prefill": _c(T=600, hidden_size=384, num_experts=4, num_experts_per_tok=2,
                               moe_intermediate_size=320, num_shared_experts=1, shared_packed=1,
                               hidden_act="swigluoai", route_scale=2.0, w_std=0.2, x_scale=20.0),
    "four_shared_width_64": _c(T=16, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                               moe_intermediate_size=256, num_shared_experts=4,
                               shared_intermediate_size=64),
}


@pytest.mark.parametrize("name", list(MX4) + list(MX4_128))
def test_mxfp4_layer_matches_oracle(name, monkeypatch):
    cfg = MX4.get(name) or MX4_128[name]
    if name in MX4 and cfg["T"] > 64:
        monkeypatch.setenv("MOE_GEMM_TILE", "32")   # keep the 32-row kernel on the big edge case
    inp = synth.generate(cfg)
    assert inp.w_gate.dtype == np.uint8 and inp.w_gate.shape[2] == cfg["hidden_size"] // 2
    ov = oracle_view(inp)
    dev = Dev(inp)
    for det in (True, False):
        st = run_stages(dev, deterministic=det)
        check_routing(cfg, inp, st)
        c, off, sr, rp = O.permute(st["idx"], cfg["num_experts"])
        assert np.array_equal(st["offsets"], off) and np.array_equal(st["sorted_rows"], sr)
        ref = O.moe_forward(ov, cfg, logits=st["logits"], want_hidden=True)
        tol = TOL["bf16"]
        eh = rel_err(st["h"], ref["h"])
        assert eh <= tol, f"h rel err {eh:.3e}"
        if ref["h_shared"] is not None:
            assert rel_err(st["h_shared"], ref["h_shared"]) <= tol
        e = rel_err(st["out"], ref["out"])
        say(f"[mxfp4] {name} det={det} max rows/expert {c.max()} h {eh:.2e} out {e:.2e}")
        assert e <= tol
    for det in (1, 0):
        res = dev.forward(deterministic=det)
        check_routing(cfg, inp, res)
        ref = O.moe_forward(ov, cfg, logits=res["logits"])
        assert rel_err(res["out"], ref["out"]) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["k512_packed_four_stages", "packed_clamp_prefill"])
def test_mxfp4_weights_and_their_bf16_values_agree(name):
    """The same layer with MXFP4 weights and with bf16 tensors holding the
    dequantised values (exact in bf16), on both tile kernels: the paths
    differ only in where the weights come from, so the outputs agree to fp32
    summation order."""
    cfg = MX4.get(name) or MX4_128[name]
    inp = synth.generate(cfg)
    ov = oracle_view(inp)
    E1 = cfg["num_experts"] + 1
    bf = lambda st: np.stack([synth.f32_to_bf16_bits(st[e].astype(np.float32)) for e in range(E1)])
    dq = synth.MoeInputs(**{**inp.__dict__, "cfg": dict(cfg, weight_format="dtype"), "mx": None,
                            "w_gate": bf(ov.w_gate), "w_up": bf(ov.w_up), "w_down": bf(ov.w_down)})
    for e in (0, E1 - 1):
        assert np.array_equal(O.as_f64(dq.w_gate[e]), ov.w_gate[e])
    a = Dev(inp).forward(deterministic=1)
    b = Dev(dq).forward(deterministic=1)
    assert np.array_equal(a["idx"], b["idx"])
    assert rel_err(a["out"], b["out"]) <= 2e-3


@pytest.mark.parametrize("name", ["trinity_nano_decode_T32_mxfp4", "minimax_m3_decode_T64_mxfp4",
                                  "trinity_nano_prefill_T8192_mxfp4"])
def test_mxfp4_full_size(name):
    """Every output row of both combine modes against one oracle run (the
    router GEMM is fixed-order, so both calls produce the same logits)."""
    inp = generated(name)
    cfg = inp.cfg
    dev = Dev(inp)
    say(f"[mxfp4-full] {name} T={dev.T}")
    runs = [dev.forward(deterministic=det) for det in (1, 0)]
    assert np.array_equal(runs[0]["logits"], runs[1]["logits"])
    ref = O.moe_forward(oracle_view(inp), cfg, logits=runs[0]["logits"])
    for det, res in zip((1, 0), runs):
        check_routing(cfg, inp, res)
        assert np.array_equal(res["idx"], ref["idx"])
        e = rel_err(res["out"], ref["out"])
        say(f"[mxfp4-full] {name} det={det} all {dev.T} tokens compared, rel err {e:.3e}")
        assert e <= TOL["bf16"]
