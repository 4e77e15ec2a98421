"""GPU parity of the layer with MXFP8 expert weights (OCP MX: E4M3 codes and
one E8M0 scale per 32 inputs, scales block-major; the MXFP8 export of
mlxcel #763 "Validation"), through the C ABI.

The oracle runs the layer on the exactly dequantised weights (the codes and
scales the GPU reads), fed the GPU's own router logits: routing and grouping
exactly, h, h_shared and the output at the layer's bf16 bar
(max|err| <= 2e-2 max|ref|). The GPU converts codes to bf16 exactly (a power-
of-two scale on a 4-bit significand), so its arithmetic differs from the bf16
path only in where the weights come from. Cases cover both tile kernels (32
rows for decode-sized batches, 128 rows otherwise), several tiles per
expert, two separate shared experts (their scale matrices side by side and
the shared down projection's K segments), the packed shared slot with
clamp-SwiGLU, no shared expert, one token, 128 experts, and both combine
modes; at full size the M3-shaped decode and prefill layers and the
Trinity-like decode layer, on every token."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, generated, rel_err, say
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


def oracle_view(inp):
    """The inputs with every MX (MXFP8 or MXFP4) expert weight stack replaced
    by its lazily dequantised float64 view, and an MXFP8 router by its
    dequantised values."""
    d = dict(inp.__dict__)
    wf = inp.cfg.get("weight_format", "dtype")
    if wf != "dtype":
        elem = "e2m1" if wf == "mxfp4" else "e4m3"
        for w, key in (("w_gate", "gate"), ("w_up", "up"), ("w_down", "down"),
                       ("ws_gate", "shared_gate"), ("ws_up", "shared_up"),
                       ("ws_down", "shared_down")):
            if d[w] is not None:
                d[w] = O.MxStacked(d[w], inp.mx[key], elem)
    if inp.cfg.get("router_format", "f32") == "mxfp8":
        d["w_router"] = O.mx_dequantize(inp.w_router, inp.mx["router"])
    return synth.MoeInputs(**d)


MX = {
    "several_tiles": custom(T=300, hidden_size=256, num_experts=4, num_experts_per_tok=2,
                            moe_intermediate_size=256, num_shared_experts=1,
                            shared_intermediate_size=256, weight_format="mxfp8"),
    "two_shared": custom(T=33, hidden_size=512, num_experts=8, num_experts_per_tok=2,
                         moe_intermediate_size=256, num_shared_experts=2,
                         shared_intermediate_size=128, weight_format="mxfp8"),
    "no_shared_k_eq_E": custom(T=20, hidden_size=256, num_experts=4, num_experts_per_tok=4,
                               moe_intermediate_size=256, num_shared_experts=0,
                               weight_format="mxfp8"),
    "packed_clamp": custom(T=64, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                           moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                           hidden_act="swigluoai", route_scale=2.0, w_std=0.2, x_scale=20.0,
                           weight_format="mxfp8"),
    "one_token": custom(T=1, hidden_size=256, num_experts=8, num_experts_per_tok=3,
                        moe_intermediate_size=256, num_shared_experts=1,
                        shared_intermediate_size=256, weight_format="mxfp8"),
    "m3_like_128_experts": custom(T=48, hidden_size=768, num_experts=128, num_experts_per_tok=4,
                                  moe_intermediate_size=256, num_shared_experts=1,
                                  shared_packed=1, route_scale=2.0, weight_format="mxfp8"),
    # K lengths that are multiples of three 128-input steps: the variant with
    # whole 128-byte weight rows per K-step, routed and shared (packed, and
    # two separate shared experts whose down projection is K-segmented)
    "k128_packed": custom(T=40, hidden_size=768, num_experts=16, num_experts_per_tok=4,
                          moe_intermediate_size=768, num_shared_experts=1, shared_packed=1,
                          hidden_act="swigluoai", route_scale=2.0, weight_format="mxfp8"),
    "k128_two_shared": custom(T=33, hidden_size=768, num_experts=8, num_experts_per_tok=2,
                              moe_intermediate_size=768, num_shared_experts=2,
                              shared_intermediate_size=384, weight_format="mxfp8"),
}


# the 128-row tile kernel: batches beyond the decode size, K lengths that
# are not multiples of 256 (the AFMoE width 1408), ragged last K-steps
MX_128 = {
    "afmoe_shape_two_shared": custom(T=700, hidden_size=512, num_experts=8, num_experts_per_tok=6,
                                     moe_intermediate_size=448, num_shared_experts=2,
                                     shared_intermediate_size=192, x_scale=22.6,
                                     weight_format="mxfp8"),
    "packed_clamp_prefill": custom(T=600, hidden_size=384, num_experts=4, num_experts_per_tok=2,
                                   moe_intermediate_size=320, num_shared_experts=1,
                                   shared_packed=1, hidden_act="swigluoai", route_scale=2.0,
                                   w_std=0.2, x_scale=20.0, weight_format="mxfp8"),
}


@pytest.mark.parametrize("name", list(MX) + list(MX_128))
def test_mxfp8_layer_matches_oracle(name, monkeypatch):
    cfg = MX.get(name) or MX_128[name]
    if name in MX and cfg["T"] > 64:
        monkeypatch.setenv("MOE_GEMM_TILE", "32")   # keep the 32-row kernel on the big edge case
    inp = synth.generate(cfg)
    assert inp.w_gate.dtype == np.uint8
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
        say(f"[mxfp8] {name} det={det} max rows/expert {c.max()} h {eh:.2e} out {e:.2e}")
        assert e <= tol
    for det in (1, 0):
        res = dev.forward(deterministic=det)
        check_routing(cfg, inp, res)
        ref = O.moe_forward(ov, cfg, logits=res["logits"])
        assert rel_err(res["out"], ref["out"]) <= TOL["bf16"]


def test_mxfp8_weights_and_their_bf16_values_agree():
    """The same layer with MXFP8 weights and with the bf16 tensors holding
    the dequantised values (exact in bf16): the two GPU paths differ only in
    where the weights come from, so the outputs agree to fp32 summation
    order."""
    cfg = MX["packed_clamp"]
    inp = synth.generate(cfg)
    ov = oracle_view(inp)
    E1 = cfg["num_experts"] + 1
    bf = lambda st: np.stack([synth.f32_to_bf16_bits(st[e].astype(np.float32)) for e in range(E1)])
    dq = synth.MoeInputs(**{**inp.__dict__, "cfg": dict(cfg, weight_format="dtype"), "mx": None,
                            "w_gate": bf(ov.w_gate), "w_up": bf(ov.w_up), "w_down": bf(ov.w_down)})
    for e in (0, E1 - 1):  # bf16 holds the dequantised values exactly
        assert np.array_equal(O.as_f64(dq.w_gate[e]), ov.w_gate[e])
    a = Dev(inp).forward(deterministic=1)
    b = Dev(dq).forward(deterministic=1)
    assert np.array_equal(a["idx"], b["idx"])
    assert rel_err(a["out"], b["out"]) <= 2e-3


@pytest.mark.parametrize("name", ["trinity_nano_decode_T32_mxfp8", "minimax_m3_decode_T64_mxfp8",
                                  "minimax_m3_prefill_T8192_mxfp8"])
def test_mxfp8_full_size(name):
    """Every output row of both combine modes against one oracle run (the
    router GEMM is fixed-order, so both calls produce the same logits)."""
    inp = generated(name)
    cfg = inp.cfg
    dev = Dev(inp)
    say(f"[mxfp8-full] {name} T={dev.T}")
    runs = [dev.forward(deterministic=det) for det in (1, 0)]
    assert np.array_equal(runs[0]["logits"], runs[1]["logits"])
    ref = O.moe_forward(oracle_view(inp), cfg, logits=runs[0]["logits"])
    for det, res in zip((1, 0), runs):
        check_routing(cfg, inp, res)
        assert np.array_equal(res["idx"], ref["idx"])
        e = rel_err(res["out"], ref["out"])
        say(f"[mxfp8-full] {name} det={det} all {dev.T} tokens compared, rel err {e:.3e}")
        assert e <= TOL["bf16"]
