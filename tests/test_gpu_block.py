"""GPU parity of the MoE block around the layer (mlxcel #845 "What the original
body missed": out = h + post_mlp_norm(layer(pre_mlp_norm(h))); Gemma-style
w + 1 scales for MiniMax-M3, mlxcel #763 Norms bullet), through the C ABI:

  * moe_rms_norm against the oracle's RMSNorm, every row-shape class
    (one, two, three and four 8-column groups per thread, rows narrower than
    a wave), bf16 and fp32, plain and Gemma-style, in place;
  * moe_combine_norm_residual against the combine written out in float64
    followed by the oracle's RMSNorm, both combine modes, in place;
  * moe_block_forward against the oracle's block fed the GPU's own router
    logits: routing exactly; the output within the layer's bar on the
    normalised branch plus the final rounding of out; also with MXFP8 and
    MXFP4 expert weights (the oracle on their exact values).

Bars: the RMSNorm stages are elementwise, so each element may carry the
storage rounding of its own value (2^-8 relative for bf16 stores of a value
computed in fp32, 1e-6 for fp32) over the fp32 arithmetic (1e-5 of the row
maximum). The block's out = h + b sums the residual with a branch b whose
error is the layer's (2e-2 max|b| in bf16, 1e-4 in fp32), and out itself is
rounded once more (2^-8 |out| in bf16)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.moe_harness import TOL, Dev, custom, say
from tests.test_gpu_mxfp8 import oracle_view
from workloads import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_moe_transformer_amd as moe  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


STORE = {"bf16": 2.0 ** -8, "f32": 1e-6}


def _host(t, shape):
    if t.dtype == torch.bfloat16:
        return t.view(shape).float().cpu().numpy().astype(np.float64)
    return t.view(shape).cpu().numpy().astype(np.float64)


def _stored(a, dtype):
    """float32 array -> stored values (bf16 bits for bf16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return synth.f32_to_bf16_bits(a) if dtype == "bf16" else a


def _assert_elementwise(got, ref, dtype, what):
    bound = STORE[dtype] * np.abs(ref) + 1e-5 * np.max(np.abs(ref), axis=-1, keepdims=True)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements off, worst {np.max(np.abs(got - ref)):.3e}"


# --------------------------------------------------------------------------
# moe_rms_norm

@pytest.mark.parametrize("H", [64, 320, 1024, 2048, 4160, 6144, 8192])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rms_norm(H, dtype):
    T = 37
    rng = np.random.default_rng(H)
    x = (rng.standard_normal((T, H)) * rng.uniform(0.01, 50.0, (T, 1))).astype(np.float32)
    x[3] = 0.0                                   # a zero row: eps keeps it zero
    xs = _stored(x, dtype)
    cfg = {"hidden_size": H, "num_experts": 8, "num_experts_per_tok": 2,
           "moe_intermediate_size": 64, "dtype": dtype}
    for add_one in (0, 1):
        w = (rng.standard_normal(H) * 0.1 + (0.0 if add_one else 1.0)).astype(np.float32)
        norm = {"eps": 1e-5, "add_one": add_one}
        xd = moe.to_device(xs).view(-1)
        wd = moe.to_device(w)
        y = torch.empty_like(xd)
        moe.moe_rms_norm(cfg, norm, T, xd, wd, y)
        ref = O.rms_norm(xs, w, 1e-5, bool(add_one))
        torch.cuda.synchronize()
        _assert_elementwise(_host(y, (T, H)), ref, dtype, f"H={H} {dtype} add_one={add_one}")
        assert np.all(_host(y, (T, H))[3] == 0.0)
        moe.moe_rms_norm(cfg, norm, T, xd, wd, xd)          # in place
        torch.cuda.synchronize()
        assert torch.equal(xd, y)


# --------------------------------------------------------------------------
# moe_combine_norm_residual

@pytest.mark.parametrize("H,k,dtype", [(1024, 8, "bf16"), (6144, 4, "bf16"), (2048, 6, "f32"),
                                       (320, 11, "bf16")])
def test_combine_norm_residual(H, k, dtype):
    T = 29
    rng = np.random.default_rng(7 + H)
    cfg = {"hidden_size": H, "num_experts": 16, "num_experts_per_tok": k,
           "moe_intermediate_size": 64, "dtype": dtype}
    acc = rng.standard_normal((T, H)).astype(np.float32)
    yp = _stored(rng.standard_normal((T * k, H)) * 3.0, dtype)
    row_pos = rng.permutation(T * k).astype(np.int32)
    tw = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    res = _stored(rng.standard_normal((T, H)) * 10.0, dtype)
    post = (rng.standard_normal(H) * 0.1 + 1.0).astype(np.float32)
    norm = {"eps": 1e-5, "add_one": 0}
    d = moe.to_device
    accd, ypd, rpd, twd, resd, postd = d(acc), d(yp).view(-1), d(row_pos), d(tw), d(res).view(-1), d(post)
    ys = O.as_f64(yp)
    for gather in (True, False):
        v = acc.astype(np.float64)
        if gather:
            for j in range(k):
                v = v + tw[:, j:j + 1].astype(np.float64) * ys[row_pos.reshape(T, k)[:, j]]
        ref = O.as_f64(res) + O.rms_norm(v, post, 1e-5, False)
        out = torch.empty_like(resd)
        moe.moe_combine_norm_residual(cfg, norm, T, accd, ypd if gather else None, rpd, twd,
                                      postd, resd, out)
        torch.cuda.synchronize()
        got = _host(out, (T, H))
        # branch error (fp32 arithmetic) plus the storage rounding of out
        bound = STORE[dtype] * np.abs(ref) + 1e-5 * np.max(np.abs(ref - O.as_f64(res)))
        assert np.all(np.abs(got - ref) <= bound), f"gather={gather}"
        inplace = resd.clone()
        moe.moe_combine_norm_residual(cfg, norm, T, accd, ypd if gather else None, rpd, twd,
                                      postd, inplace, inplace)
        torch.cuda.synchronize()
        assert torch.equal(inplace, out)


# --------------------------------------------------------------------------
# moe_block_forward

BLOCK = {
    "tiny_fp32": custom(T=64, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                        moe_intermediate_size=128, num_shared_experts=1, dtype="f32",
                        bias_limit=0.1, router_bf16_values=False),
    "afmoe_like_two_shared": custom(T=300, hidden_size=512, num_experts=16, num_experts_per_tok=6,
                                    moe_intermediate_size=256, num_shared_experts=2,
                                    x_scale=22.6),
    "m3_like_gemma_clamp": custom(T=200, hidden_size=768, num_experts=32, num_experts_per_tok=4,
                                  moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                                  hidden_act="swigluoai", route_scale=2.0, w_std=0.2,
                                  norm_add_one=1),
    "one_token_softmax": custom(T=1, hidden_size=256, num_experts=8, num_experts_per_tok=3,
                                moe_intermediate_size=256, num_shared_experts=1,
                                score_func="softmax"),
    # MX expert weights inside the block: MXFP8 on the 128-row tiles, MXFP4 on
    # the 32-row decode tiles
    "m3_like_mxfp8": custom(T=300, hidden_size=768, num_experts=16, num_experts_per_tok=4,
                            moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                            hidden_act="swigluoai", route_scale=2.0, norm_add_one=1,
                            weight_format="mxfp8"),
    "trinity_like_mxfp4_decode": custom(T=32, hidden_size=1024, num_experts=64,
                                        num_experts_per_tok=8, moe_intermediate_size=256,
                                        num_shared_experts=1, shared_intermediate_size=256,
                                        route_scale=2.826, weight_format="mxfp4"),
    # ... and with the 8-bit router as well (the q4r8 checkpoint widths)
    "trinity_like_q4r8_decode": custom(T=32, hidden_size=1024, num_experts=64,
                                       num_experts_per_tok=8, moe_intermediate_size=256,
                                       num_shared_experts=1, shared_intermediate_size=256,
                                       route_scale=2.826, weight_format="mxfp4",
                                       router_bf16_values=False, router_format="mxfp8"),
}


def run_block(dev, nw, deterministic, h=None, out=None):
    T, c = dev.T, dev.keys
    h = dev.x if h is None else h
    E, k, H = c["num_experts"], c["num_experts_per_tok"], c["hidden_size"]
    logits = torch.empty(T * E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    if out is None:
        out = torch.empty(T * H, dtype=moe.torch_dtype(c), device="cuda")
    ws = moe.alloc_block_workspace(c, T)
    moe.moe_block_forward(c, nw, T, h, moe.to_device(nw["pre"]), moe.to_device(nw["post"]),
                          dev.w_router, dev.expert_bias, dev.w_gate, dev.w_up, dev.w_down,
                          dev.ws_gate, dev.ws_up, dev.ws_down, logits, idx, w, out,
                          deterministic, ws, mx=dev.mx)
    torch.cuda.synchronize()
    return dict(logits=logits.view(T, E).cpu().numpy(), idx=idx.view(T, k).cpu().numpy(),
                w=w.view(T, k).cpu().numpy(), out=_host(out, (T, H)))


def check_block(cfg, inp, nw, res, tokens=None):
    """Routing exactly and out within the block's bar (see the module text)."""
    if inp.mx is not None:   # MX weights: the oracle runs on their exact values
        inp = oracle_view(inp)
    if tokens is not None:
        inp = synth.MoeInputs(**{**inp.__dict__, "x": inp.x[tokens]})
        res = {key: v[tokens] for key, v in res.items()}
    ref = O.block_forward(inp, cfg, nw["pre"], nw["post"], nw["eps"], bool(nw["add_one"]),
                          logits=res["logits"])
    assert np.array_equal(res["idx"], ref["idx"])
    assert np.max(np.abs(res["w"] - ref["w"]) / np.maximum(np.abs(ref["w"]), 1e-30)) <= 1e-6
    branch = ref["out"] - O.as_f64(inp.x)
    err = np.abs(res["out"] - ref["out"])
    bound = TOL[cfg["dtype"]] * np.max(np.abs(branch)) + STORE[cfg["dtype"]] * np.abs(ref["out"])
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"block out: worst err/bound {worst:.3f}"
    return worst


@pytest.mark.parametrize("name", list(BLOCK))
def test_block_forward_matches_oracle(name):
    cfg = BLOCK[name]
    inp = synth.generate(cfg)
    nw = synth.norm_weights(cfg)
    dev = Dev(inp)
    outs = []
    for det in (1, 0):
        res = run_block(dev, nw, det)
        worst = check_block(cfg, inp, nw, res)
        say(f"[block] {name} det={det} worst err/bound {worst:.3f}")
        outs.append(res["out"])
    # in place: out written over the input rows
    hcopy = dev.x.clone()
    res = run_block(dev, nw, 1, h=hcopy, out=hcopy)
    assert np.array_equal(res["out"], outs[0])


def test_block_with_decode_tiles(monkeypatch):
    """The 32-row GEMM tiles inside the block (decode-sized batches)."""
    monkeypatch.setenv("MOE_GEMM_TILE", "32")
    cfg = custom(T=48, hidden_size=768, num_experts=64, num_experts_per_tok=4,
                 moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                 hidden_act="swigluoai", route_scale=2.0, norm_add_one=1)
    inp = synth.generate(cfg)
    nw = synth.norm_weights(cfg)
    dev = Dev(inp)
    for det in (1, 0):
        check_block(cfg, inp, nw, run_block(dev, nw, det))


def test_zero_down_weights_return_the_residual():
    """With every down projection zero the branch is RMSNorm(0) = 0 and the
    block returns its input bit for bit."""
    cfg = custom(T=40, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                 moe_intermediate_size=128, num_shared_experts=1)
    inp = synth.generate(cfg)
    inp.w_down[:] = 0
    inp.ws_down[:] = 0
    nw = synth.norm_weights(cfg)
    dev = Dev(inp)
    for det in (1, 0):
        res = run_block(dev, nw, det)
        assert np.array_equal(res["out"], O.as_f64(inp.x))
