"""The whole layer (bf16, MXFP8 and MXFP4 weights, decode- and
prefill-sized) and the MoE block captured in a HIP graph (through torch's
graph capture) and replayed: every replay must equal an eager call on the same inputs. Also:
layer calls on two streams at once, with their own workspaces, equal the
same calls made one after the other.

The entry points allocate nothing, copy nothing and never synchronise with
the host, so a caller can capture them. Each check replays the graph several
times with eager library calls and input updates in between, and compares
every replay with an eager result: bitwise in the fixed-order mode, and at
the layer's float bar against the eager fixed-order output with fp32
atomics."""
import numpy as np
import pytest

from tests.moe_harness import TOL, Dev, custom, generated, rel_err, say
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
    "trinity_nano_decode_T32": None,
    "ragged_prefill": custom(T=333, hidden_size=256, num_experts=16, num_experts_per_tok=4,
                             moe_intermediate_size=192, num_shared_experts=1, route_scale=2.0),
    "mxfp8_decode": custom(T=48, hidden_size=768, num_experts=16, num_experts_per_tok=4,
                           moe_intermediate_size=768, num_shared_experts=1, shared_packed=1,
                           hidden_act="swigluoai", route_scale=2.0, weight_format="mxfp8"),
    "mxfp8_prefill": custom(T=400, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                            moe_intermediate_size=256, num_shared_experts=2,
                            shared_intermediate_size=128, weight_format="mxfp8"),
    "mxfp4_decode": custom(T=48, hidden_size=1024, num_experts=16, num_experts_per_tok=4,
                           moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                           hidden_act="swigluoai", route_scale=2.0, weight_format="mxfp4"),
    "q4r8_decode": custom(T=32, hidden_size=1024, num_experts=64, num_experts_per_tok=8,
                          moe_intermediate_size=256, num_shared_experts=1,
                          shared_intermediate_size=256, route_scale=2.826,
                          weight_format="mxfp4", router_format="mxfp8"),
}


def _inputs(name):
    cfg = CASES[name]
    return generated(name) if cfg is None else synth.generate(cfg)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    inp = _inputs(name)
    dev = Dev(inp)
    c, T = dev.keys, dev.T
    H = c["hidden_size"]
    dt = moe.torch_dtype(c)
    x_a = dev.x.clone()
    # a second input: the same tokens in reverse order
    x_b = dev.x.reshape(T, H).flip(0).contiguous().view_as(dev.x)
    out_g = torch.empty(T * H, dtype=dt, device="cuda")

    def layer(out, det):
        moe.moe_layer_forward(c, T, dev.x, dev.w_router, dev.expert_bias, dev.w_gate, dev.w_up,
                              dev.w_down, dev.ws_gate, dev.ws_up, dev.ws_down, None, None, None,
                              None, out, det, dev.ws, mx=dev.mx)

    def eager(x_src, det):
        dev.x.copy_(x_src)
        out = torch.empty(T * H, dtype=dt, device="cuda")
        layer(out, det)
        torch.cuda.synchronize()
        return out.clone()

    for det in (1, 0):
        ref = {"a": eager(x_a, 1), "b": eager(x_b, 1)}
        layer(out_g, det)  # warm-up on the capture inputs
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer(out_g, det)
        torch.cuda.synchronize()
        for rep, key in enumerate(["a", "b", "a", "b"]):
            dev.x.copy_(x_a if key == "a" else x_b)
            out_g.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = out_g.clone()
            # eager library work between replays (other buffers)
            eager(x_b if key == "a" else x_a, det)
            if det:
                assert torch.equal(got, ref[key]), f"{name} replay {rep} differs from eager"
            else:
                e = rel_err(got.float().cpu().numpy(), ref[key].float().cpu().numpy())
                assert e <= TOL[inp.cfg["dtype"]], f"{name} replay {rep}: rel err {e:.3e}"
            say(f"[graph] {name} det={det} replay {rep} ok")
        del g


def test_block_graph_replays_match_eager():
    """moe_block_forward (pre-norm, layer, post-norm + residual) in a graph."""
    cfg = custom(T=120, hidden_size=512, num_experts=16, num_experts_per_tok=4,
                 moe_intermediate_size=256, num_shared_experts=1, shared_packed=1,
                 hidden_act="swigluoai", route_scale=2.0, norm_add_one=1)
    inp = synth.generate(cfg)
    nw = synth.norm_weights(cfg)
    dev = Dev(inp)
    c, T, H = dev.keys, dev.T, cfg["hidden_size"]
    ws = moe.alloc_block_workspace(c, T)
    pre, post = moe.to_device(nw["pre"]), moe.to_device(nw["post"])
    h0 = dev.x.clone()
    h_in = dev.x.clone()
    out_g = torch.empty_like(h_in)

    def block(out):
        moe.moe_block_forward(c, nw, T, h_in, pre, post, dev.w_router, dev.expert_bias,
                              dev.w_gate, dev.w_up, dev.w_down, dev.ws_gate, dev.ws_up,
                              dev.ws_down, None, None, None, out, 1, ws)

    ref = torch.empty_like(h_in)
    block(ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block(out_g)
    torch.cuda.synchronize()
    for rep in range(4):
        h_in.copy_(h0)
        out_g.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"block replay {rep} differs from eager"
        block(torch.empty_like(h_in))   # eager work between replays
        torch.cuda.synchronize()
    say("[graph] block: 4 replays equal the eager call")


def test_two_streams_with_own_workspaces():
    """Concurrent layer calls on two streams (each with its own workspace and
    outputs) give the same bits as the same calls made one after another."""
    devs = [Dev(_inputs("ragged_prefill")), Dev(_inputs("trinity_nano_decode_T32"))]
    outs = [torch.empty(d.T * d.keys["hidden_size"], dtype=moe.torch_dtype(d.keys), device="cuda")
            for d in devs]

    def call(d, out, stream):
        moe.moe_layer_forward(d.keys, d.T, d.x, d.w_router, d.expert_bias, d.w_gate, d.w_up,
                              d.w_down, d.ws_gate, d.ws_up, d.ws_down, None, None, None, None,
                              out, 1, d.ws, stream)

    seq = []
    for d, o in zip(devs, outs):
        call(d, o, torch.cuda.current_stream())
        torch.cuda.synchronize()
        seq.append(o.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(5):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for d, o, st in zip(devs, outs, streams):
            call(d, o, st)
        torch.cuda.synchronize()
        for o, r in zip(outs, seq):
            assert torch.equal(o, r), f"concurrent call {rep} differs"
    say("[streams] 5 rounds of concurrent calls equal the sequential ones")

