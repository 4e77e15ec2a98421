"""The whole layer captured in a HIP graph (through torch's graph capture) and
replayed: every replay must equal an eager call on the same inputs.

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
                              None, out, det, dev.ws)

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
