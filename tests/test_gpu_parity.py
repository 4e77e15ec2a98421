"""GPU parity of every stage and of the whole layer against the float64 oracle,
through the C ABI, on seeded inputs that span several tiles and ragged tails.

Routing is compared with the oracle fed the GPU's own fp32 router logits:
indices bit-exact, weights to 1e-6 relative; the grouping is integer-exact;
hidden activations and outputs meet the layer's float bar
(bf16: max|err| <= 2e-2 max|ref|, fp32: 1e-4 max|ref|)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
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


# edge-case workloads: ragged T, N/K tails, k == E, no shared expert, packed
# shared + clamp-SwiGLU without norm, fp32, one token, one expert, many experts
EDGE = {
    "ragged_bf16": custom(T=77, hidden_size=192, num_experts=5, num_experts_per_tok=3,
                          moe_intermediate_size=64, num_shared_experts=2,
                          shared_intermediate_size=64),
    "k_eq_E_no_shared": custom(T=40, hidden_size=128, num_experts=4, num_experts_per_tok=4,
                               moe_intermediate_size=128, num_shared_experts=0),
    "packed_swigluoai_nonorm": custom(T=300, hidden_size=256, num_experts=16,
                                      num_experts_per_tok=4, moe_intermediate_size=128,
                                      num_shared_experts=1, shared_packed=1,
                                      hidden_act="swigluoai", route_norm=0, route_scale=2.0,
                                      w_std=0.05),
    "clamp_swigluoai": custom(T=130, hidden_size=256, num_experts=8, num_experts_per_tok=2,
                              moe_intermediate_size=128, num_shared_experts=1, shared_packed=1,
                              hidden_act="swigluoai", route_scale=2.0, w_std=0.2, x_scale=20.0),
    "fp32_ragged": custom(T=33, hidden_size=128, num_experts=6, num_experts_per_tok=2,
                          moe_intermediate_size=64, num_shared_experts=1, dtype="f32",
                          bias_limit=0.1, router_bf16_values=False),
    "one_token": custom(T=1, hidden_size=256, num_experts=8, num_experts_per_tok=3,
                        moe_intermediate_size=128, num_shared_experts=1),
    "one_expert": custom(T=50, hidden_size=128, num_experts=1, num_experts_per_tok=1,
                         moe_intermediate_size=64, num_shared_experts=0, route_scale=2.826),
    "many_experts_k32": custom(T=20, hidden_size=64, num_experts=1024, num_experts_per_tok=32,
                               moe_intermediate_size=64, num_shared_experts=1),
    "e300_k8": custom(T=257, hidden_size=128, num_experts=300, num_experts_per_tok=8,
                      moe_intermediate_size=64, num_shared_experts=1, route_scale=2.826),
    # softmax scoring (HF "AFMoE" doc: sigmoid or softmax scores)
    "softmax_norm": custom(T=150, hidden_size=128, num_experts=16, num_experts_per_tok=4,
                           moe_intermediate_size=64, num_shared_experts=1,
                           score_func="softmax", route_scale=1.5),
    # the MiniMax-M2 router shape (256 experts, top-8; mlxcel #763 summary)
    "m2_shape_softmax_nonorm": custom(T=40, hidden_size=128, num_experts=256,
                                      num_experts_per_tok=8, moe_intermediate_size=64,
                                      num_shared_experts=0, score_func="softmax",
                                      route_norm=0, route_scale=2.0),
    "m2_shape_sigmoid": custom(T=70, hidden_size=128, num_experts=256, num_experts_per_tok=8,
                               moe_intermediate_size=64, num_shared_experts=1),
    # group-limited routing (mlxcel #845 "Routing detail": n_group)
    "grouped_e64_g8_keep3": custom(T=150, hidden_size=128, num_experts=64, num_experts_per_tok=6,
                                   moe_intermediate_size=64, num_shared_experts=1, n_group=8,
                                   topk_group=3),
    "grouped_e256_g8_keep4_softmax": custom(T=90, hidden_size=128, num_experts=256,
                                            num_experts_per_tok=8, moe_intermediate_size=64,
                                            num_shared_experts=0, n_group=8, topk_group=4,
                                            score_func="softmax", route_scale=2.5),
    "grouped_pairs_keep1": custom(T=33, hidden_size=64, num_experts=12, num_experts_per_tok=2,
                                  moe_intermediate_size=64, num_shared_experts=1, n_group=6,
                                  topk_group=1),
}


def _inputs(name):
    if name in EDGE:
        return synth.generate(EDGE[name])
    return generated(name)


def run_stages(dev: Dev, deterministic=False):
    """Every entry point called on its own, with explicit buffers."""
    c, T = dev.keys, dev.T
    E, k, H, I = c["num_experts"], c["num_experts_per_tok"], c["hidden_size"], c["moe_intermediate_size"]
    S = c["num_shared_experts"]
    Is = c["shared_intermediate_size"] or I
    f32, i32, dt = torch.float32, torch.int32, moe.torch_dtype(c)
    z = lambda n, d: torch.empty(max(n, 1), dtype=d, device="cuda")
    logits, idx, w, counts = z(T * E, f32), z(T * k, i32), z(T * k, f32), z(E, i32)
    offs, sr, rp = z(E + 1, i32), z(T * k, i32), z(T * k, i32)
    h, hs = z(T * k * I, dt), (z(T * S * Is, dt) if S else None)
    acc, out = z(T * H, f32), z(T * H, dt)
    yp = z(T * k * H, dt) if deterministic else None
    say(f"[stages] {c['hidden_size']}x{E}x{k} T={T} {c['dtype']}")
    moe.moe_router_logits(c, T, dev.x, dev.w_router, logits, dev.ws, mx=dev.mx)
    moe.moe_route(c, T, logits, dev.expert_bias, idx, w, counts)
    moe.moe_permute(c, T, idx, offs, sr, rp, dev.ws)
    moe.moe_grouped_gate_up_swiglu(c, T, dev.x, dev.w_gate, dev.w_up, dev.ws_gate, dev.ws_up,
                                   offs, sr, h, hs, dev.ws, mx=dev.mx)
    moe.moe_grouped_down(c, T, h, dev.w_down, hs, dev.ws_down, offs, sr, w, acc, yp, dev.ws,
                         mx=dev.mx)
    moe.moe_combine(c, T, acc, yp, rp, w, out)
    torch.cuda.synchronize()
    g = lambda t, *shape: t[: int(np.prod(shape))].view(*shape).float().cpu().numpy() \
        if t.dtype in (torch.bfloat16,) else t[: int(np.prod(shape))].view(*shape).cpu().numpy()
    return dict(logits=g(logits, T, E), idx=g(idx, T, k), w=g(w, T, k), counts=g(counts, E),
                offsets=g(offs, E + 1), sorted_rows=g(sr, T * k), row_pos=g(rp, T * k),
                h=g(h, T * k, I).astype(np.float64),
                h_shared=(g(hs, T, S * Is).astype(np.float64) if S else None),
                out=g(out, T, H).astype(np.float64))


def check_routing(cfg, inp, st):
    k = cfg["num_experts_per_tok"]
    s, keys, idx, w = O.route(st["logits"], inp.expert_bias, k, cfg["score_func"],
                              bool(cfg["route_norm"]), cfg["route_scale"],
                              cfg.get("n_group", 1), cfg.get("topk_group", 1))
    assert np.array_equal(st["idx"], idx), "routing indices differ from the oracle"
    assert np.max(np.abs(st["w"] - w) / np.maximum(np.abs(w), 1e-30)) <= 1e-6
    return s, keys, idx, w


@pytest.mark.parametrize("name", list(EDGE) + ["tiny_fp32_T64", "trinity_nano_decode_T32"])
def test_stages_match_oracle(name):
    inp = _inputs(name)
    cfg = inp.cfg
    dev = Dev(inp)
    for det in (False, True):
        st = run_stages(dev, deterministic=det)
        Lref = O.router_logits(inp.x, inp.w_router)
        assert rel_err(st["logits"], Lref) <= 1e-5
        check_routing(cfg, inp, st)
        counts, offsets, sr, rp = O.permute(st["idx"], cfg["num_experts"])
        assert np.array_equal(st["counts"], counts)
        assert np.array_equal(st["offsets"], offsets)
        assert np.array_equal(st["sorted_rows"], sr)
        assert np.array_equal(st["row_pos"], rp)
        ref = O.moe_forward(inp, cfg, logits=st["logits"], want_hidden=True)
        tol = TOL[cfg["dtype"]]
        assert rel_err(st["h"], ref["h"]) <= tol
        if ref["h_shared"] is not None:
            assert rel_err(st["h_shared"], ref["h_shared"]) <= tol
        e = rel_err(st["out"], ref["out"])
        say(f"[stages] {name} det={det} out rel err {e:.3e}")
        assert e <= tol


def test_clamp_is_exercised():
    """The clamp-SwiGLU case drives most gate/up pre-activations past the limit."""
    inp = _inputs("clamp_swigluoai")
    x = O.as_f64(inp.x)
    g = x @ O.as_f64(inp.w_gate[0]).T
    u = x @ O.as_f64(inp.w_up[0]).T
    frac = np.mean((g > 7.0) | (np.abs(u) > 7.0))
    assert frac > 0.5


@pytest.mark.parametrize("name", ["tiny_fp32_T64", "trinity_nano_decode_T32", "afmoe_default_T4096"])
def test_layer_forward_full(name):
    inp = generated(name)
    cfg = inp.cfg
    dev = Dev(inp)
    for det in (0, 1):
        say(f"[layer] {name} det={det}")
        res = dev.forward(deterministic=det)
        check_routing(cfg, inp, res)
        ref = O.moe_forward(inp, cfg, logits=res["logits"])
        e = rel_err(res["out"], ref["out"])
        say(f"[layer] {name} det={det} rel err {e:.3e}")
        assert e <= TOL[cfg["dtype"]]


def test_router_logits_in_path():
    inp = generated("trinity_nano_decode_T32")
    dev = Dev(inp)
    a = dev.forward(deterministic=1)
    L = torch.from_numpy(a["logits"]).cuda().reshape(-1)
    b = dev.forward(deterministic=1, logits_in=L, want_logits=False)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["out"], b["out"])


def test_deterministic_repeats_bitwise():
    inp = _inputs("e300_k8")
    dev = Dev(inp)
    a, b = dev.forward(deterministic=1), dev.forward(deterministic=1)
    assert np.array_equal(a["out"], b["out"])
    c = dev.forward(deterministic=0)
    assert np.array_equal(a["idx"], c["idx"]) and np.array_equal(a["w"], c["w"])


# (E, k): the k rounds of wave reductions (at most 64 tokens with sigmoid
# scores and E <= 256 select by ranks instead)
TIE_CASES = [(300, 8), (256, 8), (128, 8), (64, 6), (7, 3)]


@pytest.mark.parametrize("E,k", [(256, 8), (200, 32), (128, 8), (129, 4), (64, 6), (33, 1),
                                 (8, 8), (7, 3)])
def test_route_rank_selection_equals_the_rounds(E, k, monkeypatch):
    """The rank selection (one workgroup per token; decode-sized batches) and
    the k arg-max rounds (one wavefront per token) forced on the same
    logits, random and with exact ties: indices, weights and expert counts
    bitwise equal."""
    cfg = dict(synth.layer_keys(EDGE["e300_k8"]), num_experts=E, num_experts_per_tok=k)
    T = 97
    rng = np.random.default_rng(E * 31 + k)
    Lr = rng.standard_normal((T, E)).astype(np.float32) * 3
    Lt = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, E)).astype(np.float32)
    b = (rng.uniform(-0.05, 0.05, E)).astype(np.float32)
    for L in (Lr, Lt):
        res = []
        for knob in ("1", "0"):
            monkeypatch.setenv("MOE_ROUTE_RANK", knob)
            idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
            w = torch.empty(T * k, dtype=torch.float32, device="cuda")
            cnt = torch.empty(E, dtype=torch.int32, device="cuda")
            moe.moe_route(cfg, T, torch.from_numpy(L).cuda(), torch.from_numpy(b).cuda(), idx, w,
                          cnt)
            torch.cuda.synchronize()
            res.append((idx.cpu().numpy(), w.cpu().numpy(), cnt.cpu().numpy()))
        for a, b_ in zip(res[0], res[1]):
            assert np.array_equal(a, b_)
        _, _, ridx, _ = O.route(L, b, k, "sigmoid", True, cfg["route_scale"])
        assert np.array_equal(res[0][0].reshape(T, k), ridx)


@pytest.mark.parametrize("score_func", ["sigmoid", "softmax"])
@pytest.mark.parametrize("E,k", TIE_CASES)
def test_route_exact_ties_from_host_logits(E, k, score_func):
    """Host-built fp32 logits with exactly equal values: lowest index wins."""
    cfg = dict(synth.layer_keys(EDGE["e300_k8"]), num_experts=E, num_experts_per_tok=k,
               score_func=score_func)
    T = 64
    rng = np.random.default_rng(7)
    L = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, E)).astype(np.float32)
    b = np.zeros(E, np.float32)
    b[rng.choice(E, min(20, E // 2), replace=False)] = 0.25
    Ld = torch.from_numpy(L).cuda()
    bd = torch.from_numpy(b).cuda()
    idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, T, Ld, bd, idx, w)
    torch.cuda.synchronize()
    _, keys, ridx, rw = O.route(L, b, k, score_func, True, cfg["route_scale"])
    assert O.boundary_gap(keys, k) == 0.0
    assert np.array_equal(idx.view(T, k).cpu().numpy(), ridx)
    assert np.allclose(w.view(T, k).cpu().numpy(), rw, rtol=1e-6, atol=0)


@pytest.mark.parametrize("E,k,n_group,topk_group", [(256, 8, 8, 4), (64, 6, 8, 3), (12, 2, 6, 1),
                                                    (1024, 32, 64, 8), (96, 5, 32, 3)])
def test_route_grouped_exact_ties_from_host_logits(E, k, n_group, topk_group):
    """Host-built fp32 logits from four values, so keys and group scores tie
    exactly: the kept groups and the selection match the oracle bit for bit
    (lower group, then lower expert index, wins)."""
    cfg = dict(synth.layer_keys(EDGE["e300_k8"]), num_experts=E, num_experts_per_tok=k,
               n_group=n_group, topk_group=topk_group)
    T = 64
    rng = np.random.default_rng(E + k)
    L = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, E)).astype(np.float32)
    b = np.zeros(E, np.float32)
    b[rng.choice(E, min(20, E // 2), replace=False)] = 0.25
    idx = torch.empty(T * k, dtype=torch.int32, device="cuda")
    w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, T, torch.from_numpy(L).cuda(), torch.from_numpy(b).cuda(), idx, w)
    torch.cuda.synchronize()
    _, keys, ridx, rw = O.route(L, b, k, "sigmoid", True, cfg["route_scale"], n_group, topk_group)
    got = idx.view(T, k).cpu().numpy()
    assert np.array_equal(got, ridx)
    gs = E // n_group
    assert all(len({int(e) // gs for e in row}) <= topk_group for row in got)
    assert np.allclose(w.view(T, k).cpu().numpy(), rw, rtol=1e-6, atol=0)


def test_zero_tokens_is_a_no_op():
    cfg = synth.layer_keys(EDGE["one_token"])
    ws = moe.alloc_workspace(cfg, 1)
    out = torch.full((256,), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward(cfg, 0, out, None, None, out, out, out, out, out, out, None, None,
                          None, None, out, 0, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


@pytest.mark.parametrize("name", ["many_experts_k32", "one_token", "one_expert",
                                  "k_eq_E_no_shared", "fp32_ragged", "clamp_swigluoai",
                                  "softmax_norm", "m2_shape_softmax_nonorm"])
def test_layer_forward_small_batches(name):
    """T*k <= 1024: the layer routes and groups in one workgroup; indices must
    match the oracle bit for bit and the output the layer's bar, in both
    combine modes."""
    inp = _inputs(name)
    cfg = inp.cfg
    assert inp.x.shape[0] * cfg["num_experts_per_tok"] <= 1024
    dev = Dev(inp)
    for det in (1, 0):
        res = dev.forward(deterministic=det)
        check_routing(cfg, inp, res)
        ref = O.moe_forward(inp, cfg, logits=res["logits"])
        e = rel_err(res["out"], ref["out"])
        say(f"[small] {name} det={det} rel err {e:.3e}")
        assert e <= TOL[cfg["dtype"]]


@pytest.mark.parametrize("E,k", TIE_CASES)
def test_layer_forward_exact_ties_small_batch(E, k):
    """Host-built logits with exactly equal values through the single entry
    point at a decode-sized batch (64 tokens): lowest index wins, indices in
    selection order."""
    cfg = dict(EDGE["e300_k8"], num_experts=E, num_experts_per_tok=k)
    inp = synth.generate(cfg, T=64)
    dev = Dev(inp)
    T = 64
    rng = np.random.default_rng(11)
    L = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, E)).astype(np.float32)
    b = np.zeros(E, np.float32)
    b[rng.choice(E, min(20, E // 2), replace=False)] = 0.25
    dev.expert_bias = torch.from_numpy(b).cuda()
    Ld = torch.from_numpy(L).cuda().reshape(-1)
    res = dev.forward(deterministic=1, logits_in=Ld, want_logits=False)
    _, keys, ridx, rw = O.route(L, b, k, "sigmoid", True, synth.layer_keys(cfg)["route_scale"])
    assert O.boundary_gap(keys, k) == 0.0
    assert np.array_equal(res["idx"], ridx)
    assert np.allclose(res["w"], rw, rtol=1e-6, atol=0)


@pytest.mark.parametrize("T,H,E", [(40, 2048, 64), (127, 1472, 33), (5, 64, 8)])
def test_small_batch_router_planes(T, H, E):
    """Batches under 128 tokens: the router leaves one partial plane per
    64-input group (32 planes at H=2048, 23 at H=1472, one at H=64) and the
    single entry point's routing kernel sums them in plane order, the router
    entry point's reduce kernel likewise: the two logit arrays agree bit for
    bit, match the float64 oracle, two identical router rows give identical
    logit columns, and routing matches the oracle on those logits."""
    cfg = custom(T=T, hidden_size=H, num_experts=E, num_experts_per_tok=4,
                 moe_intermediate_size=64, num_shared_experts=1)
    inp = synth.generate(cfg)
    inp.w_router[E - 1] = inp.w_router[3]  # a duplicated router row
    dev = Dev(inp)
    res = dev.forward(deterministic=1)
    logits = torch.empty(T * E, dtype=torch.float32, device="cuda")
    moe.moe_router_logits(dev.keys, T, dev.x, dev.w_router, logits, dev.ws)
    torch.cuda.synchronize()
    L = logits.view(T, E).cpu().numpy()
    assert np.array_equal(res["logits"], L)
    assert rel_err(L, O.router_logits(inp.x, inp.w_router)) <= 1e-5
    assert np.array_equal(L[:, 3], L[:, E - 1])
    check_routing(cfg, inp, res)
