"""The seeded generator: deterministic, per-block streams (a smaller T is a
prefix of a larger one), bf16 rounding to nearest-even (checked against
torch's float32 -> bfloat16 conversion), and the skewed workload's stored
parameters."""
import numpy as np
import pytest
import torch

from workloads import synth


def test_generation_is_deterministic_and_prefix_stable():
    cfg = synth.config("trinity_nano_decode_T32")
    a = synth.generate(cfg, experts=False)
    b = synth.generate(cfg, experts=False)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_router, b.w_router)
    big = synth.generate(cfg, T=300, experts=False)
    assert np.array_equal(big.x[:32], a.x)


def test_bf16_rounding_matches_torch():
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    ours = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_value_ranges():
    cfg = synth.config("tiny_fp32_T64")
    inp = synth.generate(cfg)
    assert np.all(np.abs(inp.expert_bias) <= 0.1)
    assert abs(float(inp.w_gate.std()) - 0.02) < 0.002
    assert abs(float(inp.x.std()) - 1.0) < 0.05


def test_skew_parameters_are_applied():
    cfg = synth.config("skewed_afmoe_T8192")
    sk = synth.load_skew(cfg["skew"])
    base = synth.generate(cfg, T=256, experts=False, apply_skew=False)
    inp = synth.generate(cfg, T=256, experts=False)
    a, c = sk["tie_pair"]
    assert np.array_equal(inp.w_router[c], inp.w_router[a])
    assert inp.expert_bias[c] == inp.expert_bias[a]
    hot = np.array(sk["hot_experts"])
    assert np.all(inp.expert_bias[hot] > base.expert_bias[hot])
    assert abs(sk["hot_share"] - 0.60) <= 0.01
    assert 0.03 <= sk["tie_straddle_rate"] <= 0.07


def test_mxfp8_quantiser():
    """Scales follow the OCP MX rule 2^(floor(log2 amax) - 8); codes are the
    round-to-nearest-even E4M3 cast (torch's) of the clamped scaled values;
    the MXFP8 workload draws the same fp32 weights as the bf16 one."""
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
    w[3, 32:64] = 0.0                                   # an all-zero block
    # blocks with scale 2^0 (maximum 448): every non-negative E4M3 value up to
    # code 0x3E (subnormals included), then the midpoints between neighbours
    # (exact ties: the even code wins) and values just off them
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    w[7, :32] = np.concatenate([[448.0], vals[:31]])
    w[7, 32:64] = np.concatenate([[448.0], vals[31:62]])
    w[8, :32] = np.concatenate([[448.0], (vals[:31] + vals[1:32]) / 2])
    w[8, 32:64] = np.concatenate([[448.0], np.nextafter((vals[:31] + vals[1:32]) / 2, 1)])
    w[8, 64:96] = -w[8, :32]
    codes, sc = synth.quantize_mxfp8(w)
    assert codes.shape == w.shape and sc.shape == (8, 48) and sc.dtype == np.uint8
    amax = np.abs(w.astype(np.float64)).reshape(48, 8, 32).max(2)
    nz = amax > 0
    assert np.array_equal(sc.T[nz].astype(np.int64), np.floor(np.log2(amax[nz])).astype(np.int64) - 8 + 127)
    v = w.astype(np.float64).reshape(48, 8, 32) / np.exp2(sc.T.astype(np.float64) - 127)[:, :, None]
    ref = torch.from_numpy(np.clip(v, -448, 448).reshape(48, 256)).to(torch.float8_e4m3fn)
    assert np.array_equal(ref.view(torch.uint8).numpy(), codes)
    assert np.array_equal(codes[7, 1:32], np.arange(31)) and np.all(codes[8, 1:32] % 2 == 0)
    assert np.all(codes[3, 32:64] & 0x7F == 0)
    cfg = synth.config("trinity_nano_decode_T32_mxfp8")
    a = synth.generate(cfg)
    b = synth.generate(synth.config("trinity_nano_decode_T32"))
    assert np.array_equal(a.x, b.x) and a.mx["down"].shape == (128, 256 // 32, 1024)
    # expert 5's gate matrix is the quantised fp32 draw of its own stream
    tmp = np.empty((256, 1024), np.float32)
    synth._fill_normal(tmp, synth._stream(0, synth.TID_GATE, 5), cfg["w_std"], False)
    assert np.array_equal(synth.f32_to_bf16_bits(tmp), b.w_gate[5])
    g, gs = synth.quantize_mxfp8(tmp)
    assert np.array_equal(a.w_gate[5], g) and np.array_equal(a.mx["gate"][5], gs)


def test_mxfp4_quantiser():
    """OCP rule (scale 2^(floor(log2 amax) - 2), clamp to +-6, nearest E2M1
    value, ties to the even code) against the hand-worked block and against
    a brute-force nearest-value search; input 2j in the low nibble."""
    import json
    import os
    from oracle import moe_oracle as O
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "mxfp4_hand_example.json")))["quantise"]
    w = np.zeros((1, 32), np.float32)
    w[0, :5] = g["inputs"]
    p, sc = synth.quantize_mxfp4(w)
    assert p.shape == (1, 16) and sc.shape == (1, 1) and sc[0, 0] == g["scale_byte"]
    codes = O.unpack_fp4(p)[0]
    assert [int(c) for c in codes[:5]] == [int(c, 16) for c in g["codes"]]
    assert np.all(codes[5:] == 0)

    rng = np.random.default_rng(3)
    w = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    w[2, 64:96] = 0.0                                   # an all-zero block
    w[5, 0:32] = 7.0                                    # saturates: amax 7 -> scale 1, 7 -> 6
    w[5, 0] = 6.0
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (mags[1:] + mags[:-1]) / 2
    w[6, 0:8] = np.r_[6.0, mids]                         # every tie, scale 2^0
    w[6, 8:16] = -np.r_[mids[:7], 0.0]
    p, sc = synth.quantize_mxfp4(w)
    assert p.shape == (24, 128) and sc.shape == (8, 24)
    amax = np.abs(w.astype(np.float64)).reshape(24, 8, 32).max(2)
    nz = amax > 0
    assert np.array_equal(sc.T[nz].astype(np.int64),
                          np.floor(np.log2(amax[nz])).astype(np.int64) - 2 + 127)
    assert np.all(sc.T[~nz] == 0)
    v = w.astype(np.float64).reshape(24, 8, 32) / np.exp2(sc.T.astype(np.float64) - 127)[:, :, None]
    a = np.minimum(np.abs(v), 6.0)
    dist = np.abs(a[..., None] - mags)
    best = dist.min(-1, keepdims=True)
    cand = dist == best                                  # one or two nearest codes
    even = cand & (np.arange(8) % 2 == 0)
    ref = np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1))
    ref = (ref | np.where(np.signbit(v), 8, 0)).reshape(24, 256)
    got = O.unpack_fp4(p)
    assert np.array_equal(got, ref)
    assert np.all(got[5, :32] & 7 == 7)
    cfg = synth.config("trinity_nano_decode_T32_mxfp4")
    a4 = synth.generate(cfg)
    a8 = synth.generate(synth.config("trinity_nano_decode_T32_mxfp8"))
    assert np.array_equal(a4.x, a8.x) and a4.w_gate.shape == (128, 256, 512)
    assert a4.mx["down"].shape == (128, 256 // 32, 1024) and a4.ws_down.shape == (1, 1024, 128)
    tmp = np.empty((256, 1024), np.float32)
    synth._fill_normal(tmp, synth._stream(0, synth.TID_GATE, 5), cfg["w_std"], False)
    q, qs = synth.quantize_mxfp4(tmp)
    assert np.array_equal(a4.w_gate[5], q) and np.array_equal(a4.mx["gate"][5], qs)


def test_mxfp8_router_is_the_quantised_fp32_router():
    """The 8-bit router of the q4r8 workloads is the MXFP8 quantisation of the
    same fp32 draw the fp32-router workload uses; the oracle refuses raw
    codes (they have no value without their scales)."""
    from oracle import moe_oracle as O
    a = synth.generate(synth.config("trinity_nano_decode_T32_q4r8"))
    b = synth.generate(synth.config("trinity_nano_decode_T32_mxfp4"))
    codes, sc = synth.quantize_mxfp8(b.w_router)
    assert np.array_equal(a.w_router, codes) and np.array_equal(a.mx["router"], sc)
    assert np.array_equal(a.w_gate, b.w_gate) and np.array_equal(a.x, b.x)
    with pytest.raises(ValueError):
        O.as_f64(a.w_router)
    wr = O.mx_dequantize(a.w_router, a.mx["router"])
    # within MXFP8's error on the fp32 draw: half a step of 3 mantissa bits
    # (2^-4 of an element), or the OCP rule's clip of a block maximum that
    # lands in (448, 512) x scale to 448 (at most 1/8 of the block maximum)
    w64 = b.w_router.astype(np.float64)
    blk_max = np.abs(w64).reshape(128, -1, 32).max(2, keepdims=True)
    err = np.abs(wr - w64).reshape(128, -1, 32)
    assert np.all(err <= np.maximum(np.abs(w64).reshape(128, -1, 32) * 2.0 ** -4, blk_max / 8))
