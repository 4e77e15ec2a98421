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
