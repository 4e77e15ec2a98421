"""Host-side logic of bench.py (no GPU): the algorithmic FLOPs and bytes the
roofline divides by, the routing report, kernel-name shortening of profiler
output, the HBM traffic summary built from PMC counter files (calibration
scaling included) and its source fingerprint, and the one-GPU contract."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_formulas_by_hand():
    cfg = dict(hidden_size=64, num_experts=4, num_experts_per_tok=2, moe_intermediate_size=32,
               num_shared_experts=1, shared_intermediate_size=16, dtype="bf16",
               weight_format="dtype")
    T = 3
    idx = np.array([[0, 1], [1, 2], [0, 2]])          # experts 0, 1, 2 touched (3 of 4)
    a = bench.algorithmic(cfg, T, idx)
    H, E, k, I, S, Is = 64, 4, 2, 32, 1, 16
    assert a["flops"] == T * (2 * H * E + 6 * k * H * I + 6 * S * H * Is)
    assert a["touched"] == 3
    assert a["bytes"] == 3 * 3 * H * I * 2 + S * 3 * H * Is * 2 + 4 * E * H + 2 * T * H * 2 + 4 * E
    assert a["gate_up_flops"] == 4 * T * H * (k * I + S * Is)
    # MX weights: codes plus one scale byte per 32 weights
    a8 = bench.algorithmic(dict(cfg, weight_format="mxfp8"), T, idx)
    a4 = bench.algorithmic(dict(cfg, weight_format="mxfp4"), T, idx)
    w = 3 * 3 * H * I + S * 3 * H * Is                 # weights moved
    assert a8["bytes"] - a4["bytes"] == pytest.approx(w * 0.5)
    assert a["bytes"] - a8["bytes"] == pytest.approx(w * (2 - 1 - 1 / 32))


def test_routing_report_by_hand():
    cfg = dict(num_experts=4, num_experts_per_tok=2)
    # token 0: keys sigmoid(0) + b = 0.5 each for experts 0 and 3 with bias 0,
    # expert 1 higher: top-2 = {1, 0 or 3}; the 2nd and 3rd keys tie exactly
    L = np.array([[0.0, 2.0, -3.0, 0.0], [4.0, -1.0, 3.0, -2.0]], np.float32)
    idx = np.array([[1, 0], [0, 2]])
    r = bench.routing_report(cfg, idx, L, np.zeros(4, np.float32))
    assert r["touched_experts"] == 3 and r["empty_experts"] == 1
    assert r["max_rows"] == 2 and r["mean_rows"] == 1.0
    assert r["top10pct_share"] == 0.5                  # the top max(1, E // 10) = 1 expert: 2 of 4 rows
    assert r["boundary_key_gap"]["tied_tokens"] == 1 and r["boundary_key_gap"]["min"] == 0.0
    s = 1 / (1 + np.exp(-np.array([4.0, 3.0, -1.0])))
    r2 = bench.routing_report(cfg, idx[1:], L[1:], np.zeros(4, np.float32))
    assert r2["boundary_key_gap"]["min"] == pytest.approx(s[1] - s[2], rel=1e-12)


@pytest.mark.parametrize("name,short", [
    ("_ZN12_GLOBAL__N_118moe_gate_up_kernelIDF16bLi0EEEv8GemmArgs", "moe_gate_up_kernel"),
    ("_Z25moe_gate_up_decode_kernelILi3ELi4EEv8GemmArgs", "moe_gate_up_decode_kernel"),
    ("void (anonymous namespace)::moe_down_kernel<__bf16, 0>(GemmArgs)", "moe_down_kernel"),
    ("combine_kernel(float const*, void const*)", "combine_kernel"),
])
def test_kernel_name_shortening(name, short):
    assert bench._short(name) == short


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_summary_scaling_and_fingerprint(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled so that a plain copy of
    256 MiB reads and writes 256 MiB; records carry the GEMM sources'
    fingerprint and are ignored once it changes."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    d = tmp_path / "run"
    kern = "_Z18moe_gate_up_kernelIDF16bLi0EEv8GemmArgs"
    line = {"roofline": {"kernel": "moe_gate_up_kernel"},
            "layer": {"gate_up_bytes": 1000 * 1024},
            "config": {"workload": "wl"}}
    os.makedirs(d)
    (d / "bench.json").write_text(json.dumps(line) + "\n")
    _counter_csv(d / "pmc_FETCH_SIZE", [(kern, "FETCH_SIZE", 900), (kern, "FETCH_SIZE", 1100)])
    _counter_csv(d / "pmc_WRITE_SIZE", [(kern, "WRITE_SIZE", 100)])
    copy = "__amd_rocclr_copyBuffer"
    _counter_csv(d / "cal_FETCH_SIZE", [(copy, "FETCH_SIZE", 131072)])    # half of 256 MiB
    _counter_csv(d / "cal_WRITE_SIZE", [(copy, "WRITE_SIZE", 262144)])
    monkeypatch.setattr(bench, "gemm_source_sha", lambda: "sha-a")
    text = bench.summarize_traffic(str(d))
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))["records"][0]
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (1000 * 2 + 100) * 1024
    assert "ratio 2.10" in text
    assert bench.traffic_from_profile("moe_gate_up_kernel", "wl", "sha-a") == rec["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile("moe_gate_up_kernel", "wl", "sha-b") is None
    assert bench.traffic_from_profile("moe_gate_up_kernel", "other", "sha-a") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_layer_report_prices_prefill_on_mfma_and_decode_on_hbm():
    """The roofline object of a prefill-sized batch is the gate/up kernel
    against the bf16 MFMA peak; a decode-sized batch (at most 32 rows per
    expert on average) against HBM; achieved = algorithmic work / the
    kernel's mean time."""
    from workloads import synth
    m = dict(ms=2.0, ms_min=1.9, ms_max=2.2, ms_warm=1.8, ms_write_flush=2.5, ms_graph=None,
             roof_mean_ms=1.0, roof_stage="gate_up", stage_ms={"gate_up": 1.0})
    for name, bound in (("minimax_m3_prefill_T8192", "mfma"), ("minimax_m3_decode_T64", "hbm"),
                        ("trinity_nano_decode_T32", "hbm")):
        cfg = synth.config(name)
        T, E, k = cfg["T"], cfg["num_experts"], cfg["num_experts_per_tok"]
        idx = (np.arange(T * k).reshape(T, k) % E).astype(np.int64)
        L = np.zeros((T, E), np.float32)
        layer, roof = bench.layer_report(name, cfg, T, m, idx, L, np.zeros(E, np.float32), 5)
        alg = bench.algorithmic(cfg, T, idx)
        assert roof["bound"] == bound and layer["bound"] == bound
        if bound == "mfma":
            assert roof["achieved"] == pytest.approx(alg["gate_up_flops"] / 1e-3 / 1e12)
            assert roof["peak"] == bench.PEAK_BF16_TFLOPS and roof["unit"] == "TFLOP/s"
        else:
            assert roof["achieved"] == pytest.approx(alg["gate_up_bytes"] / 1e-3 / 1e9)
            assert roof["peak"] == bench.PEAK_HBM_GBS and roof["unit"] == "GB/s"
        assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
        assert layer["frac_hbm_peak"] == pytest.approx(alg["bytes"] / 2e-3 / 1e9 / 8000.0)
        assert layer["frac_bf16_peak"] == pytest.approx(alg["flops"] / 2e-3 / 1e12 / 2516.6)


def test_fused_ffn_roofline():
    """Where the stage-call pass ran the fused decode FFN, the roofline object
    is that kernel against HBM, over every touched and shared expert weight,
    x and the fp32 partial planes."""
    from workloads import synth
    cfg = synth.config("trinity_nano_decode_T32")
    T, E, k, H = cfg["T"], cfg["num_experts"], cfg["num_experts_per_tok"], cfg["hidden_size"]
    I, Is = cfg["moe_intermediate_size"], cfg["shared_intermediate_size"]
    idx = (np.arange(T * k).reshape(T, k) % E).astype(np.int64)
    m = dict(ms=2.0, ms_min=1.9, ms_max=2.2, ms_warm=1.8, ms_write_flush=2.5, ms_graph=None,
             roof_mean_ms=0.5, roof_stage="ffn", stage_ms={"ffn": 0.5})
    layer, roof = bench.layer_report("trinity_nano_decode_T32", cfg, T, m, idx,
                                     np.zeros((T, E), np.float32), np.zeros(E, np.float32), 5)
    touched = len(np.unique(idx))
    want = (touched * 3 * H * I * 2 + 3 * H * Is * 2 + T * H * 2
            + 4 * H * (I // 128 * T * k + Is // 128 * T))
    assert roof["kernel"] == "moe_ffn_decode_kernel" and roof["bound"] == "hbm"
    assert roof["algorithmic_bytes"] == want
    assert roof["achieved"] == pytest.approx(want / 0.5e-3 / 1e9)


def test_gate_up_kernel_names_follow_the_library_selection():
    """The roofline kernel's name: 32-row tiles for decode-sized batches,
    256-row tiles for bf16 batches with >= 384 rows per expert and H, I >=
    1024, else the 128-row tiles (the selection in the library's API)."""
    from workloads import synth
    want = {"minimax_m3_prefill_T8192": "moe_gate_up_kernel",
            "minimax_m3_decode_T64": "moe_gate_up_decode_kernel",
            "trinity_nano_decode_T32": "moe_gate_up_decode_kernel",
            "trinity_nano_prefill_T8192": "moe_gate_up_kernel",
            "afmoe_default_T4096": "moe_gate_up_wide_kernel",
            "skewed_afmoe_T8192": "moe_gate_up_wide_kernel",
            "minimax_m3_prefill_T8192_mxfp8": "moe_gate_up_kernel"}
    for name, kern in want.items():
        cfg = synth.config(name)
        assert bench.gate_up_kernel(cfg, cfg["T"]) == kern, name
    assert bench._short("(anonymous namespace)::moe_gate_up_wide_kernel(GemmArgs)") == \
        "moe_gate_up_wide_kernel"
