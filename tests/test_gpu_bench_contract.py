"""The bench's JSON line (the contract its callers read): run bench.py with
its defaults (the MiniMax-M3-shaped T=8192 headline, the two decode layers
nested) with few steps and a small CPU sample, and check every field: the
metric and its unit, one GPU, the timed steps, the dtype, the workload
config, the roofline object of the dominant kernel (bound, achieved, peak,
frac; the HBM traffic from the committed counter summaries when they match
the current GEMM sources, else null), each decode layer's own HBM roofline,
and the CPU baseline (the oracle)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check_roofline(rf, bound):
    assert rf["bound"] == bound
    assert rf["unit"] == ("TFLOP/s" if bound == "mfma" else "GB/s")
    assert rf["peak"] == (2516.6 if bound == "mfma" else 8000.0)
    assert 0 < rf["achieved"] and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rf["traffic"] is None or rf["traffic"] > 0
    assert rf["ms_per_launch"] > 0


def test_bench_json_line():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
           "--cpu-sample", "16", "--no-block"]
    print(f"[bench-contract] running {' '.join(cmd[2:])}", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=400, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    L = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "decode", "layer"):
        assert key in L, key
    assert L["n_gpus"] == 1 and L["steps"] == 2 and L["warmup"] == 1
    assert L["unit"] == "tokens/s" and L["value"] > 0 and L["higher_is_better"] is True
    assert L["dtype"] == "bf16" and L["config"]["workload"] == "minimax_m3_prefill_T8192"
    assert L["value"] == pytest.approx(8192 / (L["ms_per_step"] * 1e-3), rel=1e-6)
    assert L["layer"]["ms_median"] == L["ms_per_step"]
    assert L["layer"]["ms_min"] <= L["ms_per_step"] <= L["layer"]["ms_max"]
    _check_roofline(L["roofline"], "mfma")
    assert L["roofline"]["kernel"] == "moe_gate_up_kernel"
    dec = L["decode"]
    assert set(dec) == {"minimax_m3_decode_T64", "trinity_nano_decode_T32"}
    for name, T in (("minimax_m3_decode_T64", 64), ("trinity_nano_decode_T32", 32)):
        d = dec[name]
        assert d["steps"] == 10
        assert d["tokens_per_s"] == pytest.approx(T / (d["ms_per_step"] * 1e-3), rel=1e-6)
        assert 0 < d["layer"]["frac_hbm_peak"] < 1.0
        _check_roofline(d["roofline"], "hbm")
        # the Trinity-like layer takes the fused decode FFN
        want = "moe_ffn_decode_kernel" if name == "trinity_nano_decode_T32" else \
            "moe_gate_up_decode_kernel"
        assert d["roofline"]["kernel"] == want
    cb = L["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == "tokens/s"
    print(f"[bench-contract] {L['value']:.4g} tokens/s, roofline frac {L['roofline']['frac']:.3f}, "
          f"decode HBM {dec['minimax_m3_decode_T64']['layer']['frac_hbm_peak']:.3f} / "
          f"{dec['trinity_nano_decode_T32']['layer']['frac_hbm_peak']:.3f}", flush=True)
