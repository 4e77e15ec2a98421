"""The bench's JSON line (the contract its callers read): run bench.py on the
default workload with few steps and a small CPU sample, and check every
field: the metric and its unit, one GPU, the timed steps, the dtype, the
workload config, the roofline object of the dominant kernel (bound, achieved,
peak, frac, and the HBM traffic from the committed counter summaries, which
match the current GEMM sources) and the CPU baseline (the oracle)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[bench-contract] running bench.py --steps 3 --warmup 1 --cpu-sample 256", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--cpu-sample", "256"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    L = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in L, key
    assert L["n_gpus"] == 1 and L["steps"] == 3 and L["warmup"] == 1
    assert L["unit"] == "tokens/s" and L["value"] > 0 and L["higher_is_better"] is True
    assert L["dtype"] == "bf16" and L["config"]["workload"] == "afmoe_default_T4096"
    assert L["value"] == pytest.approx(4096 / (L["ms_per_step"] * 1e-3), rel=1e-6)
    rf = L["roofline"]
    assert rf["bound"] in ("mfma", "hbm") and rf["unit"] in ("TFLOP/s", "GB/s")
    assert 0 < rf["achieved"] and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rf["traffic"] is not None and rf["traffic"] > 0, "traffic records do not match the sources"
    cb = L["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == "tokens/s"
    print(f"[bench-contract] {L['value']:.4g} tokens/s, roofline frac {rf['frac']:.3f}", flush=True)
