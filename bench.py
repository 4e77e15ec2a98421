"""Benchmark of the sparse-MoE feed-forward layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer (router GEMM, routing, grouping,
gate/up + activation, down + combine, output cast) over one batch of seeded
synthetic inputs that are resident in HBM before timing starts, through the
layer's single entry point moe_layer_forward on one stream.

Timing protocol (every timed number): W untimed warm-up steps, then K timed
steps; before each timed step a 1 GiB buffer (more than the 256 MB MALL) is
written and then read back, outside the timed events, so expert weights come
from HBM as they do in a many-layer model (the read-back leaves the caches
holding clean lines, as the previous layers' weight reads would: after the
write alone, the layer's reads would also pay for writing the flush's dirty
lines back, reported beside it as the write-only figure); HIP events on the
layer's stream bracket the layer call alone, and the step time is the median
of the K (min and max beside it). The K timed steps are bracketed by device
synchronisation. The per-stage breakdown comes from a second pass over the
stage entry points with the same flushes and HIP events around each call.

By default the headline is the MiniMax-M3-shaped layer at T = 8192 (the
prefill target, MFMA-bound), and the same JSON line carries the two decode
layers (MiniMax-M3-shaped at T = 64, Trinity-like at T = 32; HBM-bound),
each with its own roofline object; --workload NAME benches one workload.

Prints ONE JSON line: tokens/s of the layer, its TFLOP/s (fraction of bf16
MFMA peak) and GB/s (fraction of HBM peak), the roofline of the dominant
kernel, and the float64 CPU oracle timed on a bounded sample of the same
workload (a baseline, not the target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE-layer tokens/s + % bf16 MFMA peak (prefill) / % HBM GB/s (decode) "
          "on 1 MI355X")
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz (dense)
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "minimax_m3_prefill_T8192"
# decode layers carried in the default line; the M3 decode batch is the first
# 64 tokens of the M3 prefill batch (same weights)
DECODE_WORKLOADS = ("minimax_m3_decode_T64", "trinity_nano_decode_T32")
FLUSH_BYTES = 1 << 30


def algorithmic(cfg: dict, T: int, idx: np.ndarray | None):
    """FLOPs and HBM bytes the layer must move (not padded or re-read work).
    F = T*(2HE + 6kHI + 6 S H Is); B = touched experts' weights + shared
    weights + router + x + out."""
    H, E, k = cfg["hidden_size"], cfg["num_experts"], cfg["num_experts_per_tok"]
    I, S = cfg["moe_intermediate_size"], cfg["num_shared_experts"]
    Is = cfg["shared_intermediate_size"] or I
    bx = 2 if cfg["dtype"] == "bf16" else 4
    # bytes per expert weight: MX codes plus one E8M0 scale byte per 32
    bw = {"mxfp8": 1 + 1 / 32, "mxfp4": 0.5 + 1 / 32}.get(cfg.get("weight_format"), bx)
    flops = T * (2 * H * E + 6 * k * H * I + 6 * S * H * Is)
    touched = E if idx is None else int(np.unique(idx).size)
    bytes_ = touched * 3 * H * I * bw + S * 3 * H * Is * bw + 4 * E * H + 2 * T * H * bx + 4 * E
    gate_up_flops = 4 * T * H * (k * I + S * Is)
    gate_up_bytes = touched * 2 * H * I * bw + S * 2 * H * Is * bw + T * H * bx \
        + (T * k * I + T * S * Is) * bx
    # the fused decode FFN: every weight of the touched and shared experts, x,
    # and its fp32 partial planes (one per 128-column slice of I and I_s)
    ffn_flops = 6 * T * H * (k * I + S * Is)
    ffn_bytes = touched * 3 * H * I * bw + S * 3 * H * Is * bw + T * H * bx \
        + 4 * H * (I // 128 * T * k + S * Is // 128 * T)
    return dict(flops=flops, bytes=bytes_, touched=touched, gate_up_flops=gate_up_flops,
                gate_up_bytes=gate_up_bytes, ffn_flops=ffn_flops, ffn_bytes=ffn_bytes)


GEMM_SOURCES = ("moe_gemm.hip", "moe_gemm_wide.hip", "moe_gemm_decode.hip", "moe_gemm_common.h",
                "moe_common.h", "moe_kernels.h", "moe_small_sort.h")


def gate_up_kernel(cfg: dict, T: int) -> str:
    """Name of the grouped gate/up kernel the library runs for this workload
    (the 32-row tile kernel for decode-sized batches; the 256-row one for
    bf16 batches with at least 384 rows per expert and H, I >= 1024; else the
    128-row one)."""
    H, I, k, E = cfg["hidden_size"], cfg["moe_intermediate_size"], cfg["num_experts_per_tok"], \
        cfg["num_experts"]
    S, Is = cfg["num_shared_experts"], cfg["shared_intermediate_size"] or I
    fits = H % 256 == 0 and I % 256 == 0 and (S * Is) % 256 == 0
    dec = cfg["dtype"] == "bf16" and fits and T * k <= 32 * E
    if dec:
        return "moe_gate_up_decode_kernel"
    wide = (cfg["dtype"] == "bf16" and cfg.get("weight_format", "dtype") == "dtype"
            and T * k >= 384 * E and H >= 1024 and I >= 1024)
    return "moe_gate_up_wide_kernel" if wide else "moe_gate_up_kernel"


def gemm_source_sha() -> str:
    """Fingerprint of the grouped-GEMM kernel's sources (a traffic figure taken
    on other sources is stale)."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_moe_transformer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic_records() -> list:
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            return json.load(f).get("records", [])
    except (OSError, ValueError):
        return []


def routing_report(cfg: dict, idx: np.ndarray, logits: np.ndarray, bias: np.ndarray) -> dict:
    """What the routing did on this batch (from the GPU's own outputs): the
    expert-load histogram in summary, and the smallest gap between the k-th
    and (k+1)-th selection key of any token (keys formed in float64 from the
    fp32 logits, as the selection does; zero means an exact tie at the
    boundary, decided by the lower index). With group-limited routing the gap
    is that of the ungrouped keys."""
    E, k = cfg["num_experts"], cfg["num_experts_per_tok"]
    T = idx.shape[0]
    counts = np.bincount(idx.reshape(-1), minlength=E)
    L = logits.astype(np.float64)
    with np.errstate(over="ignore"):  # exp(-L) -> inf gives the exact score 0
        if cfg.get("score_func", "sigmoid") == "softmax":
            z = np.exp(L - L.max(axis=1, keepdims=True))
            sc = z / z.sum(axis=1, keepdims=True)
        else:
            sc = 1.0 / (1.0 + np.exp(-L))
    keys = sc + bias.astype(np.float64)[None, :]
    gap = None
    if k < E and T:
        part = -np.sort(-keys, axis=1)[:, k - 1:k + 1]
        g = part[:, 0] - part[:, 1]
        gap = {"min": float(g.min()), "tied_tokens": int((g == 0).sum())}
    order = np.sort(counts)[::-1]
    n10 = max(1, E // 10)
    return {"touched_experts": int((counts > 0).sum()), "empty_experts": int((counts == 0).sum()),
            "max_rows": int(counts.max()), "mean_rows": T * k / E,
            "top10pct_share": float(order[:n10].sum() / max(1, T * k)),
            "boundary_key_gap": gap}


def traffic_from_profile(kernel: str, workload: str, src_sha: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed PMC
    summaries, or None if there is none or it was taken on other sources."""
    for rec in _traffic_records():
        if (rec.get("kernel"), rec.get("workload"), rec.get("source_sha256")) == \
                (kernel, workload, src_sha):
            return rec.get("hbm_bytes_per_launch")
    return None


# ---------------------------------------------------------------------------
# rocprofv3 summaries (no GPU needed): the text files under profiles/

def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name: str) -> str:
    """Kernel name without template arguments and parameter list."""
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    n = n.split("(")[0].split("<")[0].strip()
    if n.startswith("_ZN12_GLOBAL__N_1"):  # mangled, anonymous namespace
        n = "_Z" + n[len("_ZN12_GLOBAL__N_1"):]
    if n.startswith("_Z"):  # mangled: _Z<len><name>...
        i = 2
        while i < len(n) and n[i].isdigit():
            i += 1
        ln = int(n[2:i]) if i > 2 else 0
        n = n[i:i + ln] if ln else n
    return n


def summarize_trace(d: str) -> str:
    """Markdown table of a `rocprofv3 --kernel-trace --stats` run (per kernel:
    calls, average / min / max duration, share of GPU time)."""
    rows = _csv_rows(d, "kernel_stats.csv")
    agg = {}
    for r in rows:
        k = _short(r["Name"])
        a = agg.setdefault(k, [0, 0.0, float("inf"), 0.0])
        a[0] += int(r["Calls"])
        a[1] += float(r["TotalDurationNs"])
        a[2] = min(a[2], float(r["MinNs"]))
        a[3] = max(a[3], float(r["MaxNs"]))
    total = sum(a[1] for a in agg.values()) or 1.0
    out = ["| kernel | calls | avg us | min us | max us | share of GPU time |",
           "|---|---|---|---|---|---|"]
    for k, a in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| {k} | {a[0]} | {a[1] / a[0] / 1e3:.1f} | {a[2] / 1e3:.1f} | "
                   f"{a[3] / 1e3:.1f} | {100 * a[1] / total:.1f}% |")
    return "\n".join(out)


def _pmc_means(d: str, counter: str) -> dict:
    """Mean value of one PMC counter per kernel (short name) over dispatches."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_traffic(d: str, kernel: str | None = None) -> str:
    """HBM traffic per launch from two `rocprofv3 --pmc` runs of the bench
    (FETCH_SIZE and WRITE_SIZE, KiB per dispatch) scaled by what the same
    counters read for a plain copy of known size; writes profiles/traffic.json
    for the bench's roofline object and returns a markdown summary. Expects
    d/bench.json (the bench line of the same workload), d/pmc_FETCH_SIZE,
    d/pmc_WRITE_SIZE, d/cal_FETCH_SIZE, d/cal_WRITE_SIZE (rocprofv3 outputs)."""
    with open(os.path.join(d, "bench.json")) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    kernel = kernel or line["roofline"]["kernel"]
    fetch = _pmc_means(os.path.join(d, "pmc_FETCH_SIZE"), "FETCH_SIZE")
    write = _pmc_means(os.path.join(d, "pmc_WRITE_SIZE"), "WRITE_SIZE")
    cal_f = _pmc_means(os.path.join(d, "cal_FETCH_SIZE"), "FETCH_SIZE")
    cal_w = _pmc_means(os.path.join(d, "cal_WRITE_SIZE"), "WRITE_SIZE")
    copy_bytes = 256 * 1024 * 1024
    ck = [k for k in cal_f if "copy" in k.lower()]
    if not ck:
        raise SystemExit(f"no copy kernel in the calibration run: {sorted(cal_f)}")
    f_scale = copy_bytes / (cal_f[ck[0]] * 1024)
    w_scale = copy_bytes / (cal_w[ck[0]] * 1024)
    alg = line["roofline"].get("algorithmic_bytes", line["layer"]["gate_up_bytes"])
    hbm = fetch[kernel] * 1024 * f_scale + write[kernel] * 1024 * w_scale
    wl = line["config"]["workload"]
    rec = {"kernel": kernel, "workload": wl, "source_sha256": gemm_source_sha(),
           "fetch_kib": fetch[kernel], "write_kib": write[kernel],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg}
    recs = [r for r in _traffic_records() if (r.get("kernel"), r.get("workload")) != (kernel, wl)]
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump({"records": recs + [rec]}, f, indent=1)
    out = [f"Calibration: a plain copy of 256 MiB reads FETCH_SIZE = {cal_f[ck[0]]:.0f} KiB "
           f"and WRITE_SIZE = {cal_w[ck[0]]:.0f} KiB per dispatch, so counter values are "
           f"scaled by {f_scale:.3f} (fetch) and {w_scale:.3f} (write) to get bytes.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
           "|---|---|---|---|---|"]
    for k in sorted(set(fetch) | set(write)):
        fk, wk = fetch.get(k, 0.0), write.get(k, 0.0)
        out.append(f"| {k} | {fk:.0f} | {wk:.0f} | {fk * 1024 * f_scale / 1e6:.1f} | "
                   f"{wk * 1024 * w_scale / 1e6:.1f} |")
    out += ["", f"{kernel}: {hbm / 1e6:.0f} MB moved per launch against {alg / 1e6:.0f} MB "
                f"algorithmic: ratio {hbm / alg:.2f}."]
    return "\n".join(out)


def cpu_baseline(name: str, cfg: dict, inp, sample_tokens: int):
    """The float64 oracle (as it stands) on the first `sample_tokens` tokens."""
    from oracle import moe_oracle as O
    from workloads import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    wts = {n: getattr(inp, n) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    if cfg.get("weight_format", "dtype") != "dtype":  # MX stacks, one expert at a time
        keys = {"w_gate": "gate", "w_up": "up", "w_down": "down", "ws_gate": "shared_gate",
                "ws_up": "shared_up", "ws_down": "shared_down"}
        elem = "e2m1" if cfg.get("weight_format") == "mxfp4" else "e4m3"
        wts = {n: (O.MxStacked(a, inp.mx[keys[n]], elem) if a is not None else None)
               for n, a in wts.items()}
    wr = inp.w_router
    if cfg.get("router_format", "f32") == "mxfp8":   # the 8-bit router's exact values
        wr = O.mx_dequantize(inp.w_router, inp.mx["router"])
    sub = synth.MoeInputs(cfg=dict(cfg, T=sample_tokens), x=inp.x[:sample_tokens],
                          w_router=wr, expert_bias=inp.expert_bias, **wts)
    t0 = time.perf_counter()
    O.moe_forward(sub, cfg)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"float64 numpy oracle, whole layer on the first {sample_tokens} of "
                      f"{cfg['T']} tokens of {name} ({dt:.1f} s wall)"}


def _launch_ms(torch, stream, fn, n):
    """Average duration of n back-to-back launches on `stream` (HIP events)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def block_measurements(moe, synth, cfg, keys, T, ordered, args, stream, t, layer_ms):
    """The MoE block around the layer, out = h + post_norm(layer(pre_norm(h))):
    the whole block per step, and the two row kernels it adds (pre-norm, and
    the finalising combine with post-norm and residual, beside the plain
    combine) with their algorithmic HBM bytes."""
    import torch
    nw = synth.norm_weights(cfg)
    norm = {"eps": nw["eps"], "add_one": nw["add_one"]}
    pre_w, post_w = moe.to_device(nw["pre"]), moe.to_device(nw["post"])
    hout = torch.empty_like(t["out"])
    xn = torch.empty_like(t["x"])

    def block():
        moe.moe_block_forward(keys, norm, T, t["x"], pre_w, post_w, t["wr"], t["b"], t["wg"],
                              t["wu"], t["wd"], t["sg"], t["su"], t["sd"], None, None, None, hout,
                              int(ordered), t["ws"], stream, mx=t["mx"])

    for _ in range(args.warmup):
        block()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        block()
    torch.cuda.synchronize()
    ms_block = (time.perf_counter() - t0) * 1e3 / args.steps
    # the stage tensors still hold the last eager step's acc / y_perm / row_pos / w
    n = max(args.steps, 10)
    H, k = cfg["hidden_size"], cfg["num_experts_per_tok"]
    bx = 2 if cfg["dtype"] == "bf16" else 4
    ms_pre = _launch_ms(torch, stream, lambda: moe.moe_rms_norm(
        keys, norm, T, t["x"], pre_w, xn, stream), n)
    ms_post = _launch_ms(torch, stream, lambda: moe.moe_combine_norm_residual(
        keys, norm, T, t["acc"], t["yp"], t["rp"], t["w"], post_w, t["x"], hout, stream), n)
    ms_comb = _launch_ms(torch, stream, lambda: moe.moe_combine(
        keys, T, t["acc"], t["yp"], t["rp"], t["w"], t["out"], stream), n)
    gathered = T * k * (H * bx + 8) if ordered else 0
    b_pre = 2 * T * H * bx + 4 * H
    b_comb = 4 * T * H + gathered + T * H * bx
    b_post = b_comb + T * H * bx + 4 * H
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    return {"entry": "moe_block_forward", "ms_per_step": ms_block,
            "ms_over_layer": ms_block - layer_ms, "rms_norm_eps": norm["eps"],
            "norm_add_one": norm["add_one"],
            "pre_norm": {"kernel": "rmsnorm_kernel", "ms_per_launch": ms_pre, "bytes": b_pre,
                         "gbs": gbs(b_pre, ms_pre), "frac_hbm_peak": gbs(b_pre, ms_pre) / PEAK_HBM_GBS},
            "combine_norm_residual": {"kernel": "combine_norm_kernel", "ms_per_launch": ms_post,
                                      "bytes": b_post, "gbs": gbs(b_post, ms_post),
                                      "frac_hbm_peak": gbs(b_post, ms_post) / PEAK_HBM_GBS},
            "combine": {"kernel": "combine_kernel", "ms_per_launch": ms_comb, "bytes": b_comb,
                        "gbs": gbs(b_comb, ms_comb), "frac_hbm_peak": gbs(b_comb, ms_comb) / PEAK_HBM_GBS}}


def upload(moe, inp, T=None):
    """The workload's tensors on the GPU (x limited to its first T rows)."""
    d = moe.to_device
    x = inp.x if T is None else inp.x[:T]
    return dict(x=d(x), wr=d(inp.w_router), b=d(inp.expert_bias), wg=d(inp.w_gate),
                wu=d(inp.w_up), wd=d(inp.w_down), sg=d(inp.ws_gate), su=d(inp.ws_up),
                sd=d(inp.ws_down),
                mx={key: d(v) for key, v in inp.mx.items()} if inp.mx is not None else None)


def flush_caches(flush, i, read_back=True):
    """Write the 1 GiB flush buffer, then (read_back) read it all: weights of
    the next call come from HBM and the caches hold clean lines."""
    flush.fill_(i & 0xFF)
    if read_back:
        flush.view(-1, 1 << 20).amax(dim=1)


def measure_layer(moe, cfg, t, T, steps, warmup, ordered, flush):
    """Time one workload by the protocol: stage-call pass and layer pass, each
    with a 1 GiB flush before every timed step and HIP events around the
    layer (or each stage); medians over `steps` steps; plus the warm figure of
    back-to-back calls. Returns timings and the stage tensors."""
    import torch
    keys = synth_keys(cfg)
    E, k, H, I = cfg["num_experts"], cfg["num_experts_per_tok"], cfg["hidden_size"], \
        cfg["moe_intermediate_size"]
    S = cfg["num_shared_experts"]
    Is = cfg["shared_intermediate_size"] or I
    dt = moe.torch_dtype(keys)
    dev = t["x"].device
    ws = moe.alloc_block_workspace(keys, T)
    f32, i32 = torch.float32, torch.int32
    # where the layer takes the fused decode FFN, the stage-call pass calls its
    # entry points (moe_expert_ffn, moe_combine_partials) instead of the
    # grouping and the two grouped GEMMs
    parts_bytes = moe.moe_expert_ffn_size(keys, T)
    fused = (parts_bytes is not None and os.environ.get("MOE_DECODE_FFN") != "0"
             and os.environ.get("MOE_GEMM_TILE") != "128")
    st = dict(
        logits=torch.empty(T * E, dtype=f32, device=dev),
        idx=torch.empty(T * k, dtype=i32, device=dev),
        w=torch.empty(T * k, dtype=f32, device=dev),
        # grouping outputs start as zeros: the fused stage pass never writes
        # them, and the block's combine timings still gather through row_pos
        offs=torch.zeros(E + 1, dtype=i32, device=dev),
        sr=torch.zeros(T * k, dtype=i32, device=dev),
        rp=torch.zeros(T * k, dtype=i32, device=dev),
        parts=torch.empty(max(parts_bytes or 0, 4) // 4, dtype=f32, device=dev),
        h=torch.empty(T * k * I, dtype=dt, device=dev),
        hs=torch.empty(T * S * Is, dtype=dt, device=dev) if S else None,
        acc=torch.empty(T * H, dtype=f32, device=dev),
        out=torch.empty(T * H, dtype=dt, device=dev),
        yp=torch.empty(T * k * H, dtype=dt, device=dev) if ordered else None,
        ws=ws)
    x, mx = t["x"], t["mx"]
    stages = (["router", "route", "ffn", "combine"] if fused else
              ["router", "route", "permute", "gate_up", "down", "combine"])

    def fused_step(events=None):
        s = torch.cuda.current_stream()
        rec = (lambda i: events[i].record(s)) if events else (lambda i: None)
        rec(0)
        moe.moe_router_logits(keys, T, x, t["wr"], st["logits"], ws, s, mx=mx)
        rec(1)
        moe.moe_route(keys, T, st["logits"], t["b"], st["idx"], st["w"], None, s)
        rec(2)
        moe.moe_expert_ffn(keys, T, x, t["wg"], t["wu"], t["wd"], t["sg"], t["su"], t["sd"],
                           st["idx"], st["parts"], s, mx=mx)
        rec(3)
        moe.moe_combine_partials(keys, T, st["parts"], st["w"], st["out"], s)
        rec(4)

    def step(events=None):
        if fused:
            return fused_step(events)
        s = torch.cuda.current_stream()
        rec = (lambda i: events[i].record(s)) if events else (lambda i: None)
        rec(0)
        moe.moe_router_logits(keys, T, x, t["wr"], st["logits"], ws, s, mx=mx)
        rec(1)
        moe.moe_route(keys, T, st["logits"], t["b"], st["idx"], st["w"], None, s)
        rec(2)
        moe.moe_permute(keys, T, st["idx"], st["offs"], st["sr"], st["rp"], ws, s)
        rec(3)
        moe.moe_grouped_gate_up_swiglu(keys, T, x, t["wg"], t["wu"], t["sg"], t["su"],
                                       st["offs"], st["sr"], st["h"], st["hs"], ws, s, mx=mx)
        rec(4)
        moe.moe_grouped_down(keys, T, st["h"], t["wd"], st["hs"], t["sd"], st["offs"], st["sr"],
                             st["w"], st["acc"], st["yp"], ws, s, mx=mx)
        rec(5)
        moe.moe_combine(keys, T, st["acc"], st["yp"], st["rp"], st["w"], st["out"], s)
        rec(6)

    def layer():
        moe.moe_layer_forward(keys, T, x, t["wr"], t["b"], t["wg"], t["wu"], t["wd"], t["sg"],
                              t["su"], t["sd"], None, None, None, None, st["out"], int(ordered),
                              ws, torch.cuda.current_stream(), mx=mx)

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # stage-call pass: flush, then the six stage calls with events between
    sev = [[ev() for _ in range(len(stages) + 1)] for _ in range(steps)]
    for i in range(steps):
        flush_caches(flush, i)
        step(sev[i])
    torch.cuda.synchronize()
    per_stage = {s: [sev[i][j].elapsed_time(sev[i][j + 1]) for i in range(steps)]
                 for j, s in enumerate(stages)}
    stage_ms = {s: float(np.median(v)) for s, v in per_stage.items()}
    # the roofline kernel's stage: the fused FFN, else the grouped gate/up
    roof_stage = "ffn" if fused else "gate_up"
    roof_mean = float(np.mean(per_stage[roof_stage]))

    # the timed steps: flush (outside the events), then the layer call alone;
    # everything is queued on one stream and synchronised once, so the flush
    # also hides the host's launch of the layer's kernels
    for _ in range(warmup):
        layer()
    torch.cuda.synchronize()
    lev = [(ev(), ev()) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush_caches(flush, i)
        lev[i][0].record(stream)
        layer()
        lev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = [a.elapsed_time(b) for a, b in lev]

    # the same with the write-only flush (dirty lines left in the caches)
    wev = [(ev(), ev()) for _ in range(steps)]
    for i in range(steps):
        flush_caches(flush, i, read_back=False)
        wev[i][0].record(stream)
        layer()
        wev[i][1].record(stream)
    torch.cuda.synchronize()
    ms_write_flush = float(np.median([a.elapsed_time(b) for a, b in wev]))

    # warm: back-to-back calls (weights partly in the MALL), for comparison
    t0 = time.perf_counter()
    for _ in range(steps):
        layer()
    torch.cuda.synchronize()
    ms_warm = (time.perf_counter() - t0) * 1e3 / steps

    # decode-sized batches: the layer call captured once in a HIP graph and
    # replayed, each replay after the same flush (events around the replay)
    ms_graph = None
    if T * cfg["num_experts_per_tok"] <= 32 * cfg["num_experts"]:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        gev = [(ev(), ev()) for _ in range(steps)]
        for i in range(steps):
            flush_caches(flush, i)
            gev[i][0].record(stream)
            graph.replay()
            gev[i][1].record(stream)
        torch.cuda.synchronize()
        ms_graph = float(np.median([a.elapsed_time(b) for a, b in gev]))
        del graph
    return dict(ms=float(np.median(per_call)), ms_min=float(np.min(per_call)),
                ms_max=float(np.max(per_call)), wall_s=wall, ms_warm=ms_warm,
                ms_write_flush=ms_write_flush, ms_graph=ms_graph,
                stage_ms=stage_ms, roof_mean_ms=roof_mean, roof_stage=roof_stage, st=st, keys=keys,
                stream=stream)


def synth_keys(cfg):
    from workloads import synth
    return synth.layer_keys(cfg)


def layer_report(name, cfg, T, m, idx_h, logits_h, bias, steps):
    """The measured figures of one workload: tokens/s, the layer against both
    rooflines, the dominant kernel's roofline object and the routing report."""
    alg = algorithmic(cfg, T, idx_h)
    ms = m["ms"]
    tflops = alg["flops"] / (ms * 1e-3) / 1e12
    gbs = alg["bytes"] / (ms * 1e-3) / 1e9
    peak_mm = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_F32_MFMA_TFLOPS
    k, E = cfg["num_experts_per_tok"], cfg["num_experts"]
    # prefill-sized batches are priced against the MFMA peak, decode-sized
    # ones (at most 32 rows per expert on average) against HBM
    decode = T * k <= 32 * E
    gu_ms = m["roof_mean_ms"]
    fused = m["roof_stage"] == "ffn"
    kname = "moe_ffn_decode_kernel" if fused else gate_up_kernel(cfg, T)
    k_flops = alg["ffn_flops"] if fused else alg["gate_up_flops"]
    k_bytes = alg["ffn_bytes"] if fused else alg["gate_up_bytes"]
    gu_tf = k_flops / (gu_ms * 1e-3) / 1e12
    gu_gb = k_bytes / (gu_ms * 1e-3) / 1e9
    if decode:
        roof = {"bound": "hbm", "achieved": gu_gb, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gu_tf, "peak": peak_mm, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_from_profile(kname, name, gemm_source_sha())
    roof["kernel"] = kname
    roof["algorithmic_bytes"] = k_bytes
    roof["algorithmic_flops"] = k_flops
    roof["ms_per_launch"] = gu_ms
    roof["launches_timed"] = steps
    roof["frac_other_roof"] = (gu_gb / PEAK_HBM_GBS) if not decode else (gu_tf / peak_mm)
    layer = {"tflops": tflops, "frac_bf16_peak": tflops / peak_mm, "gbs": gbs,
             "frac_hbm_peak": gbs / PEAK_HBM_GBS, "flops": alg["flops"], "bytes": alg["bytes"],
             "arith_intensity": alg["flops"] / alg["bytes"],
             "gate_up_flops": alg["gate_up_flops"], "gate_up_bytes": alg["gate_up_bytes"],
             "ffn_flops": alg["ffn_flops"], "ffn_bytes": alg["ffn_bytes"],
             "bound": "hbm" if decode else "mfma", "touched_experts": alg["touched"],
             "stage_ms": m["stage_ms"], "ms_median": ms, "ms_min": m["ms_min"],
             "ms_max": m["ms_max"], "ms_per_step_warm": m["ms_warm"],
             "ms_per_step_write_flush": m["ms_write_flush"],
             "ms_per_step_graph": m["ms_graph"],
             "frac_hbm_peak_write_flush": alg["bytes"] / (m["ms_write_flush"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "frac_bf16_peak_warm": alg["flops"] / (m["ms_warm"] * 1e-3) / 1e12 / peak_mm,
             "frac_hbm_peak_warm": alg["bytes"] / (m["ms_warm"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "routing": routing_report(cfg, idx_h, logits_h, bias)}
    return layer, roof


def run_workload(moe, name, cfg, t, T, args, flush, steps):
    import torch
    print(f"[bench] timing {name} (T={T}, {steps} steps)", file=sys.stderr, flush=True)
    m = measure_layer(moe, cfg, t, T, steps, args.warmup, args.combine == "ordered", flush)
    st = m["st"]
    E, k = cfg["num_experts"], cfg["num_experts_per_tok"]
    idx_h = st["idx"].view(T, k).cpu().numpy()
    logits_h = st["logits"].view(T, E).cpu().numpy()
    torch.cuda.synchronize()
    return m, idx_h, logits_h


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps of the headline workload (decode layers: 5x as many)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="bench one workload only (default: the M3-shaped T=8192 layer with "
                         "the two decode layers nested)")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens for the CPU oracle baseline (0 = skip; default 1024, or T "
                         "if smaller)")
    ap.add_argument("--combine", choices=["atomic", "ordered"], default="ordered",
                    help="down-projection combine: fp32 atomics into the output rows, or "
                         "per-row expert outputs summed in a fixed order by moe_combine")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the measurements of the MoE block around the layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (3 times): the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 kernel-trace run and exit")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs (see "
                         "summarize_traffic), write profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_traffic:
        print(summarize_traffic(args.summarize_traffic))
        return
    if args.copy_calibration:
        import torch
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is described in the design notes, not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_moe_transformer_amd as moe
    from workloads import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    name = args.workload or DEFAULT_WORKLOAD
    with_decode = args.workload is None
    cfg = synth.config(name)
    keys = synth.layer_keys(cfg)
    T = cfg["T"]
    E, k, H, I = cfg["num_experts"], cfg["num_experts_per_tok"], cfg["hidden_size"], \
        cfg["moe_intermediate_size"]
    S = cfg["num_shared_experts"]
    Is = cfg["shared_intermediate_size"] or I
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    inp = synth.generate(cfg)
    t = upload(moe, inp)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=t["x"].device)
    decode_steps = 5 * args.steps

    steps = decode_steps if T * k <= 32 * E else args.steps
    m, idx_h, logits_h = run_workload(moe, name, cfg, t, T, args, flush, steps)
    layer, roof = layer_report(name, cfg, T, m, idx_h, logits_h, inp.expert_bias, steps)
    ms = m["ms"]

    blk = None
    if not args.no_block:
        st = m["st"]
        blk = block_measurements(moe, synth, cfg, keys, T, args.combine == "ordered", args,
                                 m["stream"],
                                 dict(x=t["x"], wr=t["wr"], b=t["b"], wg=t["wg"], wu=t["wu"],
                                      wd=t["wd"], sg=t["sg"], su=t["su"], sd=t["sd"],
                                      acc=st["acc"], yp=st["yp"], rp=st["rp"], w=st["w"],
                                      out=st["out"], ws=st["ws"], mx=t["mx"]), m["ms_warm"])
    del m

    decode = None
    if with_decode:
        decode = {}
        for dname in DECODE_WORKLOADS:
            dcfg = synth.config(dname)
            dT = dcfg["T"]
            same = {kk: v for kk, v in dcfg.items() if kk not in ("T", "name")} == \
                {kk: v for kk, v in cfg.items() if kk not in ("T", "name")}
            if same and dT <= T:
                # the first dT tokens of the same batch, same weights
                dinp, dt_ = inp, dict(t, x=t["x"][:dT])
            else:
                print(f"[bench] generating {dname}", file=sys.stderr, flush=True)
                dinp = synth.generate(dcfg)
                dt_ = upload(moe, dinp)
            dm, didx, dlog = run_workload(moe, dname, dcfg, dt_, dT, args, flush, decode_steps)
            dl, droof = layer_report(dname, dcfg, dT, dm, didx, dlog, dinp.expert_bias,
                                     decode_steps)
            decode[dname] = {"tokens_per_s": dT / (dm["ms"] * 1e-3), "ms_per_step": dm["ms"],
                             "steps": decode_steps, "layer": dl, "roofline": droof}
            del dm
    del flush

    sample = args.cpu_sample
    if sample is None:
        sample = min(T, 1024)
    if sample > 0:
        print(f"[bench] float64 oracle on {sample} tokens of {name}", file=sys.stderr, flush=True)
    cpu = cpu_baseline(name, cfg, inp, sample) if sample > 0 else None

    line = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the workload, random weights)",
        "config": {"workload": name, "tokens": T, "hidden_size": H, "num_experts": E,
                   "num_experts_per_tok": k, "moe_intermediate_size": I,
                   "num_shared_experts": S, "shared_intermediate_size": Is,
                   "shared_packed": cfg["shared_packed"], "hidden_act": cfg["hidden_act"],
                   "expert_weights": (cfg["weight_format"]
                                      if cfg.get("weight_format", "dtype") != "dtype"
                                      else cfg["dtype"]),
                   "combine": args.combine, "entry": "moe_layer_forward",
                   "timing": "median of K steps, each after a 1 GiB write + read-back flush "
                             "(outside the events)"},
        "layer": layer,
        "roofline": roof,
        "decode": decode,
        "block": blk,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
