"""Training-step throughput of the GPT-2 step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_124m]

One step = forward + backward of one 16x1024 micro-batch, global clip at 1.0
and AdamW (the full hot path). Inputs are synthetic, seeded, and resident in
device memory before the timed region. Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec on 1 MI355X, GPT-2 124M B=16 T=1024 bf16; MFMA util %"
PEAK_BF16_TFLOPS = 2516.6      # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def model_flops_per_token(cfg, T):
    """6 N + 6 L d (T + 1): N = parameters except the position table (tied
    head counted once), attention as causal pairs, forward + backward."""
    from transformer_lm_step_gpt_amd.inputs import ModelConfig  # noqa: F401
    d, F, L, Vp = cfg.n_embd, cfg.mlp_hidden, cfg.n_layer, cfg.padded_vocab_size
    per_layer = 2 * d + 3 * d * d + 3 * d + d * d + d + 2 * d + F * d + F + d * F + d
    N = Vp * d + L * per_layer + 2 * d
    if cfg.window_even or cfg.window_odd:
        pairs = 0.0
        for l in range(L):
            W = cfg.window_even if l % 2 == 0 else cfg.window_odd
            W = W if W and W < T else T
            pairs += (W * (W + 1) / 2 + (T - W) * W) / T
        attn = 6 * 2 * d * pairs
    else:
        attn = 6 * L * d * (T + 1)
    return 6 * N + attn


def cpu_baseline(w, seq):
    """Time the float64 CPU oracle on one sequence of the same workload."""
    from oracle import gpt_oracle as O
    from transformer_lm_step_gpt_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = w.model
    rng = np.random.default_rng(0)
    params = {n: (rng.standard_normal(s) * 0.02 if len(s) == 2 else (np.ones(s) if "ln" in n and n.endswith("weight")
                                                                       else np.zeros(s)))
              for n, s, _, _ in O.param_table(cfg)}
    m = O.zeros_like_params(params)
    x, y = next(I.batches(w, 1, seq))
    t0 = time.perf_counter()
    O.train_step(params, m, m, [(x, y)], cfg, w.lr, 1)
    dt = time.perf_counter() - t0
    return {"value": round(seq / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one {seq}-token sequence of {w.name}: float64 forward, backward, clip and AdamW over all "
                      f"{sum(int(np.prod(s)) for _, s, _, _ in O.param_table(cfg))} parameters, {dt:.1f} s"}


# Sources of the kernels whose HBM traffic is recorded in profiles/traffic.txt:
# a recorded figure is used only while these files are unchanged.
KERNEL_SOURCES = ["transformer_lm_step_gpt_amd/csrc/gemm_mfma_kernel.h", "transformer_lm_step_gpt_amd/csrc/gemm_common.h",
                  "transformer_lm_step_gpt_amd/csrc/common.h"]


def sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic.txt (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when absent, recorded for another kernel, or taken on other sources."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel") != kernel or rec.get("sources_sha") != sources_sha():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain elementwise copy of known size (fp32 dst = src * 1), for scaling
    the FETCH_SIZE / WRITE_SIZE counters: it reads and writes exactly n * 4 bytes."""
    import torch
    n = 64 << 20
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"copy_kernel_bytes_read": 4 * n, "copy_kernel_bytes_written": 4 * n, "launches": 13,
                      "copy_GBps": round(8 * n / (ms * 1e-3) / 1e9, 1)}))


def rocprof_summary(d):
    """Markdown table from a rocprofv3 --stats kernel_stats.csv (per-kernel totals)."""
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))[0]
    rows = list(csv.DictReader(open(f)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| kernel | calls | total ms | avg us | % |")
    print("|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"| `{r['Name'][:140]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
              f"{float(r['AverageNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / tot:.1f} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-table", action="store_true", help="print per-kernel-class times to stderr")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the counter-calibration copy kernel")
    ap.add_argument("--rocprof-summary", metavar="DIR", help="print a table from a rocprofv3 --stats output dir")
    a = ap.parse_args()
    if a.rocprof_summary:
        rocprof_summary(a.rocprof_summary)
        return
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: the step runs on exactly one GPU (asked for {a.gpus}); the multi-GPU data-parallel "
              "path is a design, not an implementation.", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_lm_step_gpt_amd import inputs as I
    from transformer_lm_step_gpt_amd.gpt import GPT

    w = I.WORKLOADS[a.workload]
    cfg = w.model
    B, T = w.batch, w.seq_len
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = GPT(cfg, seed=w.init_seed, device=dev)
    it = I.batches(w)
    # one step = w.accum micro-batches (consecutive batches of the stream) + clip + AdamW
    n_batches = max(w.accum, min(a.warmup + a.steps, 8))
    data = [next(it) for _ in range(n_batches)]
    toks = [(torch.tensor(x, device=dev), torch.tensor(y, device=dev)) for x, y in data]
    torch.cuda.synchronize()

    step_no = [0]

    def step(i):
        for j in range(w.accum):
            x, y = toks[(i * w.accum + j) % len(toks)]
            model.forward_backward(x, y, 1.0 / w.accum, sync=False)
        step_no[0] += 1
        model.clip_and_adamw(w.lr, step_no[0], sync=False)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    # dominant kernel: time every launch during one untimed step, group by
    # kernel instantiation name
    model.set_kernel_timing(-1)
    model.reset_kernel_timing()
    step(0)
    torch.cuda.synchronize()
    table = model.kernel_timing()
    names = model.kernel_name_timing()
    dom = max(names, key=lambda r: r["ms"])["name"]
    model.set_kernel_timing(0)
    model.set_kernel_timing_filter(dom)
    model.reset_kernel_timing()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    timed = next(r for r in model.kernel_name_timing() if r["name"] == dom)
    model.set_kernel_timing_filter(None)
    # the same steps again with no timing event anywhere (reported beside the
    # timed region, whose dominant-kernel launches are bracketed by events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    dt_plain = time.perf_counter() - t1

    tokens = a.steps * w.accum * B * T
    tps = tokens / dt
    fpt = model_flops_per_token(cfg, T)
    mfu = tps * fpt / (PEAK_BF16_TFLOPS * 1e12)
    n = max(timed["launches"], 1)
    avg_ms = timed["ms"] / n
    if timed["flops"] > 0:
        achieved = timed["flops"] / n / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
        per_launch = {"flops": timed["flops"] / n}
    else:
        achieved = timed["bytes"] / n / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
        per_launch = {"bytes": timed["bytes"] / n}
    traffic = recorded_traffic(dom)
    roof["traffic"] = round(traffic) if traffic is not None else None
    roof.update({"kernel": dom, "avg_launch_ms": round(avg_ms, 4), "launches": timed["launches"],
                 "algorithmic_per_launch": per_launch})
    # In the timed steps the weight-gradient products share the GPU with the
    # input-gradient chain (side stream), so their live launch durations
    # include that sharing; the untimed step above runs every launch alone.
    iso = next(r for r in names if r["name"] == dom)
    if iso["launches"] and iso["ms"] > 0:
        iso_ms = iso["ms"] / iso["launches"]
        if iso["flops"] > 0:
            iso_ach = iso["flops"] / iso["launches"] / (iso_ms * 1e-3) / 1e12
            iso_frac = iso_ach / PEAK_BF16_TFLOPS
        else:
            iso_ach = iso["bytes"] / iso["launches"] / (iso_ms * 1e-3) / 1e9
            iso_frac = iso_ach / PEAK_HBM_GBS
        roof["alone"] = {"avg_launch_ms": round(iso_ms, 4), "achieved": round(iso_ach, 2), "frac": round(iso_frac, 4),
                         "launches": iso["launches"]}
    if a.kernel_table:
        tot = sum(r["ms"] for r in table)
        print(f"step (untimed, all launches timed): {tot:.3f} ms", file=sys.stderr)
        for rows, width in ((table, 18), (names, 72)):
            for r in sorted(rows, key=lambda r: -r["ms"]):
                if r["launches"] and r["ms"] > 0:
                    rate = (f"{r['flops'] / (r['ms'] * 1e-3) / 1e12:8.1f} TFLOP/s" if r["flops"] else
                            f"{r['bytes'] / (r['ms'] * 1e-3) / 1e9:8.1f} GB/s")
                    print(f"{r['name'][:width]:>{width}s} {r['ms']:9.3f} ms {100 * r['ms'] / tot:5.1f}% "
                          f"x{r['launches']:4d} {rate}", file=sys.stderr)
    out = {
        "metric": METRIC, "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(1e3 * dt / a.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.precision == "bf16" else "fp32",
        "data": "synthetic (seeded Zipf(1.1) tokens with end-of-text document starts; random-init weights)",
        "config": {"workload": f"{w.name}: {w.description}", "global_batch": B * w.accum, "seq_len": T,
                   "parallelism": "single GPU"},
        "mfma_util_pct": round(100 * mfu, 2),
        "model_flops_per_token": fpt,
        "roofline": roof,
        "uninstrumented": {"ms_per_step": round(1e3 * dt_plain / a.steps, 3),
                           "value": round(tokens / dt_plain, 1),
                           "mfma_util_pct": round(100 * tokens / dt_plain * fpt / (PEAK_BF16_TFLOPS * 1e12), 2)},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
