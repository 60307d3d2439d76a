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


def full_square_flops_per_token(cfg, T):
    """6 N + 12 L d T: the same N, attention counted over the full T x T
    score matrix (the PaLM-paper convention), reported beside the causal count."""
    return model_flops_per_token(cfg, T) - 6 * cfg.n_layer * cfg.n_embd * (T + 1) + 12 * cfg.n_layer * cfg.n_embd * T \
        if not (cfg.window_even or cfg.window_odd) else None


# Muon's learning rate and momentum for the --muon line (the article's defaults)
MUON_LR, MUON_MOMENTUM = 0.02, 0.95


def cpu_baseline(w, seq, muon=False):
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
    O.train_step(params, m, m, [(x, y)], cfg, w.lr, 1, muon=(MUON_LR, MUON_MOMENTUM) if muon else None)
    dt = time.perf_counter() - t0
    opt = "Muon on the hidden matrices and AdamW on the rest" if muon else "AdamW"
    return {"value": round(seq / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one {seq}-token sequence of {w.name}: float64 forward, backward, clip and {opt} over all "
                      f"{sum(int(np.prod(s)) for _, s, _, _ in O.param_table(cfg))} parameters, {dt:.1f} s"}


def cpu_table():
    """The float64 CPU oracle on one sequence of each parity configuration's
    shape, with all host threads and with one: 64 tokens of the tiny fp32
    model, 256 of the char model and 1024 of GPT-2 124M (that one with all
    threads only); a full step, clip and update included."""
    from transformer_lm_step_gpt_amd import inputs as I
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    rows = []
    for w, seq, one in ((I.TINY_FP32, 64, True), (I.CHAR_BF16, 256, True), (I.GPT2_124M, 1024, False)):
        for single in ((False, True) if one else (False,)):
            if single and threadpool_limits is None:
                continue
            if single:
                with threadpool_limits(limits=1):
                    r = cpu_baseline(w, seq)
                r["cores"] = 1
            else:
                r = cpu_baseline(w, seq)
            rows.append({"workload": w.name, **r})
            print(json.dumps(rows[-1]), flush=True)


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


def stream_ceiling():
    """PyTorch's own streaming rates on this GPU, the practical ceiling the
    bandwidth-bound kernels are read against: a device copy (read + write)
    and a sum (read) of fp32 buffers of 200 MB to 3.3 GB."""
    import torch

    def timed(f, n=20):
        for _ in range(3):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    rows = []
    for mb in (200, 800, 1650, 3300):
        n = mb * 2**20 // 4
        a = torch.randn(n, device="cuda:0")
        b = torch.empty_like(a)
        t_copy = timed(lambda: b.copy_(a))
        t_sum = timed(lambda: a.sum())
        rows.append({"MB": mb, "copy_GBps": round(8 * n / t_copy / 1e9, 1), "sum_GBps": round(4 * n / t_sum / 1e9, 1)})
        del a, b
    print(json.dumps({"stream_ceiling": rows, "peak_GBps": PEAK_HBM_GBS}))


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


def trace_gaps(d, steps):
    """Idle GPU time per step from a rocprofv3 --kernel-trace kernel_trace.csv.

    Steps are delimited by the AdamW launch that ends each one; the last
    `steps` steps are analysed (the uninstrumented steps at the end of a bench
    run). Reports per step: wall time (AdamW end to AdamW end), time with at
    least one kernel running, the rest (idle), and on the queue with the most
    launches (the main stream) the sum of gaps between consecutive kernels."""
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))[0]
    rows = list(csv.DictReader(open(f)))
    ks = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r.get("Queue_Id", r.get("Stream_Id", "0")),
                  r["Kernel_Name"]) for r in rows), key=lambda k: k[0])
    ends = [k[1] for k in ks if "adamw_kernel" in k[3]]
    if len(ends) < steps + 1:
        raise SystemExit(f"trace holds {len(ends)} AdamW launches, need {steps + 1}")
    out = []
    for i in range(len(ends) - steps, len(ends)):
        t0, t1 = ends[i - 1], ends[i]
        sel = [k for k in ks if k[0] >= t0 and k[1] <= t1]
        busy, cur_s, cur_e = 0, None, None
        for a, b, _, _ in sel:
            if cur_e is None or a > cur_e:
                if cur_e is not None:
                    busy += cur_e - cur_s
                cur_s, cur_e = a, b
            else:
                cur_e = max(cur_e, b)
        if cur_e is not None:
            busy += cur_e - cur_s
        queues = {}
        for k in sel:
            queues.setdefault(k[2], []).append(k)
        main = max(queues.values(), key=len)
        gaps = sum(max(0, main[j + 1][0] - main[j][1]) for j in range(len(main) - 1))
        out.append({"wall_ms": (t1 - t0) / 1e6, "busy_ms": busy / 1e6, "idle_ms": (t1 - t0 - busy) / 1e6,
                    "kernels": len(sel), "queues": len(queues), "main_queue_kernels": len(main),
                    "main_queue_gap_ms": gaps / 1e6})
    keys = list(out[0])
    print("| step | " + " | ".join(keys) + " |")
    print("|---" * (len(keys) + 1) + "|")
    for i, o in enumerate(out):
        print(f"| {i} | " + " | ".join(f"{o[k]:.3f}" if isinstance(o[k], float) else str(o[k]) for k in keys) + " |")
    med = {k: float(np.median([o[k] for o in out])) for k in keys}
    print("| median | " + " | ".join(f"{med[k]:.3f}" for k in keys) + " |")


# rocprofv3 kernel names -> the library's kernel classes of the bandwidth-bound steps
PMC_CLASSES = [("embed_fwd_kernel", "embed_fwd"), ("layernorm_fwd_kernel", "layernorm_fwd"),
               ("layernorm_bwd_kernel", "layernorm_bwd"), ("cross_entropy_reg_kernel", "cross_entropy"),
               ("embed_piece_kernel", "embed_bwd"), ("embed_segment_kernel", "embed_bwd"),
               ("embed_wpe_kernel", "embed_bwd"), ("reduce_jobs_stage", "partial_reduce"),
               ("grad_norm_partial_kernel", "grad_norm"), ("grad_norm_final_kernel", "grad_norm"),
               ("adamw_kernel", "adamw")]


def _pmc_means(d, counter):
    """Mean value of `counter` per dispatch of each kernel name in a rocprofv3 --pmc output dir."""
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))[0]
    acc = {}
    for r in csv.DictReader(open(f)):
        if r.get("Counter_Name", counter) != counter:
            continue
        v = acc.setdefault(r["Kernel_Name"], [0.0, 0])
        v[0] += float(r["Counter_Value"])
        v[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def trace_step_durations(d, step):
    """Per kernel name: (summed duration in ns, dispatches) of the kernels of
    AdamW-delimited step `step` (0-based) in a rocprofv3 --kernel-trace run."""
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))[0]
    ks = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in csv.DictReader(open(f))),
                key=lambda k: k[0])
    ends = [k[1] for k in ks if "adamw_kernel" in k[2]]
    t0 = ends[step - 1] if step > 0 else 0
    t1 = ends[step]
    out = {}
    for a, b, n in ks:
        if a >= t0 and b <= t1:
            v = out.setdefault(n, [0, 0])
            v[0] += b - a
            v[1] += 1
    return out


def pmc_table(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, kernel_json, trace_dir=None, trace_step=1):
    """Markdown table: per bandwidth-bound kernel class, algorithmic bytes per
    launch (the library's count), HBM bytes per launch from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, each scaled by what it reads for a plain copy
    of known size), and the algorithmic GB/s of the class's launches timed
    alone (bench.py's all-launches-timed step)."""
    copy_bytes = 4.0 * (64 << 20)
    cf = _pmc_means(cal_fetch_dir, "FETCH_SIZE")
    cw = _pmc_means(cal_write_dir, "WRITE_SIZE")
    kf = max(cf.items(), key=lambda kv: kv[1])[1]     # the copy kernel dominates the calibration run
    kw = max(cw.items(), key=lambda kv: kv[1])[1]
    fetch_factor, write_factor = copy_bytes / (kf * 1024), copy_bytes / (kw * 1024)
    fm, wm = _pmc_means(fetch_dir, "FETCH_SIZE"), _pmc_means(write_dir, "WRITE_SIZE")
    kj = json.load(open(kernel_json))
    cls = {r["name"]: r for r in kj["classes"]}
    per_step = kj["launch_steps"]
    print(f"FETCH_SIZE factor {fetch_factor:.4f}, WRITE_SIZE factor {write_factor:.4f} (copy of {copy_bytes:.0f} bytes)")
    dur = trace_step_durations(trace_dir, trace_step) if trace_dir else None
    src = ("rocprofv3 kernel durations of the serialized step" if dur else "HIP events around each launch")
    print(f"alone durations from {src}")
    print("| class | launches/step | kernels | algorithmic MB/launch | counter MB/launch | counter/alg | "
          "alone us/launch | alg GB/s alone | of 8 TB/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    for c in dict.fromkeys(c for _, c in PMC_CLASSES):
        names = [n for n in fm if any(sub in n and cc == c for sub, cc in PMC_CLASSES)]
        r = cls.get(c)
        if not names or not r or not r["launches"]:
            continue
        # every kernel of the class runs once per library launch of it
        hbm = sum(fm[n] * 1024 * fetch_factor + wm.get(n, 0.0) * 1024 * write_factor for n in names)
        alg = r["bytes"] / r["launches"]
        us = 1e3 * r["ms"] / r["launches"]
        if dur:
            tn = [n for n in dur if any(sub in n and cc == c for sub, cc in PMC_CLASSES)]
            if tn:
                us = 1e-3 * sum(dur[n][0] for n in tn) / r["launches"]
        gbs = alg / (us * 1e-6) / 1e9
        short = ", ".join(sorted({n.split("(")[0].replace("void ", "").replace("gk::", "")[:40] for n in names}))
        print(f"| {c} | {r['launches'] / per_step:.0f} | {short} | {alg / 1e6:.1f} | {hbm / 1e6:.1f} | "
              f"{hbm / alg:.2f} | {us:.1f} | {gbs:.0f} | {100 * gbs / PEAK_HBM_GBS:.0f}% |")
    # the dominant kernel of the step (largest summed time in the all-launches-timed step)
    dom = max(kj["kernels"], key=lambda r: r["ms"])
    names = [n for n in fm if dom["name"] in n]
    if names:
        n = names[0]
        fb, wb = fm[n] * 1024 * fetch_factor, wm.get(n, 0.0) * 1024 * write_factor
        per = dom["flops"] / dom["launches"] if dom["flops"] else dom["bytes"] / dom["launches"]
        unit = "FLOP" if dom["flops"] else "bytes"
        print(f"\ndominant kernel: {dom['name']}")
        print(f"kernel: {dom['name']}")
        print(f"sources_sha: {sources_sha()}")
        print(f"fetch_bytes_per_launch: {fb:.0f}")
        print(f"write_bytes_per_launch: {wb:.0f}")
        print(f"hbm_bytes_per_launch: {fb + wb:.0f}")
        print(f"algorithmic {unit} per launch (mean over its launches): {per:.0f}")


# counters of one rocprofv3 pass (eight SQ counters and one GRBM counter) for --sq-table
SQ_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
               "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
SQ_KERNELS = ["attn_fwd_mfma_kernel", "attn_bwd_dq_mfma_kernel", "attn_bwd_dkdv_mfma_kernel", "layernorm_bwd_kernel",
              "layernorm_fwd_kernel", "cross_entropy_reg_kernel",
              "gemm_mfma_kernel<256, 256, 64, 2, 1, 2, 2, 4, false, false, 0, 0, 0, true>",
              "gemm_mfma_kernel<256, 256, 64, 2, 1, 2, 2, 4, true, true, 0, 1, 0, false>"]


def sq_table(d):
    """Markdown table of instruction-mix counters per kernel (means per dispatch)
    from a rocprofv3 --pmc run with SQ_COUNTERS; rocprofv3 serialises dispatches
    while it collects counters, so each figure is the kernel alone.
    GRBM_GUI_ACTIVE is summed over the XCDs (Num_Xcc in the run's agent info),
    so the kernel's GPU cycles are GRBM_GUI_ACTIVE / Num_Xcc; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs) and VALU busy =
    4 SQ_ACTIVE_INST_VALU / (cycles x SIMDs)."""
    import csv
    import glob
    m = {c: _pmc_means(d, c) for c in SQ_COUNTERS}
    info = sorted(glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True))[0]
    gpu = next(r for r in csv.DictReader(open(info)) if r["Agent_Type"] == "GPU")
    xcc, simds = int(gpu["Num_Xcc"]), int(gpu["Simd_Count"])
    print(f"{xcc} XCDs, {simds} SIMDs; cycles = GRBM_GUI_ACTIVE / {xcc} (2400 cycles per us at 2.4 GHz)")
    print("| kernel | cycles | MFMA busy | VALU busy | VALU instr per MFMA instr | LDS instr | "
          "LDS bank-conflict cycles per LDS instr |")
    print("|---|---|---|---|---|---|---|")
    for sub in SQ_KERNELS:
        names = [n for n in m["GRBM_GUI_ACTIVE"] if sub in n]
        if not names:
            continue
        n = names[0]
        g = m["GRBM_GUI_ACTIVE"][n] / xcc
        get = lambda c: m[c].get(n, 0.0)
        mf = 100 * get("SQ_VALU_MFMA_BUSY_CYCLES") / max(g * simds, 1)
        va = 100 * 4 * get("SQ_ACTIVE_INST_VALU") / max(g * simds, 1)
        ratio = get("SQ_INSTS_VALU") / get("SQ_INSTS_MFMA") if get("SQ_INSTS_MFMA") else float("nan")
        lds = get("SQ_INSTS_LDS")
        conf = get("SQ_LDS_BANK_CONFLICT") / lds if lds else 0.0
        short = n.split("(")[0].replace("void ", "").replace("gk::", "")
        print(f"| `{short}` | {g:.0f} | {mf:.1f}% | {va:.1f}% | {ratio:.1f} | {lds:.0f} | {conf:.3f} |")


def generate_bench(a):
    """Sampling with the key/value cache on the 124M model (a second workload,
    not the headline): B sequences of a T0-token prompt, n_new tokens each,
    top-k 50, temperature 1. A decode step is HBM-bound: it reads every bf16
    weight matrix once (the tied head included) plus the cached keys and values
    of the tokens so far."""
    import torch
    from transformer_lm_step_gpt_amd import inputs as I
    from transformer_lm_step_gpt_amd.gpt import GPT
    w = I.GPT2_124M
    cfg = w.model
    B, T0, n_new = cfg.max_batch, 128, 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = GPT(cfg, seed=w.init_seed, device=dev)
    prompt = torch.tensor(next(I.batches(w, B, T0))[0], device=dev)
    for _ in range(2):
        model.generate(prompt, n_new, 1.0, 50, 1)
    reps = max(1, a.steps // 5)
    t0 = time.perf_counter()
    for r in range(reps):
        model.generate(prompt, 1, 1.0, 50, r)
    t_prefill = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for r in range(reps):
        model.generate(prompt, n_new, 1.0, 50, r)
    t_all = (time.perf_counter() - t0) / reps
    step_s = (t_all - t_prefill) / (n_new - 1)
    d, L = cfg.n_embd, cfg.n_layer
    per_layer_w = 3 * d * d + d * d + 2 * cfg.mlp_hidden * d
    weight_bytes = 2.0 * (L * per_layer_w + cfg.padded_vocab_size * d)
    mean_pos = T0 + n_new / 2
    cache_bytes = 2.0 * B * mean_pos * 2 * d * L
    achieved = (weight_bytes + cache_bytes) / step_s / 1e9
    print(json.dumps({
        "metric": "decode tokens/s, sampling with a key/value cache (GPT-2 124M bf16, B=16, prompt 128, 128 new, "
                  "top-k 50)", "value": round(B / step_s, 1), "unit": "tokens/s", "ms_per_decode_step": round(1e3 * step_s, 4),
        "prefill_ms": round(1e3 * t_prefill, 3), "higher_is_better": True, "dtype": "bf16", "n_gpus": 1,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes_per_step": round(weight_bytes + cache_bytes)}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-table", action="store_true", help="print per-kernel-class times to stderr")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the counter-calibration copy kernel")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the float64 CPU oracle on the parity configurations with all threads and with one")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="print PyTorch's copy and sum rates on this GPU (the practical streaming ceiling)")
    ap.add_argument("--rocprof-summary", metavar="DIR", help="print a table from a rocprofv3 --stats output dir")
    ap.add_argument("--trace-gaps", metavar="DIR", help="idle time per step from a rocprofv3 --kernel-trace output "
                                                         "dir (the last --steps steps)")
    ap.add_argument("--head-fp8", action="store_true", help="the same step with the FP8 head (e4m3 lm_head "
                                                              "forward product; a separate line, not the headline)")
    ap.add_argument("--muon", action="store_true", help="the same step with Muon on the blocks' hidden matrices "
                    "and AdamW on the rest (gpt_clip_and_muon) instead of AdamW everywhere")
    ap.add_argument("--generate", action="store_true", help="time sampling with the key/value cache instead "
                                                               "(a second workload; prints its own line)")
    ap.add_argument("--kernel-json", metavar="PATH", help="write the per-class and per-kernel timings of the "
                                                          "all-launches-timed step to PATH")
    ap.add_argument("--pmc-table", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR",
                                                     "KERNEL_JSON"),
                    help="HBM traffic table of the bandwidth-bound kernels from rocprofv3 --pmc runs")
    ap.add_argument("--sq-table", metavar="DIR", help="instruction-mix and utilisation table from a rocprofv3 --pmc "
                    "run with the counters of SQ_COUNTERS")
    ap.add_argument("--pmc-trace", metavar="DIR", help="with --pmc-table: take the alone durations from this "
                                                       "rocprofv3 --kernel-trace run's serialized step")
    ap.add_argument("--pmc-trace-step", type=int, default=None,
                    help="with --pmc-trace: AdamW-delimited index of the serialized step (default: --warmup)")
    a = ap.parse_args()
    if a.pmc_table:
        pmc_table(*a.pmc_table, trace_dir=a.pmc_trace,
                  trace_step=a.pmc_trace_step if a.pmc_trace_step is not None else a.warmup)
        return
    if a.rocprof_summary:
        rocprof_summary(a.rocprof_summary)
        return
    if a.sq_table:
        sq_table(a.sq_table)
        return
    if a.trace_gaps:
        trace_gaps(a.trace_gaps, a.steps)
        return
    if a.copy_calibration:
        copy_calibration()
        return
    if a.stream_ceiling:
        stream_ceiling()
        return
    if a.cpu_table:
        cpu_table()
        return
    if a.generate:
        generate_bench(a)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: the step runs on exactly one GPU (asked for {a.gpus}); the multi-GPU data-parallel "
              "path is a design, not an implementation.", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_lm_step_gpt_amd import inputs as I
    from transformer_lm_step_gpt_amd.gpt import GPT

    w = I.WORKLOADS[a.workload]
    cfg = w.model.replace(head_fp8=True) if a.head_fp8 else w.model
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
        if a.muon:
            model.clip_and_muon(w.lr, MUON_LR, MUON_MOMENTUM, step_no[0], sync=False)
        else:
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
    if a.kernel_json:
        with open(a.kernel_json, "w") as fh:
            json.dump({"launch_steps": 1, "classes": table, "kernels": names}, fh)
    dom = max(names, key=lambda r: r["ms"])["name"]
    model.set_kernel_timing(0)
    model.set_kernel_timing_filter(dom)
    model.reset_kernel_timing()

    # one event on the main stream at every step boundary: per-step times for
    # the median and minimum beside the mean
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record()
    for i in range(a.steps):
        step(i)
        bounds[i + 1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    per_step = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(a.steps))
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
        "metric": METRIC + ("; FP8 head (e4m3 lm_head forward)" if a.head_fp8 else "") +
                  ("; Muon on the hidden matrices" if a.muon else ""),
        "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(1e3 * dt / a.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16+fp8 head" if a.head_fp8 else "bf16") if cfg.precision == "bf16" else "fp32",
        "data": "synthetic (seeded Zipf(1.1) tokens with end-of-text document starts; random-init weights)",
        "config": {"workload": f"{w.name}: {w.description}", "global_batch": B * w.accum, "seq_len": T,
                   "parallelism": "single GPU"},
        "mfma_util_pct": round(100 * mfu, 2),
        "model_flops_per_token": fpt,
        "ms_per_step_median": round(per_step[len(per_step) // 2] if len(per_step) % 2 else
                                    0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2]), 3),
        "ms_per_step_min": round(per_step[0], 3),
        "roofline": roof,
        "uninstrumented": {"ms_per_step": round(1e3 * dt_plain / a.steps, 3),
                           "value": round(tokens / dt_plain, 1),
                           "mfma_util_pct": round(100 * tokens / dt_plain * fpt / (PEAK_BF16_TFLOPS * 1e12), 2)},
    }
    fsq = full_square_flops_per_token(cfg, T)
    if fsq is not None:
        out["full_square"] = {"model_flops_per_token": fsq,
                              "mfma_util_pct": round(100 * tps * fsq / (PEAK_BF16_TFLOPS * 1e12), 2)}
    if a.muon:
        out["optimizer"] = {"hidden_matrices": f"muon (lr {MUON_LR}, momentum {MUON_MOMENTUM}, Nesterov, 5 "
                                               "Newton-Schulz steps in bf16)", "rest": f"adamw (lr {w.lr})"}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, T, muon=a.muon)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
