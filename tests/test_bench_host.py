"""Host logic of bench.py (no GPU): the FLOP counts behind mfma_util_pct, the
idle-time analysis of a kernel trace, the traffic record lookup and the
one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_lm_step_gpt_amd import inputs as I  # noqa: E402


def test_model_flops_gpt2_124m():
    # N = all parameters except wpe, tied head once, vocabulary padded to 50304
    L, d, F, Vp, T = 12, 768, 3072, 50304, 1024
    per_layer = 4 * d + (3 * d * d + 3 * d) + (d * d + d) + (F * d + F) + (d * F + d)
    N = Vp * d + L * per_layer + 2 * d
    assert N == 123_689_472
    assert bench.model_flops_per_token(I.GPT2_124M.model, T) == 6 * N + 6 * L * d * (T + 1) == 798_815_232
    assert bench.full_square_flops_per_token(I.GPT2_124M.model, T) == 6 * N + 12 * L * d * T == 855_383_040
    # 16 x 1024 tokens per micro-step: 13.088 TFLOP
    assert abs(16 * 1024 * 798_815_232 / 1e12 - 13.088) < 1e-3


@pytest.mark.parametrize("T,W", [(2048, 256), (2048, 2048), (64, 17), (64, 1), (100, 200)])
def test_window_pair_count_closed_form(T, W):
    # the closed form inside model_flops_per_token against counting visible keys per query
    Wc = W if W < T else T
    brute = sum(min(Wc, i + 1) for i in range(T))
    assert Wc * (Wc + 1) // 2 + (T - Wc) * Wc == brute


def test_model_flops_speedrun_block():
    c = I.SPEEDRUN_BLOCK.model
    T = I.SPEEDRUN_BLOCK.seq_len
    d, L = c.n_embd, c.n_layer
    base = bench.model_flops_per_token(I.GPT2_124M.model, 1024) - 6 * 12 * 768 * 1025   # 6N, same N
    pairs = sum(sum(min(c.window_even if l % 2 == 0 else c.window_odd, i + 1) for i in range(T)) for l in range(L))
    assert bench.model_flops_per_token(c, T) == pytest.approx(base + 12 * d * pairs / T, rel=1e-12)
    assert abs(bench.model_flops_per_token(c, T) / 1e6 - 812.1) < 0.05
    assert bench.full_square_flops_per_token(c, T) is None   # windows: no full-square figure


def _trace(tmp_path, kernels):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w") as fh:
        fh.write('"Kind","Queue_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for q, name, a, b in kernels:
            fh.write(f'"KERNEL_DISPATCH",{q},"{name}",{a},{b}\n')
    return str(d)


def test_trace_gaps(tmp_path, capsys):
    ms = 1_000_000
    ks = [(1, "gk::adamw_kernel", 0, 1 * ms),                # end of the previous step
          (1, "fwd", 2 * ms, 4 * ms), (2, "side", 3 * ms, 6 * ms), (1, "bwd", 5 * ms, 7 * ms),
          (1, "gk::adamw_kernel", 8 * ms, 9 * ms)]
    bench.trace_gaps(_trace(tmp_path, ks), 1)
    out = capsys.readouterr().out.splitlines()
    row = [c.strip() for c in out[2].split("|")[1:-1]]
    # wall 1 -> 9 ms; busy: [2, 7] and [8, 9] = 6 ms; idle 2 ms; 4 kernels on 2 queues;
    # the main queue (3 launches) has gaps 4->5 and 7->8 = 2 ms
    assert row == ["0", "8.000", "6.000", "2.000", "4", "2", "3", "2.000"]


def test_trace_gaps_needs_enough_steps(tmp_path):
    ks = [(1, "gk::adamw_kernel", 0, 10)]
    with pytest.raises(SystemExit):
        bench.trace_gaps(_trace(tmp_path, ks), 1)


def test_recorded_traffic_lookup():
    rec = {}
    with open(os.path.join(ROOT, "profiles", "traffic.txt")) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    assert bench.recorded_traffic("no such kernel") is None
    got = bench.recorded_traffic(rec["kernel"])
    if rec["sources_sha"] == bench.sources_sha():
        assert got == float(rec["hbm_bytes_per_launch"])
    else:
        assert got is None   # the record was taken on other kernel sources


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
