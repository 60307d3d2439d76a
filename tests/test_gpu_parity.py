"""End-to-end parity of the GPU training step (through the C ABI) with the
CPU float64 oracle.

fp32 path: loss rel err <= 1e-5; every gradient tensor and every updated
parameter tensor max|a-b|/max|b| <= 1e-4 (parameters whose gradient is
within rounding of zero are excluded: there AdamW's first step is +-lr by
sign). bf16 path: loss rel err <= 2e-2, gradient cosine >= 0.99 (over all tensors
and for each tensor), parameter cosine after the step >= 0.999, update
direction cosine >= 0.9. Full-shape cases run distinct sequences.
"""

import math
import sys

import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_step_gpt_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def relmax(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def cosine(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    return float(a @ b / max(np.linalg.norm(a) * np.linalg.norm(b), 1e-300))


def make(cfg, seed):
    from transformer_lm_step_gpt_amd.gpt import GPT
    return GPT(cfg, seed=seed, device="cuda:0")


TINY_SPEED = I.ModelConfig(n_layer=2, n_head=2, n_embd=64, mlp_hidden=256, block_size=48, vocab_size=61,
                           padded_vocab_size=64, max_batch=3, precision="fp32", pos_encoding="rope",
                           qk_rmsnorm=True, mlp_act="relu2", window_even=7, window_odd=48, logit_softcap=3.0,
                           zero_init_proj=False)


def check_fp32_step(cfg, seed, batches, lr, step=1):
    """k micro-steps (scale 1/k), clip, AdamW on the GPU vs the oracle."""
    say(f"fp32 step: {cfg} seed {seed} micro-batches {len(batches)}")
    gpu = make(cfg, seed)
    p0 = O.init_params(cfg, seed)
    # the two independent Philox/Box-Muller implementations agree
    for n in gpu.names:
        assert np.abs(gpu.get_param(n) - p0[n]).max() <= 2e-7 * max(1e-30, np.abs(p0[n]).max()), n
    k = len(batches)
    losses = [gpu.forward_backward(x, y, grad_scale=1.0 / k) for x, y in batches]
    g_gpu = gpu.grads()
    norm = gpu.clip_and_adamw(lr, step)
    m0 = O.zeros_like_params(p0)
    lref, nref, gref, P1, _, _ = O.train_step(p0, m0, m0, batches, cfg, lr, step)
    assert abs(np.mean(losses) - lref) / abs(lref) <= 1e-5
    assert abs(gpu.loss_accum() - lref) / abs(lref) <= 1e-5
    assert abs(norm - nref) / nref <= 1e-4
    for n in gpu.names:
        assert relmax(g_gpu[n], gref[n]) <= 1e-4, (n, relmax(g_gpu[n], gref[n]))
    # AdamW: fed with the GPU's own gradients the oracle update must agree to 1e-6
    coef = O.clip_coefficient(O.grad_norm(g_gpu), cfg.max_grad_norm)
    P_own, _, _ = O.adamw_update(p0, {n: g_gpu[n].astype(np.float64) for n in g_gpu}, m0, m0, lr, step, cfg,
                                 O.decay_flags(cfg), grad_coef=coef)
    excluded = 0
    for n in gpu.names:
        p1 = gpu.get_param(n)
        assert relmax(p1, P_own[n]) <= 1e-6, n
        gdiff = np.abs(g_gpu[n] - gref[n]).max()
        keep = np.abs(gref[n]) > 10 * gdiff
        excluded += int((~keep).sum())
        if keep.any():
            assert np.abs(p1 - P1[n])[keep].max() <= 1e-4 * np.abs(P1[n]).max(), n
    say(f"  loss {np.mean(losses):.7f} vs {lref:.7f}, norm {norm:.6f} vs {nref:.6f}, sign-ambiguous excluded {excluded}")
    return gpu


def test_tiny_fp32_one_step():
    w = I.TINY_FP32
    x, y = next(I.batches(w))
    check_fp32_step(w.model, w.init_seed, [(x, y)], w.lr)


def test_tiny_fp32_accumulation():
    """Two micro-batches at scale 1/2 (the lecture's gradient accumulation) vs the oracle."""
    w = I.TINY_FP32
    it = I.batches(w, 2, 64)
    check_fp32_step(w.model, 11, [next(it), next(it)], 3e-4, step=3)


def test_tiny_fp32_short_sequence():
    """T < block_size and B < max_batch, ragged against every tile size."""
    w = I.TINY_FP32
    x, y = next(I.batches(w, 3, 29))
    check_fp32_step(w.model, 5, [(x, y)], w.lr)


def test_speedrun_variant_fp32():
    """RoPE, QK-RMSNorm, ReLU^2, windows 7/48, softcap 3 on a small fp32 model."""
    rng = np.random.default_rng(9)
    x = rng.integers(0, 64, (3, 48)).astype(np.int32)
    y = rng.integers(0, 64, (3, 48)).astype(np.int32)
    check_fp32_step(TINY_SPEED, 21, [(x, y)], 6e-4)


def test_causal_invariance_gpu():
    """Changing tokens after position i leaves the per-position losses at <= i bitwise unchanged."""
    w = I.TINY_FP32
    gpu = make(w.model, 1)
    x, y = next(I.batches(w))
    gpu.forward_backward(x, y)
    l1 = gpu.row_losses(4, 64)
    x2 = x.copy()
    x2[:, 40:] = (x2[:, 40:] + 1) % 65
    gpu.forward_backward(x2, y)
    l2 = gpu.row_losses(4, 64)
    assert np.array_equal(l1[:, :40], l2[:, :40])
    assert not np.array_equal(l1[:, 40:], l2[:, 40:])


def test_determinism_bitwise():
    w = I.CHAR_BF16
    cfg = w.model.replace(max_batch=8)
    x, y = next(I.batches(w, 8, 256))
    outs = []
    for _ in range(2):
        gpu = make(cfg, 2)
        loss = gpu.forward_backward(x, y)
        gpu.clip_and_adamw(6e-4, 1)
        outs.append((loss, gpu.get_param("wte"), gpu.get_param("h.3.mlp.c_fc.weight"), gpu.get_grad("wte")))
        gpu.close()
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1:], outs[1][1:]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("which", ["tiny_fp32", "tiny_speedrun_fp32", "char_bf16"])
def test_first_micro_step_writes_every_gradient(which):
    """The first micro-step after an update writes every gradient element
    (the products store, the reductions overwrite) instead of zero-filling the
    buffer and adding. After a full step, which leaves the previous step's
    gradients in the buffer, that micro-step must give exactly the gradients
    of the same micro-step added onto zeros (set_grad zero-fills the buffer
    and makes the next micro-step accumulate): a tensor or element that the
    pass did not write would keep the previous step's value."""
    if which == "tiny_fp32":
        w, cfg = I.TINY_FP32, I.TINY_FP32.model
        B, T = 4, 64
    elif which == "tiny_speedrun_fp32":
        w, cfg = I.TINY_FP32, TINY_SPEED
        B, T = 3, 48
    else:
        w, cfg = I.CHAR_BF16, I.CHAR_BF16.model.replace(max_batch=4)
        B, T = 4, 256
    it = I.batches(w, B, T) if which != "tiny_speedrun_fp32" else None
    rng = np.random.default_rng(5)
    if it is None:
        data = [(rng.integers(0, cfg.vocab_size, (B, T)).astype(np.int32),
                 rng.integers(0, cfg.vocab_size, (B, T)).astype(np.int32)) for _ in range(2)]
    else:
        data = [next(it) for _ in range(2)]
    grads = []
    for zero_first in (False, True):
        say(f"first micro-step writes: {which}, zero-filled buffer first: {zero_first}")
        gpu = make(cfg, 3)
        gpu.forward_backward(*data[0])
        gpu.clip_and_adamw(6e-4, 1)
        if zero_first:
            gpu.set_grad(gpu.names[0], np.zeros(gpu.shapes[0], np.float32))
        gpu.forward_backward(*data[1])
        grads.append(gpu.grads())
        gpu.close()
    for n in grads[0]:
        assert np.array_equal(grads[0][n], grads[1][n]), n


def test_error_paths():
    from transformer_lm_step_gpt_amd.gpt import GptError
    w = I.TINY_FP32
    gpu = make(w.model, 1)
    x, y = next(I.batches(w))
    with pytest.raises(GptError) as e:
        gpu.forward_backward(np.zeros((4, 65), np.int32), np.zeros((4, 65), np.int32))   # T > block_size
    assert e.value.status == -1
    with pytest.raises(GptError) as e:
        gpu.forward_backward(np.zeros((5, 8), np.int32), np.zeros((5, 8), np.int32))     # B > max_batch
    assert e.value.status == -1
    bad = y.copy()
    bad[1, 3] = 65
    with pytest.raises(GptError) as e:
        gpu.forward_backward(x, bad)
    assert e.value.status == -5
    with pytest.raises(GptError) as e:
        gpu.clip_and_adamw(1e-3, 0)
    assert e.value.status == -1
    # the handle keeps working after errors
    loss = gpu.forward_backward(x, y)
    assert math.isfinite(loss)
    # a non-finite gradient norm skips the update
    g = gpu.get_grad("wte")
    g[0, 0] = np.inf
    gpu.set_grad("wte", g)
    before = gpu.get_param("wte")
    with pytest.raises(GptError) as e:
        gpu.clip_and_adamw(1e-3, 1)
    assert e.value.status == -6
    assert np.array_equal(gpu.get_param("wte"), before)


def test_bad_id_without_wait_skips_update():
    """An out-of-range target in a micro-step that does not wait: the update
    that follows is skipped on the device (parameters and moments unchanged)
    and reports TOKEN_RANGE when it waits; the report clears the flag."""
    from transformer_lm_step_gpt_amd.gpt import GptError
    w = I.TINY_FP32
    gpu = make(w.model, 1)
    x, y = next(I.batches(w))
    bad = y.copy()
    bad[2, 5] = -3
    before = gpu.params()
    gpu.forward_backward(x, bad, sync=False)
    with pytest.raises(GptError) as e:
        gpu.clip_and_adamw(1e-3, 1)
    assert e.value.status == -5
    for n in gpu.names:
        assert np.array_equal(gpu.get_param(n), before[n]), n
        m, v = gpu.get_opt_state(n)
        assert not m.any() and not v.any(), n
    # cleared by the report: a clean micro-step and update go through
    gpu.forward_backward(x, y, sync=False)
    norm = gpu.clip_and_adamw(1e-3, 1)
    assert math.isfinite(norm) and norm > 0
    assert not np.array_equal(gpu.get_param("wte"), before["wte"])


# ---------------------------------------------------------------- bf16 path

def bf16_compare(gpu, cfg, p, m, v, gpu_batches, oracle_batches, lr, step, label):
    """One optimiser step on the GPU (its micro-batches at grad_scale 1/k) and in
    the oracle (its micro-batches at 1/k), then the bf16 gates: loss rel err
    <= 2e-2; gradient cosine >= 0.99 over all tensors and for every tensor whose
    oracle gradient is non-zero (tensors with an exactly zero oracle gradient
    must come out zero); parameter cosine >= 0.999 after the step; the update
    direction (parameter change) cosine >= 0.9 over all tensors. Returns the
    oracle's new (p, m, v)."""
    k = len(gpu_batches)
    losses = [gpu.forward_backward(x, y, grad_scale=1.0 / k, sync=(j + 1 == k)) for j, (x, y) in
              enumerate(gpu_batches)]
    loss = gpu.loss_accum()
    g_gpu = gpu.grads()
    p_before = {n: gpu.get_param(n) for n in gpu.names}
    norm = gpu.clip_and_adamw(lr, step)
    rows = sum(x.shape[0] * x.shape[1] for x, _ in oracle_batches)
    lref, nref, gref, p_new, m_new, v_new = O.train_step(p, m, v, oracle_batches, cfg, lr, step,
                                                         progress=say if rows >= 1024 else None)
    names = gpu.names
    gcos = cosine(np.concatenate([g_gpu[n].ravel() for n in names]), np.concatenate([gref[n].ravel() for n in names]))
    per = sorted((cosine(g_gpu[n], gref[n]), n) for n in names if np.abs(gref[n]).max() > 0)
    zero = [n for n in names if np.abs(gref[n]).max() == 0]
    gmax = max(float(np.abs(g_gpu[n]).max()) for n in names)
    p_gpu = {n: gpu.get_param(n) for n in names}
    pcos = cosine(np.concatenate([p_gpu[n].ravel() for n in names]), np.concatenate([p_new[n].ravel() for n in names]))
    ucos = cosine(np.concatenate([(p_gpu[n] - p_before[n]).ravel() for n in names]),
                  np.concatenate([(p_new[n] - p[n]).ravel() for n in names]))
    say(f"  {label}: loss {loss:.5f} vs {lref:.5f}; norm {norm:.4f} vs {nref:.4f}; grad cos {gcos:.6f}; "
        f"worst tensors {[(n, round(c, 5)) for c, n in per[:3]]}; exact-zero tensors {len(zero)}; "
        f"param cos {pcos:.7f}; update cos {ucos:.5f}")
    assert abs(loss - lref) / abs(lref) <= 2e-2
    assert abs(norm - nref) / nref <= 2e-2
    assert gcos >= 0.99
    assert per[0][0] >= 0.99, per[:3]
    for n in zero:
        assert np.abs(g_gpu[n]).max() <= 1e-6 * gmax, n
    assert pcos >= 0.999
    assert ucos >= 0.9
    return p_new, m_new, v_new


def bf16_check(w, batch, seq, steps=1, max_batch=None):
    """`steps` optimiser steps of one micro-batch of `batch` distinct sequences
    from the workload's stream, GPU at that launch shape and the oracle on the
    same sequences (one sequence per oracle micro-batch at scale 1/batch: the
    mean over all rows, with one sequence's activations in host memory at a time)."""
    cfg = w.model if max_batch is None else w.model.replace(max_batch=max_batch)
    say(f"bf16 {w.name}: B={batch} T={seq} steps={steps}")
    gpu = make(cfg, w.init_seed)
    p = O.init_params(cfg, w.init_seed)
    m = O.zeros_like_params(p)
    v = O.zeros_like_params(p)
    it = I.batches(w, batch, seq)
    for step in range(1, steps + 1):
        x, y = next(it)
        lr = 6e-4 * step / steps if steps > 1 else w.lr
        per_seq = [(x[b:b + 1], y[b:b + 1]) for b in range(batch)]
        p, m, v = bf16_compare(gpu, cfg, p, m, v, [(x, y)], per_seq, lr, step, f"step {step}")
    return gpu


@pytest.mark.timeout(600)
def test_char_bf16_trajectory():
    """char-level shape at B=4 over the full 20-step warmup schedule
    (lr_t = 6e-4 (t+1)/20): every step within tolerance of the oracle."""
    bf16_check(I.CHAR_BF16, 4, 256, steps=20, max_batch=4)


@pytest.mark.timeout(600)
def test_char_bf16_full_batch():
    """The char-level workload at its full launch shape (64 distinct sequences of 256)."""
    bf16_check(I.CHAR_BF16, 64, 256)


@pytest.mark.timeout(900)
def test_gpt2_124m_full_shape():
    """GPT-2 124M at B=16, T=1024 (the benchmark's launch configuration) on 16
    distinct sequences of the workload's stream, against the oracle on all 16."""
    bf16_check(I.GPT2_124M, 16, 1024)


@pytest.mark.timeout(900)
def test_speedrun_block_full_shape():
    """Speedrun block (RoPE, QK-RMSNorm, ReLU^2, windows 256/2048, softcap 30,
    zero-init projections) at B=8, T=2048 on 8 distinct sequences, against
    the oracle on all 8."""
    bf16_check(I.SPEEDRUN_BLOCK, 8, 2048)


@pytest.mark.timeout(600)
def test_gpt2_124m_accumulation_distinct_micro_batches():
    """Gradient accumulation over distinct consecutive micro-batches at the 124M
    shape: 4 micro-batches of 1x1024 taken in order from the accumulated
    workload's stream (each advancing it by 1024 tokens) at grad_scale 1/4,
    then clip and AdamW at lr = get_lr(1000), against the oracle's train_step
    on the same 4 sequences."""
    w = I.GPT2_124M_ACCUM
    cfg = w.model
    it = I.batches(w, 1, w.seq_len)
    mbs = [next(it) for _ in range(4)]
    assert not np.array_equal(mbs[0][0], mbs[1][0])
    lr = I_get_lr(1000)
    assert abs(lr - w.lr) <= 1e-12
    gpu = make(cfg, w.init_seed)
    p = O.init_params(cfg, w.init_seed)
    m = O.zeros_like_params(p)
    bf16_compare(gpu, cfg, p, m, m, mbs, mbs, lr, 1, "4 distinct micro-batches")


@pytest.mark.timeout(600)
def test_gpt2_124m_accumulation_full_shape():
    """The 524,288-token step at its launch shape: 32 micro-steps of 16x1024
    with grad_scale 1/32, clip, AdamW at lr = get_lr(1000). With every
    micro-batch equal, the accumulated gradient equals that of one micro-step
    at scale 1 (scaling by 2^-5 is exact in every op; only the fp32 sum of 32
    terms rounds), the mean loss equals the single loss, and the clipped
    update matches. This compares the GPU with itself; accumulation over
    distinct micro-batches is pinned to the oracle by the test above."""
    w = I.GPT2_124M_ACCUM
    x, y = I.repeated_sequence_batch(w, w.batch, w.seq_len)
    a = make(w.model, w.init_seed)
    b = make(w.model, w.init_seed)
    for _ in range(w.accum):
        a.forward_backward(x, y, grad_scale=1.0 / w.accum, sync=False)
    lb = b.forward_backward(x, y, grad_scale=1.0)
    la = a.loss_accum()
    say(f"accumulated loss {la:.6f} vs single {lb:.6f}")
    assert abs(la - lb) <= 1e-6 * abs(lb)
    ga, gb = a.grads(), b.grads()
    worst = max(relmax(ga[n], gb[n]) for n in a.names)
    say(f"  max rel grad difference {worst:.2e}")
    assert worst <= 1e-5
    lr = I_get_lr(1000)
    assert abs(lr - w.lr) <= 1e-12
    p0 = np.concatenate([a.get_param(n).ravel() for n in a.names])
    na, nb = a.clip_and_adamw(lr, 1), b.clip_and_adamw(lr, 1)
    say(f"  grad norm {na:.6f} vs {nb:.6f}")
    assert abs(na - nb) <= 1e-5 * nb
    da = np.concatenate([a.get_param(n).ravel() for n in a.names]) - p0
    db = np.concatenate([b.get_param(n).ravel() for n in a.names]) - p0
    ucos = cosine(da, db)
    say(f"  update cosine {ucos:.7f}")
    assert ucos >= 0.999


def I_get_lr(it):
    from transformer_lm_step_gpt_amd.gpt import lr_schedule
    return lr_schedule(it)
