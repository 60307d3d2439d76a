"""FP8 head (Modded-NanoGPT README technique list: FP8 matmul for the output
head), against the oracle's fp8_head_logits / head_fp8 model.

Product: both sides quantise the same bf16 operands with per-tensor fp32
scales 448 / max|t| and e4m3 rounding to nearest even, so the codes agree
exactly; what remains is the fp32 accumulation and the bf16 store of z:
max |C - ref| <= 8e-3 max |ref| (the bf16 product bar of the GEMM tests).
Training step with head_fp8: the bf16 gates (loss rel err <= 2e-2, gradient
cosine >= 0.99 overall and per tensor, parameter cosine >= 0.999, update
cosine >= 0.9). The scale recipe itself is a reading (parity unpinned against
the pages, which give none)."""

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


@pytest.fixture(scope="module")
def lib():
    from transformer_lm_step_gpt_amd import gpt as G
    assert torch.cuda.is_available()
    return G.load_library()


def relmax(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.parametrize("M,N,K,rows", [(300, 520, 128, None), (1000, 776, 256, None), (257, 136, 768, None),
                                        (5, 8, 128, None), (16384, 50304, 768, 48)])
def test_gemm_fp8_head(lib, M, N, K, rows):
    """Ragged shapes across several 256 x 256 tiles; at the head's full size
    (16384 x 50304 x 768) `rows` sampled rows are checked."""
    say(f"fp8 head product M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    At = torch.tensor(rng.normal(size=(M, K)), dtype=torch.bfloat16, device="cuda")
    Bt = torch.tensor(rng.normal(size=(N, K)) * 0.02, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    scratch = torch.zeros(int(lib.gptk_gemm_fp8_scratch_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
    st = lib.gptk_gemm_fp8(M, N, K, At.data_ptr(), Bt.data_ptr(), C.data_ptr(), scratch.data_ptr(), scratch.numel(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    A = At.float().cpu().numpy().astype(np.float64)
    B = Bt.float().cpu().numpy().astype(np.float64)
    got = C.float().cpu().numpy()
    if rows is None:
        ref = O.fp8_head_logits(A, B)
    else:
        idx = np.sort(rng.choice(M, rows, replace=False))
        sa, sb = O.fp8_scale(A), O.fp8_scale(B)
        ref = (O.fp8_quantize(A[idx], sa) @ O.fp8_quantize(B, sb).T) / (np.float64(sa) * np.float64(sb))
        got = got[idx]
    err = relmax(got, ref)
    say(f"  max rel err {err:.2e}")
    assert err <= 8e-3


def test_fp8_head_rejects_bad_shapes(lib):
    t = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = t.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.gptk_gemm_fp8(8, 8, 96, p, p, p, p, t.numel(), s) == -1      # K % 128 != 0
    assert lib.gptk_gemm_fp8(8, 12, 128, p, p, p, p, t.numel(), s) == -1    # N % 8 != 0
    assert lib.gptk_gemm_fp8(8, 8, 128, p, p, p, p, 16, s) == -1            # scratch too small


def _step(w, cfg, B, T):
    from test_gpu_parity import bf16_compare, make
    say(f"fp8 head step {w.name} B={B} T={T}")
    gpu = make(cfg, w.init_seed)
    p = O.init_params(cfg, w.init_seed)
    m = O.zeros_like_params(p)
    x, y = next(I.batches(w, B, T))
    # one oracle micro-batch holding every sequence: the activation scale is
    # taken over the whole micro-batch, as on the GPU
    bf16_compare(gpu, cfg, p, m, m, [(x, y)], [(x, y)], w.lr, 1, "fp8 head")


@pytest.mark.timeout(600)
def test_gpt2_124m_step_fp8_head():
    w = I.GPT2_124M
    _step(w, w.model.replace(head_fp8=True), 2, 1024)


@pytest.mark.timeout(600)
def test_speedrun_block_step_fp8_head_softcap():
    """With the logit softcap (30) applied to the FP8 head's logits."""
    w = I.SPEEDRUN_BLOCK
    _step(w, w.model.replace(head_fp8=True), 1, 2048)


def test_fp8_head_config_validation():
    from transformer_lm_step_gpt_amd.gpt import GptError, GPT
    for cfg in (I.TINY_FP32.model.replace(head_fp8=True),                        # fp32 precision
                I.TINY_FP32.model.replace(precision="bf16", head_fp8=True)):     # n_embd 64 % 128 != 0
        with pytest.raises(GptError) as e:
            GPT(cfg, seed=1, device="cuda:0")
        assert e.value.status == -3
