"""Seeded synthetic workloads for the GPT-2 training step.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It holds only workload definitions (model shapes, optimiser settings)
and seeded random input generators; it contains none of the training step's
arithmetic, and it imports neither the HIP binding nor the oracle.

Workloads (model shapes from "Zero to Hero, lecture 9: reproducing GPT-2
(124M)" (ai.flicky.cc), section "Раздел 1 / Архитектура" and the GPTConfig
dataclass there; the char-level shape from "Un GPT desde cero + nanoGPT"
(cursos.romerolabs.dev), section 2.2; the speedrun block variant from the
Modded-NanoGPT README (oa0.com), technique list):

  tiny_fp32     2 layers, 4 heads, d=64, MLP 256, T=64, vocab 65, B=4, fp32
  char_bf16     6 layers, 6 heads, d=384, MLP 1536, T=256, vocab 65, B=64
  gpt2_124m     12 layers, 12 heads, d=768, MLP 3072, T=1024,
                vocab 50257 padded to 50304, B=16
  gpt2_124m_accum  as gpt2_124m, 32 accumulated micro-batches of 16x1024
  speedrun_block   12 layers, 6 heads of 128, d=768, T=2048, vocab 50304, B=8,
                RoPE, QK-RMSNorm, ReLU^2 MLP, windows 256/2048, softcap 30,
                zero-init output projections, no learned position table

Input recipes:
  * tiny_fp32: tokens and targets i.i.d. uniform on [0, 65), independent.
  * char_bf16: one Dirichlet(0.5) unigram law over 65 symbols; each step a
    fresh i.i.d. stream of B*T+1 ids, x = s[:-1], y = s[1:] (the shifted
    buffer of the lecture's Tiny-Shakespeare loader).
  * GPT-2 shapes: a stream of documents [EOT, w_1..w_n], n ~ Geometric(1/600)
    on {1,2,...}, w ~ Zipf(1.1) truncated to [0, 50255], EOT id 50256 only
    at document starts (the FineWeb-Edu shard convention); x/y as above.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, Tuple

import numpy as np

EOT_ID = 50256


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Model and optimiser hyper-parameters of one workload."""

    n_layer: int
    n_head: int
    n_embd: int
    mlp_hidden: int
    block_size: int
    vocab_size: int
    padded_vocab_size: int
    max_batch: int
    precision: str = "bf16"          # "fp32" or "bf16"
    pos_encoding: str = "learned"    # "learned" or "rope"
    qk_rmsnorm: bool = False
    mlp_act: str = "gelu_tanh"       # "gelu_tanh" or "relu2"
    window_even: int = 0             # 0 = plain causal
    window_odd: int = 0
    logit_softcap: float = 0.0       # 0 = off
    zero_init_proj: bool = False
    head_fp8: bool = False           # lm_head forward product on e4m3 operands
    ln_eps: float = 1e-5
    qk_norm_eps: float = 1e-6
    rope_base: float = 10000.0
    beta1: float = 0.9
    beta2: float = 0.95
    adam_eps: float = 1e-8
    weight_decay: float = 0.1
    max_grad_norm: float = 1.0
    init_std: float = 0.02

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    batch: int
    seq_len: int
    init_seed: int
    data_seed: int
    data: str                 # "uniform", "dirichlet", "zipf_eot"
    steps: int = 1
    accum: int = 1
    lr: float = 6e-4
    description: str = ""


TINY_FP32 = Workload(
    name="tiny_fp32",
    model=ModelConfig(n_layer=2, n_head=4, n_embd=64, mlp_hidden=256, block_size=64,
                      vocab_size=65, padded_vocab_size=65, max_batch=4, precision="fp32"),
    batch=4, seq_len=64, init_seed=1, data_seed=101, data="uniform",
    description="tiny GPT fp32: L2 H4 d64 F256 T64 V65 B4")

CHAR_BF16 = Workload(
    name="char_bf16",
    model=ModelConfig(n_layer=6, n_head=6, n_embd=384, mlp_hidden=1536, block_size=256,
                      vocab_size=65, padded_vocab_size=65, max_batch=64, precision="bf16"),
    batch=64, seq_len=256, init_seed=2, data_seed=102, data="dirichlet", steps=20,
    description="char-level GPT bf16: L6 H6 d384 F1536 T256 V65 B64, 20 warmup steps")

GPT2_124M = Workload(
    name="gpt2_124m",
    model=ModelConfig(n_layer=12, n_head=12, n_embd=768, mlp_hidden=3072, block_size=1024,
                      vocab_size=50257, padded_vocab_size=50304, max_batch=16, precision="bf16"),
    batch=16, seq_len=1024, init_seed=3, data_seed=103, data="zipf_eot",
    description="GPT-2 124M bf16: L12 H12 d768 F3072 T1024 V50257->50304 B16")

GPT2_124M_ACCUM = Workload(
    name="gpt2_124m_accum",
    model=GPT2_124M.model,
    batch=16, seq_len=1024, init_seed=4, data_seed=104, data="zipf_eot", accum=32,
    lr=5.9967893984e-4,
    description="GPT-2 124M full step: 32 x 16x1024 micro-batches, lr at step 1000")

SPEEDRUN_BLOCK = Workload(
    name="speedrun_block",
    model=ModelConfig(n_layer=12, n_head=6, n_embd=768, mlp_hidden=3072, block_size=2048,
                      vocab_size=50304, padded_vocab_size=50304, max_batch=8, precision="bf16",
                      pos_encoding="rope", qk_rmsnorm=True, mlp_act="relu2",
                      window_even=256, window_odd=2048, logit_softcap=30.0,
                      zero_init_proj=True),
    batch=8, seq_len=2048, init_seed=5, data_seed=105, data="zipf_eot",
    description="speedrun block bf16: L12 H6x128 d768 T2048 B8, RoPE, QK-RMSNorm, "
                "ReLU^2, windows 256/2048, softcap 30")

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY_FP32, CHAR_BF16, GPT2_124M, GPT2_124M_ACCUM, SPEEDRUN_BLOCK)}


# ----------------------------------------------------------------------------
# token generators
# ----------------------------------------------------------------------------

def uniform_tokens(rng: np.random.Generator, vocab: int, batch: int, seq: int
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Independent i.i.d. uniform tokens and targets in [0, vocab)."""
    x = rng.integers(0, vocab, size=(batch, seq), dtype=np.int64).astype(np.int32)
    y = rng.integers(0, vocab, size=(batch, seq), dtype=np.int64).astype(np.int32)
    return x, y


def dirichlet_unigram(rng: np.random.Generator, vocab: int, alpha: float = 0.5) -> np.ndarray:
    return rng.dirichlet(np.full(vocab, alpha))


def unigram_stream(rng: np.random.Generator, probs: np.ndarray, n: int) -> np.ndarray:
    return rng.choice(len(probs), size=n, p=probs).astype(np.int32)


class ZipfEotStream:
    """Endless token stream of documents [EOT, w_1..w_n].

    n ~ Geometric(p = 1/mean_len) on {1, 2, ...}; w ~ Zipf(s) truncated to
    [0, eot-1], i.e. P(k) proportional to (k+1)^-s.
    """

    def __init__(self, seed: int, s: float = 1.1, eot: int = EOT_ID, mean_len: float = 600.0):
        self.rng = np.random.default_rng(seed)
        ranks = np.arange(1, eot + 1, dtype=np.float64)
        w = ranks ** (-s)
        self.cdf = np.cumsum(w / w.sum())
        self.cdf[-1] = 1.0
        self.eot = eot
        self.p = 1.0 / mean_len
        self.buf = np.zeros(0, dtype=np.int32)

    def _more(self, n_min: int) -> None:
        parts = [self.buf]
        have = len(self.buf)
        while have < n_min:
            n = int(self.rng.geometric(self.p))
            u = self.rng.random(n)
            words = np.searchsorted(self.cdf, u, side="right").astype(np.int32)
            words = np.minimum(words, self.eot - 1)
            doc = np.empty(n + 1, dtype=np.int32)
            doc[0] = self.eot
            doc[1:] = words
            parts.append(doc)
            have += n + 1
        self.buf = np.concatenate(parts)

    def take(self, n: int) -> np.ndarray:
        """Next n tokens, advancing the stream by n."""
        if len(self.buf) < n:
            self._more(n)
        out, self.buf = self.buf[:n].copy(), self.buf[n:]
        return out

    def peek(self, n: int) -> np.ndarray:
        if len(self.buf) < n:
            self._more(n)
        return self.buf[:n].copy()

    def next_batch(self, batch: int, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """x = buf[:-1], y = buf[1:] for a B*T+1 window; the stream advances B*T."""
        buf = self.peek(batch * seq + 1)
        self.take(batch * seq)
        return buf[:-1].reshape(batch, seq), buf[1:].reshape(batch, seq)


def batches(w: Workload, batch: int | None = None, seq: int | None = None
            ) -> Iterator[Tuple[np.ndarray, np.ndarray]]:
    """Endless iterator of (tokens, targets) int32 [B, T] for a workload."""
    B = w.batch if batch is None else batch
    T = w.seq_len if seq is None else seq
    rng = np.random.default_rng(w.data_seed)
    if w.data == "uniform":
        while True:
            yield uniform_tokens(rng, w.model.vocab_size, B, T)
    elif w.data == "dirichlet":
        p = dirichlet_unigram(rng, w.model.vocab_size)
        while True:
            s = unigram_stream(rng, p, B * T + 1)
            yield s[:-1].reshape(B, T), s[1:].reshape(B, T)
    elif w.data == "zipf_eot":
        stream = ZipfEotStream(w.data_seed)
        while True:
            yield stream.next_batch(B, T)
    else:
        raise ValueError(f"unknown data recipe {w.data!r}")


def dirichlet_probs(w: Workload) -> np.ndarray:
    """The unigram law the dirichlet recipe draws for this workload."""
    rng = np.random.default_rng(w.data_seed)
    return dirichlet_unigram(rng, w.model.vocab_size)


def repeated_sequence_batch(w: Workload, batch: int | None = None, seq: int | None = None
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """A batch whose rows are all the first sequence of the workload's stream.

    The mean loss and every gradient of such a batch equal those of the single
    sequence, so a full-size GPU step can be checked against a one-sequence
    CPU computation.
    """
    B = w.batch if batch is None else batch
    x, y = next(batches(w, 1, seq))
    return np.repeat(x, B, axis=0), np.repeat(y, B, axis=0)
