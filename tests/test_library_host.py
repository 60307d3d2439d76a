"""Host-only checks of the C-ABI library: it loads, exports every function the
headers declare, and its pure-host calls (config, sizing, validation, LR
schedule, status text) behave as documented. No kernel is launched."""

import ctypes
import glob
import os
import re

import pytest

from transformer_lm_step_gpt_amd import gpt as G
from transformer_lm_step_gpt_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"\b(gptk?_[a-z0-9_]+)\s*\(", src):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    return G.load_library()


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert len(decl) >= 30
    for name in decl:
        assert hasattr(lib, name), name
    assert decl == set(G.EXPORTED), decl ^ set(G.EXPORTED)


def test_config_default_layout(lib):
    c = G.GptConfig()
    assert lib.gpt_config_default(ctypes.byref(c)) == 0
    assert (c.n_layer, c.n_head, c.n_embd, c.mlp_hidden) == (12, 12, 768, 3072)
    assert (c.block_size, c.vocab_size, c.padded_vocab_size, c.max_batch) == (1024, 50257, 50304, 16)
    assert c.precision == 1 and c.pos_encoding == 0 and c.mlp_act == 0
    assert abs(c.beta1 - 0.9) < 1e-7 and abs(c.beta2 - 0.95) < 1e-7 and abs(c.adam_eps - 1e-8) < 1e-15
    assert abs(c.weight_decay - 0.1) < 1e-7 and c.max_grad_norm == 1.0 and abs(c.ln_eps - 1e-5) < 1e-12
    assert c.init_std == 0.02                     # double field at the end of the struct
    ref = G.to_c_config(I.GPT2_124M.model)
    assert bytes(ref) == bytes(c) or all(getattr(ref, f) == getattr(c, f) for f, _ in G.GptConfig._fields_
                                         if not f.startswith("reserved") and f not in ("logit_softcap",))


def test_workspace_bytes_all_workloads():
    sizes = {w.name: G.workspace_bytes(w.model) for w in I.WORKLOADS.values()}
    assert sizes["tiny_fp32"] < 64 << 20
    # GPT-2 124M bf16: 4 fp32 copies of 124.5M params + activations, well inside 288 GB
    assert 8 << 30 < sizes["gpt2_124m"] < 40 << 30


@pytest.mark.parametrize("change,status", [
    (dict(n_head=5), -1),                       # 64 % 5 != 0
    (dict(n_head=1, n_embd=48, mlp_hidden=192), -3),   # head dim 48
    (dict(padded_vocab_size=10), -1),
    (dict(max_batch=1000), -3),                 # max_batch * block_size > 32768
    (dict(n_layer=0), -1),
    (dict(ln_eps=0.0), -1),
])
def test_validation_errors(lib, change, status):
    cfg = I.TINY_FP32.model.replace(**change)
    c = G.to_c_config(cfg)
    n = ctypes.c_size_t()
    assert lib.gpt_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == status


def test_null_arguments(lib):
    n = ctypes.c_size_t()
    assert lib.gpt_workspace_bytes(None, ctypes.byref(n)) == -1
    assert lib.gpt_forward_backward(None, None, None, 1, 1, 1.0, None) == -1
    assert lib.gpt_clip_and_adamw(None, 1e-3, 1, None) == -1
    c = G.to_c_config(I.TINY_FP32.model)
    h = ctypes.c_void_p()
    assert lib.gpt_create(ctypes.byref(c), 1, None, 0, None, ctypes.byref(h)) == -1


def test_lr_schedule_values():
    assert abs(G.lr_schedule(0) - 6e-4 / 715) < 1e-18
    assert G.lr_schedule(714) == pytest.approx(6e-4, rel=1e-15)
    assert G.lr_schedule(1000) == pytest.approx(5.9967893984e-4, rel=1e-10)
    assert G.lr_schedule(19074) == 6e-5
    for it in (0, 100, 714, 715, 716, 5000, 19073, 20000):
        from oracle.gpt_oracle import get_lr
        assert G.lr_schedule(it) == pytest.approx(get_lr(it), rel=1e-14)


def test_status_strings(lib):
    for s in range(-6, 1):
        assert lib.gpt_status_string(s).decode()
    n = ctypes.c_int32()
    assert lib.gpt_num_kernel_classes(ctypes.byref(n)) == 0 and n.value >= 10
