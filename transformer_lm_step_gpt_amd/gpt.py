"""ctypes binding of libgpt.so (include/gpt.h, include/gpt_testing.h).

Argument marshalling only: every step of the training step runs in the
library's HIP kernels. PyTorch supplies device memory (the workspace and the
token buffers) and the HIP stream (torch's current stream).
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p
from typing import Dict, List, Optional, Tuple, Union

import numpy as np

from .inputs import ModelConfig

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpt.so")

GPT_OK = 0
STATUS_NAMES = {
    0: "GPT_OK", -1: "GPT_ERR_INVALID_ARGUMENT", -2: "GPT_ERR_WORKSPACE_TOO_SMALL", -3: "GPT_ERR_UNSUPPORTED",
    -4: "GPT_ERR_DEVICE", -5: "GPT_ERR_TOKEN_RANGE", -6: "GPT_ERR_NONFINITE",
}


class GptError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")


class GptConfig(ctypes.Structure):
    _fields_ = [
        ("n_layer", c_int32), ("n_head", c_int32), ("n_embd", c_int32), ("mlp_hidden", c_int32),
        ("block_size", c_int32), ("vocab_size", c_int32), ("padded_vocab_size", c_int32), ("max_batch", c_int32),
        ("precision", c_int32), ("pos_encoding", c_int32), ("qk_rmsnorm", c_int32), ("mlp_act", c_int32),
        ("window_even", c_int32), ("window_odd", c_int32), ("zero_init_proj", c_int32), ("head_fp8", c_int32),
        ("ln_eps", c_float), ("qk_norm_eps", c_float), ("rope_base", c_float), ("logit_softcap", c_float),
        ("beta1", c_float), ("beta2", c_float), ("adam_eps", c_float), ("weight_decay", c_float),
        ("max_grad_norm", c_float), ("reserved1", c_int32), ("init_std", c_double),
    ]


def to_c_config(cfg: ModelConfig) -> GptConfig:
    c = GptConfig()
    for f in ("n_layer", "n_head", "n_embd", "mlp_hidden", "block_size", "vocab_size", "padded_vocab_size",
              "max_batch", "window_even", "window_odd"):
        setattr(c, f, int(getattr(cfg, f)))
    c.precision = {"fp32": 0, "bf16": 1}[cfg.precision]
    c.pos_encoding = {"learned": 0, "rope": 1}[cfg.pos_encoding]
    c.qk_rmsnorm = int(cfg.qk_rmsnorm)
    c.mlp_act = {"gelu_tanh": 0, "relu2": 1}[cfg.mlp_act]
    c.zero_init_proj = int(cfg.zero_init_proj)
    c.head_fp8 = int(getattr(cfg, "head_fp8", False))
    for f in ("ln_eps", "qk_norm_eps", "rope_base", "logit_softcap", "beta1", "beta2", "adam_eps", "weight_decay",
              "max_grad_norm", "init_std"):
        setattr(c, f, float(getattr(cfg, f)))
    return c


_lib = None

# (name, restype, argtypes) of every exported function
_SIGS = [
    ("gpt_config_default", c_int32, [POINTER(GptConfig)]),
    ("gpt_workspace_bytes", c_int32, [POINTER(GptConfig), POINTER(c_size_t)]),
    ("gpt_create", c_int32, [POINTER(GptConfig), c_uint64, c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    ("gpt_destroy", c_int32, [c_void_p]),
    ("gpt_set_stream", c_int32, [c_void_p, c_void_p]),
    ("gpt_forward_backward", c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_float, POINTER(c_float)]),
    ("gpt_loss_accum", c_int32, [c_void_p, POINTER(c_float)]),
    ("gpt_clip_and_adamw", c_int32, [c_void_p, c_float, c_int32, POINTER(c_float)]),
    ("gpt_clip_and_muon", c_int32, [c_void_p, c_float, c_float, c_float, c_int32, POINTER(c_float)]),
    ("gpt_generate", c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float, c_int32, c_uint64, c_void_p,
                               c_void_p]),
    ("gpt_num_tensors", c_int32, [c_void_p, POINTER(c_int32)]),
    ("gpt_tensor_info", c_int32, [c_void_p, c_int32, POINTER(c_char_p), POINTER(c_int32), POINTER(c_int64),
                                  POINTER(c_int32)]),
    ("gpt_get_param", c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int32]),
    ("gpt_set_param", c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int32]),
    ("gpt_get_grad", c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int32]),
    ("gpt_set_grad", c_int32, [c_void_p, c_int32, c_void_p, c_int64, c_int32]),
    ("gpt_get_opt_state", c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int64, c_int32]),
    ("gpt_set_opt_state", c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int64, c_int32]),
    ("gpt_get_row_losses", c_int32, [c_void_p, c_void_p, c_int64, c_int32]),
    ("gpt_lr_schedule", c_double, [c_int32, c_int32, c_int32, c_double, c_double]),
    ("gpt_status_string", c_char_p, [c_int32]),
    ("gpt_last_error", c_char_p, [c_void_p]),
    ("gpt_set_kernel_timing", c_int32, [c_void_p, c_int32]),
    ("gpt_reset_kernel_timing", c_int32, [c_void_p]),
    ("gpt_num_kernel_classes", c_int32, [POINTER(c_int32)]),
    ("gpt_kernel_timing", c_int32, [c_void_p, c_int32, POINTER(c_char_p), POINTER(c_double), POINTER(c_int64),
                                    POINTER(c_double), POINTER(c_double)]),
    ("gpt_set_kernel_timing_filter", c_int32, [c_void_p, c_char_p]),
    ("gpt_num_kernel_names", c_int32, [c_void_p, POINTER(c_int32)]),
    ("gpt_kernel_name_timing", c_int32, [c_void_p, c_int32, POINTER(c_char_p), POINTER(c_double), POINTER(c_int64),
                                         POINTER(c_double), POINTER(c_double)]),
    # test-only kernel entry points
    ("gptk_gemm_force_config", c_int32, [c_int32, c_int32]),
    ("gptk_gemm_num_configs", c_int32, []),
    ("gptk_gemm_tune", c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    ("gptk_gemm", c_int32, [c_int32, c_int32, c_int32, c_void_p, c_int64, c_int32, c_void_p, c_int64, c_int32,
                            c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_void_p, c_int64, c_void_p]),
    ("gptk_gemm_colsum", c_int32, [c_int32, c_int32, c_int32, c_void_p, c_int64, c_int32, c_void_p, c_int64, c_int32,
                                   c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    ("gptk_attention", c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                 c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    ("gptk_attention_bwd_colsum", c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                            c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                            c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    ("gptk_attention_colsum_partial_floats", c_int64, [c_int32, c_int32, c_int32, c_int32]),
    ("gptk_layernorm", c_int32, [c_int32, c_int32, c_int32, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_int32, c_void_p]),
    ("gptk_layernorm_partial_floats", c_int64, [c_int32, c_int32]),
    ("gptk_layernorm_bwd_noalloc", c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                             c_void_p]),
    ("gptk_layernorm_noalloc_max_floats", c_int64, []),
    ("gptk_qk_prep", c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_double,
                               c_int32, c_int32, c_float, c_int32, c_void_p]),
    ("gptk_cross_entropy", c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_float, c_float, c_void_p,
                                     c_int32, c_void_p]),
    ("gptk_embed_bwd", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                 c_void_p, c_void_p]),
    ("gptk_embed_bwd_scratch_bytes", c_int64, [c_int32, c_int32]),
    ("gptk_gemm_fp8", c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                c_void_p]),
    ("gptk_gemm_fp8_scratch_bytes", c_int64, [c_int32, c_int32, c_int32]),
    ("gptk_muon_orthogonalize", c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_int64,
                                          c_void_p]),
    ("gptk_muon_scratch_bytes", c_int64, [c_int32, c_int32, c_int32]),
    ("gptk_colsum", c_int32, [c_int32, c_int32, c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
    ("gptk_colsum_partial_floats", c_int64, [c_int32, c_int32]),
    ("gptk_sample", c_int32, [c_void_p, c_int32, c_int32, c_float, c_float, c_int32, c_uint64, c_int32, c_void_p,
                              c_void_p]),
]

EXPORTED = [s[0] for s in _SIGS]


def load_library(path: str = LIB_PATH):
    """Load libgpt.so (built by transformer_lm_step_gpt_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m transformer_lm_step_gpt_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in _SIGS:
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def check(status: int, handle=None) -> None:
    if status != GPT_OK:
        lib = load_library()
        msg = lib.gpt_last_error(handle).decode() if handle else lib.gpt_status_string(status).decode()
        raise GptError(status, msg)


def workspace_bytes(cfg: ModelConfig) -> int:
    lib = load_library()
    n = c_size_t()
    c = to_c_config(cfg)
    check(lib.gpt_workspace_bytes(byref(c), byref(n)))
    return n.value


def lr_schedule(it: int, warmup: int = 715, max_steps: int = 19073, max_lr: float = 6e-4,
                min_lr: float = 6e-5) -> float:
    return load_library().gpt_lr_schedule(it, warmup, max_steps, max_lr, min_lr)


def _ptr(t) -> int:
    return t.data_ptr()


class GPT:
    """One model in a torch-allocated device workspace, driven through the C ABI."""

    def __init__(self, cfg: ModelConfig, seed: int, device=None):
        import torch
        self.torch = torch
        self.lib = load_library()
        self.cfg = cfg
        self.device = torch.device(device if device is not None else "cuda")
        c = to_c_config(cfg)
        self._ccfg = c
        n = c_size_t()
        check(self.lib.gpt_workspace_bytes(byref(c), byref(n)))
        self.workspace = torch.empty(n.value, dtype=torch.uint8, device=self.device)
        h = c_void_p()
        check(self.lib.gpt_create(byref(c), c_uint64(seed), _ptr(self.workspace), n.value, self._stream(), byref(h)))
        self.handle = h
        cnt = c_int32()
        check(self.lib.gpt_num_tensors(h, byref(cnt)))
        self.names: List[str] = []
        self.shapes: List[Tuple[int, ...]] = []
        self.decay: List[bool] = []
        for i in range(cnt.value):
            name = c_char_p()
            nd = c_int32()
            shp = (c_int64 * 2)()
            dec = c_int32()
            check(self.lib.gpt_tensor_info(h, i, byref(name), byref(nd), shp, byref(dec)))
            self.names.append(name.value.decode())
            self.shapes.append(tuple(int(shp[j]) for j in range(nd.value)))
            self.decay.append(bool(dec.value))
        self.index: Dict[str, int] = {n_: i for i, n_ in enumerate(self.names)}

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _sync_stream(self):
        check(self.lib.gpt_set_stream(self.handle, self._stream()), self.handle)

    def close(self):
        if getattr(self, "handle", None):
            self.lib.gpt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ step
    def _device_tokens(self, a):
        torch = self.torch
        if isinstance(a, np.ndarray):
            a = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
        if a.dtype != torch.int32 or a.device != self.device or not a.is_contiguous():
            a = a.to(device=self.device, dtype=torch.int32).contiguous()
        return a

    def forward_backward(self, tokens, targets, grad_scale: float = 1.0, sync: bool = True) -> Optional[float]:
        self._sync_stream()
        tok = self._device_tokens(tokens)
        tgt = self._device_tokens(targets)
        B, T = tok.shape
        self._keep = (tok, tgt)
        loss = c_float()
        st = self.lib.gpt_forward_backward(self.handle, _ptr(tok), _ptr(tgt), B, T, grad_scale,
                                           byref(loss) if sync else None)
        check(st, self.handle)
        return loss.value if sync else None

    def clip_and_adamw(self, lr: float, step: int, sync: bool = True) -> Optional[float]:
        self._sync_stream()
        norm = c_float()
        check(self.lib.gpt_clip_and_adamw(self.handle, lr, step, byref(norm) if sync else None), self.handle)
        return norm.value if sync else None

    def clip_and_muon(self, lr: float, muon_lr: float, muon_momentum: float, step: int,
                      sync: bool = True) -> Optional[float]:
        """Clip, Muon on the hidden matrices, AdamW on the rest (gpt_clip_and_muon)."""
        self._sync_stream()
        norm = c_float()
        check(self.lib.gpt_clip_and_muon(self.handle, lr, muon_lr, muon_momentum, step,
                                         byref(norm) if sync else None), self.handle)
        return norm.value if sync else None

    def generate(self, prompt, n_new: int, temperature: float = 1.0, top_k: int = 50, seed: int = 0,
                 return_logits: bool = False):
        """Sampling with the key/value cache (gpt_generate): returns int32
        [B, T0 + n_new] (numpy) and, on request, the fp32 logits of every draw
        [n_new, B, padded_vocab_size]."""
        torch = self.torch
        self._sync_stream()
        p = self._device_tokens(prompt)
        B, T0 = p.shape
        out = torch.empty((B, T0 + n_new), dtype=torch.int32, device=self.device)
        lg = (torch.empty((n_new, B, self.cfg.padded_vocab_size), dtype=torch.float32, device=self.device)
              if return_logits else None)
        check(self.lib.gpt_generate(self.handle, _ptr(p), B, T0, n_new, temperature, top_k, c_uint64(seed),
                                    _ptr(out), _ptr(lg) if lg is not None else None), self.handle)
        toks = out.cpu().numpy()
        return (toks, lg.cpu().numpy()) if return_logits else toks

    def loss_accum(self) -> float:
        out = c_float()
        check(self.lib.gpt_loss_accum(self.handle, byref(out)), self.handle)
        return out.value

    def row_losses(self, B: int, T: int) -> np.ndarray:
        buf = np.empty(B * T, dtype=np.float32)
        check(self.lib.gpt_get_row_losses(self.handle, buf.ctypes.data, buf.size, 0), self.handle)
        return buf.reshape(B, T)

    # ------------------------------------------------------------------ tensors
    def _idx(self, key: Union[int, str]) -> int:
        return self.index[key] if isinstance(key, str) else int(key)

    def _get(self, fn, key) -> np.ndarray:
        i = self._idx(key)
        out = np.empty(self.shapes[i], dtype=np.float32)
        check(fn(self.handle, i, out.ctypes.data, out.size, 0), self.handle)
        return out

    def _set(self, fn, key, arr) -> None:
        i = self._idx(key)
        a = np.ascontiguousarray(arr, dtype=np.float32)
        if a.shape != self.shapes[i]:
            raise ValueError(f"{self.names[i]}: shape {a.shape} != {self.shapes[i]}")
        check(fn(self.handle, i, a.ctypes.data, a.size, 0), self.handle)

    def get_param(self, key) -> np.ndarray:
        self._sync_stream()
        return self._get(self.lib.gpt_get_param, key)

    def set_param(self, key, arr) -> None:
        self._sync_stream()
        self._set(self.lib.gpt_set_param, key, arr)

    def get_grad(self, key) -> np.ndarray:
        self._sync_stream()
        return self._get(self.lib.gpt_get_grad, key)

    def set_grad(self, key, arr) -> None:
        self._sync_stream()
        self._set(self.lib.gpt_set_grad, key, arr)

    def get_opt_state(self, key) -> Tuple[np.ndarray, np.ndarray]:
        self._sync_stream()
        i = self._idx(key)
        m = np.empty(self.shapes[i], dtype=np.float32)
        v = np.empty(self.shapes[i], dtype=np.float32)
        check(self.lib.gpt_get_opt_state(self.handle, i, m.ctypes.data, v.ctypes.data, m.size, 0), self.handle)
        return m, v

    def params(self) -> Dict[str, np.ndarray]:
        return {n: self.get_param(n) for n in self.names}

    def grads(self) -> Dict[str, np.ndarray]:
        return {n: self.get_grad(n) for n in self.names}

    def set_params(self, params: Dict[str, np.ndarray]) -> None:
        for n, a in params.items():
            self.set_param(n, a)

    # ------------------------------------------------------------------ timing
    def set_kernel_timing(self, mask: int) -> None:
        check(self.lib.gpt_set_kernel_timing(self.handle, mask), self.handle)

    def reset_kernel_timing(self) -> None:
        check(self.lib.gpt_reset_kernel_timing(self.handle), self.handle)

    def kernel_timing(self) -> List[dict]:
        n = c_int32()
        check(self.lib.gpt_num_kernel_classes(byref(n)))
        out = []
        for i in range(n.value):
            name = c_char_p()
            ms, fl, by = c_double(), c_double(), c_double()
            launches = c_int64()
            check(self.lib.gpt_kernel_timing(self.handle, i, byref(name), byref(ms), byref(launches), byref(fl),
                                             byref(by)), self.handle)
            out.append({"class": i, "name": name.value.decode(), "ms": ms.value, "launches": launches.value,
                        "flops": fl.value, "bytes": by.value})
        return out

    def set_kernel_timing_filter(self, kernel_name) -> None:
        """Also time every launch of this kernel instantiation (None: none)."""
        arg = kernel_name.encode() if kernel_name else None
        check(self.lib.gpt_set_kernel_timing_filter(self.handle, arg), self.handle)

    def kernel_name_timing(self) -> List[dict]:
        """Per kernel name: summed event time, launches, FLOPs and bytes of the timed launches."""
        n = c_int32()
        check(self.lib.gpt_num_kernel_names(self.handle, byref(n)), self.handle)
        out = []
        for i in range(n.value):
            name, ms, launches, fl, by = c_char_p(), c_double(), c_int64(), c_double(), c_double()
            check(self.lib.gpt_kernel_name_timing(self.handle, i, byref(name), byref(ms), byref(launches), byref(fl),
                                                  byref(by)), self.handle)
            out.append({"name": name.value.decode(), "ms": ms.value, "launches": launches.value, "flops": fl.value,
                        "bytes": by.value})
        return out
