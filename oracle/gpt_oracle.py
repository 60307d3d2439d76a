"""CPU float64 oracle for one GPT-2-style training step.

TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it and
shares no code with it; the two meet only through seeded inputs.

What it computes, as plainly as possible (NumPy float64, explicit T x T
scores and probabilities, explicit per-layer loops, hand-derived backward):

  forward   x0 = wte[tok] + wpe[t]                                 (1)
            per block:  x += attn(LN1(x));  x += mlp(LN2(x))        (2)
            z = LN_f(x) . wte^T     (tied head, no bias)            (3)
            loss = mean_m [ logsumexp(z_m) - z_m[y_m] ]             (4)
  backward  chain rule through (1)-(4), grads scaled by grad_scale
  update    global L2 clip, then AdamW with decay on 2-D tensors

Sources (page title, section):
  * "Zero to Hero, lecture 9: reproducing GPT-2 (124M)" (ai.flicky.cc) --
    "Раздел 1 / Архитектура" (pre-LN block, GELU tanh approximation, final
    LayerNorm, fused c_attn with heads as a batch dimension),
    "Генерация и устройство" (token + position embeddings, lm_head),
    "Связанные веса и инициализация" (tied wte/lm_head whose gradient is the
    sum of both uses; N(0, 0.02) init, residual writers scaled by
    (2 n_layer)^-1/2, zero biases),
    "Оптимизатор, клиппинг, расписание" (AdamW betas 0.9/0.95, eps 1e-8,
    global clip at 1.0, warmup + cosine schedule, decay 0.1 on 2-D tensors),
    "Накопление градиентов" (loss divided by the number of micro-steps).
  * "NanoGPT Speedrun baseline" (cruxr.ai) -- "El Mecanismo de Atención"
    (softmax(QK^T/sqrt(d_k))V with Attn_ij = 0 for j > i),
    "Configuración del Entrenamiento" (AdamW, clip, zero_grad loop).
  * "Un GPT desde cero + nanoGPT" (cursos.romerolabs.dev) -- 2.1/2.2
    (pre-norm block, mean cross-entropy over B*T, tied head).
  * Modded-NanoGPT README (oa0.com) -- technique list: rotary positions,
    QK-Norm, ReLU^2, logit softcap, zero-initialised projections, long/short
    sliding-window attention. The README names these without formulas; the
    readings used here are stated at each function.
  * Sampling (generate): "Un GPT desde cero + nanoGPT" 2.1 (autoregressive
    generate: last position's logits divided by the temperature, softmax, one
    draw, append, repeat; 0 temperature = greedy) and the lecture's
    "Генерация и устройство" (top-k sampling with k = 50).
  * Muon (the hidden matrices' optimiser): the Modded-NanoGPT README's
    technique list names it and links its article; the pages give no formula,
    so the steps follow that article (K. Jordan et al., "Muon: An optimizer for
    hidden layers in neural networks", 2024): Nesterov momentum, then the
    quintic Newton-Schulz orthogonalisation, then a step scaled by
    sqrt(max(1, rows / cols)); every other tensor keeps AdamW.

Random initialisation uses Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11) and the Box-Muller
transform (Box and Muller, 1958), implemented here from those definitions.
"""

from __future__ import annotations

import math
from typing import Dict, List, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# Philox4x64-10 counter-based generator and Box-Muller normals
# ----------------------------------------------------------------------------

_PHILOX_M0 = 0xD2E7470EE14C6C93
_PHILOX_M1 = 0xCA5A826395121157
_PHILOX_W0 = 0x9E3779B97F4A7C15   # golden ratio Weyl increment
_PHILOX_W1 = 0xBB67AE8584CAA73B   # sqrt(3) - 1 Weyl increment
_U64 = np.uint64
_LO32 = _U64(0xFFFFFFFF)


def _mulhilo64(a: np.ndarray, m: int) -> Tuple[np.ndarray, np.ndarray]:
    """High and low 64-bit halves of the 128-bit product a * m (a uint64 array)."""
    b = _U64(m)
    a_lo, a_hi = a & _LO32, a >> _U64(32)
    b_lo, b_hi = b & _LO32, b >> _U64(32)
    ll = a_lo * b_lo
    hl = a_hi * b_lo
    lh = a_lo * b_hi
    hh = a_hi * b_hi
    mid = (ll >> _U64(32)) + (hl & _LO32) + lh          # < 2^64, no overflow
    hi = hh + (hl >> _U64(32)) + (mid >> _U64(32))
    lo = a * b
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x64 with 10 rounds on arrays of counters; returns 4 uint64 arrays.

    One round maps (c0, c1, c2, c3) with key (k0, k1) to
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
    the key is advanced by the two Weyl constants between rounds.
    """
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
        ka, kb = _U64(k0 & (2**64 - 1)), _U64(k1 & (2**64 - 1))
        for r in range(10):
            if r:
                ka = _U64((int(ka) + _PHILOX_W0) & (2**64 - 1))
                kb = _U64((int(kb) + _PHILOX_W1) & (2**64 - 1))
            hi0, lo0 = _mulhilo64(c0, _PHILOX_M0)
            hi1, lo1 = _mulhilo64(c2, _PHILOX_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ ka, lo1, hi0 ^ c3 ^ kb, lo0
    return c0, c1, c2, c3


def _unit_open(w: np.ndarray) -> np.ndarray:
    """Top 53 bits of a uint64 word mapped to the open interval (0, 1)."""
    return ((w >> _U64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def standard_normals(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard normals for (seed, stream): element e comes from Philox block
    e // 4 (counter (e//4, 0, 0, 0), key (seed, stream)); the block's words
    (0,1) and (2,3) are Box-Muller pairs giving elements 4j..4j+3 as
    (r0 cos t0, r0 sin t0, r1 cos t1, r1 sin t1)."""
    nblk = (n + 3) // 4
    out = np.empty((nblk, 4), dtype=np.float64)
    chunk = 1 << 16          # blocks per pass, sized to stay cache resident
    for b0 in range(0, nblk, chunk):
        b1 = min(nblk, b0 + chunk)
        w0, w1, w2, w3 = philox4x64_10(np.arange(b0, b1, dtype=np.uint64), 0, 0, 0, seed, stream)
        for j, (wa, wb) in enumerate(((w0, w1), (w2, w3))):
            u1, u2 = _unit_open(wa), _unit_open(wb)
            r = np.sqrt(-2.0 * np.log(u1))
            t = 2.0 * math.pi * u2
            out[b0:b1, 2 * j] = r * np.cos(t)
            out[b0:b1, 2 * j + 1] = r * np.sin(t)
    return out.reshape(-1)[:n]


# ----------------------------------------------------------------------------
# parameter table
# ----------------------------------------------------------------------------

def param_table(cfg) -> List[Tuple[str, Tuple[int, ...], bool, str]]:
    """(name, shape, decayed, init-kind) for every parameter, canonical order.

    Names follow the lecture's Hugging-Face-compatible layer names; Linear
    weights are [out, in]. The tied wte/lm_head tensor appears once. Decay
    applies to every 2-D tensor (lecture, "Оптимизатор, клиппинг,
    расписание": matrices of linear layers and embeddings; biases and
    LayerNorm parameters are not decayed).
    init-kind: "normal" (std 0.02), "proj" (std 0.02/sqrt(2L), or zero for
    the zero-init variant), "zero", "one".
    """
    d, F, L, Vp = cfg.n_embd, cfg.mlp_hidden, cfg.n_layer, cfg.padded_vocab_size
    t = [("wte", (Vp, d), True, "normal")]
    if cfg.pos_encoding == "learned":
        t.append(("wpe", (cfg.block_size, d), True, "normal"))
    for l in range(L):
        p = f"h.{l}."
        t += [
            (p + "ln_1.weight", (d,), False, "one"),
            (p + "ln_1.bias", (d,), False, "zero"),
            (p + "attn.c_attn.weight", (3 * d, d), True, "normal"),
            (p + "attn.c_attn.bias", (3 * d,), False, "zero"),
            (p + "attn.c_proj.weight", (d, d), True, "proj"),
            (p + "attn.c_proj.bias", (d,), False, "zero"),
            (p + "ln_2.weight", (d,), False, "one"),
            (p + "ln_2.bias", (d,), False, "zero"),
            (p + "mlp.c_fc.weight", (F, d), True, "normal"),
            (p + "mlp.c_fc.bias", (F,), False, "zero"),
            (p + "mlp.c_proj.weight", (d, F), True, "proj"),
            (p + "mlp.c_proj.bias", (d,), False, "zero"),
        ]
    t += [("ln_f.weight", (d,), False, "one"), ("ln_f.bias", (d,), False, "zero")]
    return t


def init_params(cfg, seed: int) -> Dict[str, np.ndarray]:
    """Initial parameters (float32 values held in float64 arrays).

    Tensor i of the table draws its normals from stream i of the seed.
    """
    out = {}
    L = cfg.n_layer
    for i, (name, shape, _decay, kind) in enumerate(param_table(cfg)):
        n = int(np.prod(shape))
        if kind == "one":
            a = np.ones(n)
        elif kind == "zero" or (kind == "proj" and cfg.zero_init_proj):
            a = np.zeros(n)
        else:
            std = cfg.init_std * ((2.0 * L) ** -0.5 if kind == "proj" else 1.0)
            a = (std * standard_normals(seed, i, n)).astype(np.float32).astype(np.float64)
        out[name] = a.reshape(shape)
    return out


def zeros_like_params(params: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.zeros_like(v) for k, v in params.items()}


# ----------------------------------------------------------------------------
# building blocks (forward + backward)
# ----------------------------------------------------------------------------

def layernorm_fwd(x, g, b, eps):
    """LayerNorm over the last axis with the biased variance (nn.LayerNorm)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    return xhat * g + b, (xhat, rstd)


def layernorm_bwd(dy, cache, g):
    xhat, rstd = cache
    dxhat = dy * g
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                 - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    red = tuple(range(dy.ndim - 1))
    return dx, (dy * xhat).sum(axis=red), dy.sum(axis=red)


_GELU_C = math.sqrt(2.0 / math.pi)


def gelu_tanh(x):
    """GELU, tanh approximation (Hendrycks and Gimpel): 0.5 x (1 + tanh(u)),
    u = sqrt(2/pi) (x + 0.044715 x^3) -- the variant the lecture keeps."""
    return 0.5 * x * (1.0 + np.tanh(_GELU_C * (x + 0.044715 * x ** 3)))


def gelu_tanh_grad(x):
    u = _GELU_C * (x + 0.044715 * x ** 3)
    t = np.tanh(u)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * _GELU_C * (1.0 + 3.0 * 0.044715 * x * x)


def relu2(x):
    """ReLU^2 (speedrun MLP activation): max(x, 0)^2."""
    r = np.maximum(x, 0.0)
    return r * r


def relu2_grad(x):
    return 2.0 * np.maximum(x, 0.0)


def rmsnorm_fwd(x, eps):
    """Parameter-free RMS normalisation over the last axis: x (mean(x^2)+eps)^-1/2
    (the reading used for the speedrun's QK-Norm)."""
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x * r, r


def rmsnorm_bwd(dy, y, r):
    return r * (dy - y * (dy * y).mean(axis=-1, keepdims=True))


def rope_tables(T, hd, base):
    """cos/sin [T, hd/2] for rotary positions: angle p * base^(-2i/hd)."""
    half = hd // 2
    inv = base ** (-2.0 * np.arange(half) / hd)
    ang = np.arange(T)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope_fwd(x, cos, sin):
    """Rotate-half pairing: (x_i, x_{i+hd/2}) rotated by the angle of pair i."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def rope_bwd(dy, cos, sin):
    """Transpose of the rotation (rotation by the negative angle)."""
    half = dy.shape[-1] // 2
    da, db = dy[..., :half], dy[..., half:]
    return np.concatenate([da * cos + db * sin, -da * sin + db * cos], axis=-1)


def attention_mask(T, window):
    """allowed[i, j]: key j is visible to query i iff j <= i and, with a
    window W > 0, i - j < W."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    ok = j <= i
    if window:
        ok &= (i - j) < window
    return ok


def attention_fwd(q, k, v, window):
    """q, k, v: [B, H, T, hd]. Explicit scores, explicit softmax, explicit P."""
    hd = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    ok = attention_mask(q.shape[2], window)
    s = np.where(ok, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.matmul(p, v), p


def attention_bwd(do, q, k, v, p):
    hd = q.shape[-1]
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) / math.sqrt(hd)
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) / math.sqrt(hd)
    return dq, dk, dv


def cross_entropy_fwd_bwd(z, y, scale):
    """Mean cross-entropy over rows and its gradient (softmax - onehot) * scale / M."""
    M = z.shape[0]
    zmax = z.max(axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    se = e.sum(axis=-1, keepdims=True)
    lse = (np.log(se) + zmax)[:, 0]
    rows = np.arange(M)
    losses = lse - z[rows, y]
    dz = e / se
    dz[rows, y] -= 1.0
    dz *= scale / M
    return losses, dz


# ----------------------------------------------------------------------------
# FP8 head (speedrun technique list: FP8 matmul for the output head)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3(x):
    """Round to the nearest OCP FP8 E4M3 value, ties to even: 3 mantissa bits,
    exponent bias 7, normal numbers down to 2^-6, subnormal steps of 2^-9,
    largest finite 448 (no infinities; larger magnitudes saturate to 448)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = 2.0 ** (np.maximum(e, -6.0) - 3.0)      # spacing of the binade holding a
    q = np.minimum(np.round(a / step) * step, E4M3_MAX)   # numpy rounds halves to even
    return np.copysign(q, x)


def fp8_scale(t):
    """Per-tensor scale 448 / max|t| in fp32 (1 for an all-zero tensor)."""
    amax = np.float32(np.abs(np.asarray(t)).max())
    return np.float32(1.0) if amax == 0 else np.float32(E4M3_MAX) / amax


def fp8_quantize(t, s):
    """e4m3 codes of t * s with the product rounded to fp32 first; returned as values."""
    return e4m3(np.asarray(t).astype(np.float32) * np.float32(s))


def fp8_head_logits(xf, wte):
    """z = xf wte^T with both operands quantised to e4m3 under per-tensor scales
    s_x = 448 / max|xf|, s_w = 448 / max|wte| (a reading: the README names the
    technique and an asymmetric rescale but no recipe), the products summed
    exactly and the result divided by s_x s_w."""
    sx, sw = fp8_scale(xf), fp8_scale(wte)
    return (fp8_quantize(xf, sx) @ fp8_quantize(wte, sw).T) / (np.float64(sx) * np.float64(sw))


# ----------------------------------------------------------------------------
# model forward + backward
# ----------------------------------------------------------------------------

def _window(cfg, layer):
    return cfg.window_even if layer % 2 == 0 else cfg.window_odd


def forward_backward(params, tokens, targets, cfg, grad_scale=1.0, want_grads=True,
                     return_logits=False, progress=None):
    """One micro-step. Returns (mean loss, grads or None, extras).

    grads are grad_scale * d(mean loss)/d(param). extras holds the per-row
    losses and, on request, the logits. progress, if given, is called with a
    short message after each layer (long runs report as they go).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    targets = np.asarray(targets, dtype=np.int64)
    B, T = tokens.shape
    d, H, L = cfg.n_embd, cfg.n_head, cfg.n_layer
    hd = d // H
    M = B * T
    if T > cfg.block_size:
        raise ValueError("sequence longer than block_size")
    rope = cfg.pos_encoding == "rope"
    if rope:
        cos, sin = rope_tables(T, hd, cfg.rope_base)

    wte = params["wte"]
    x = wte[tokens]
    if not rope:
        x = x + params["wpe"][:T][None]
    x = x.reshape(M, d)

    def heads(a):   # [M, d] -> [B, H, T, hd]
        return a.reshape(B, T, H, hd).transpose(0, 2, 1, 3)

    def merge(a):   # [B, H, T, hd] -> [M, d]
        return a.transpose(0, 2, 1, 3).reshape(M, d)

    caches = []
    for l in range(L):
        p = f"h.{l}."
        c = {}
        a1, c["ln1"] = layernorm_fwd(x, params[p + "ln_1.weight"], params[p + "ln_1.bias"], cfg.ln_eps)
        qkv = a1 @ params[p + "attn.c_attn.weight"].T + params[p + "attn.c_attn.bias"]
        q, k, v = heads(qkv[:, :d]), heads(qkv[:, d:2 * d]), heads(qkv[:, 2 * d:])
        if cfg.qk_rmsnorm:
            q, c["rq"] = rmsnorm_fwd(q, cfg.qk_norm_eps)
            k, c["rk"] = rmsnorm_fwd(k, cfg.qk_norm_eps)
            c["qn"], c["kn"] = q, k
        if rope:
            q, k = rope_fwd(q, cos, sin), rope_fwd(k, cos, sin)
        o, prob = attention_fwd(q, k, v, _window(cfg, l))
        o = merge(o)
        x = x + o @ params[p + "attn.c_proj.weight"].T + params[p + "attn.c_proj.bias"]
        a2, c["ln2"] = layernorm_fwd(x, params[p + "ln_2.weight"], params[p + "ln_2.bias"], cfg.ln_eps)
        hpre = a2 @ params[p + "mlp.c_fc.weight"].T + params[p + "mlp.c_fc.bias"]
        h = relu2(hpre) if cfg.mlp_act == "relu2" else gelu_tanh(hpre)
        x = x + h @ params[p + "mlp.c_proj.weight"].T + params[p + "mlp.c_proj.bias"]
        c.update(a1=a1, q=q, k=k, v=v, p=prob, o=o, a2=a2, hpre=hpre, h=h)
        caches.append(c)
        if progress:
            progress(f"oracle forward layer {l}")

    xf, lnf_cache = layernorm_fwd(x, params["ln_f.weight"], params["ln_f.bias"], cfg.ln_eps)
    # FP8 head: the forward product only; the backward takes the unquantised
    # operands (straight-through)
    zraw = fp8_head_logits(xf, wte) if getattr(cfg, "head_fp8", False) else xf @ wte.T
    cap = cfg.logit_softcap
    if cap:
        th = np.tanh(zraw / cap)
        z = cap * th
    else:
        z = zraw
    y = targets.reshape(M)
    losses, dz = cross_entropy_fwd_bwd(z, y, grad_scale)
    loss = float(losses.mean())
    extras = {"row_losses": losses.reshape(B, T)}
    if return_logits:
        extras["logits"] = z.reshape(B, T, -1)
    if not want_grads:
        return loss, None, extras

    g = zeros_like_params(params)
    if cap:
        dz = dz * (1.0 - th * th)
    dxf = dz @ wte
    g["wte"] += dz.T @ xf
    dx, g["ln_f.weight"], g["ln_f.bias"] = layernorm_bwd(dxf, lnf_cache, params["ln_f.weight"])

    for l in reversed(range(L)):
        p = f"h.{l}."
        c = caches[l]
        # MLP branch: x_out = x_mid + act(LN2(x_mid) Wfc^T + bfc) Wmp^T + bmp
        dh = dx @ params[p + "mlp.c_proj.weight"]
        g[p + "mlp.c_proj.weight"] = dx.T @ c["h"]
        g[p + "mlp.c_proj.bias"] = dx.sum(axis=0)
        act_grad = relu2_grad(c["hpre"]) if cfg.mlp_act == "relu2" else gelu_tanh_grad(c["hpre"])
        dhpre = dh * act_grad
        da2 = dhpre @ params[p + "mlp.c_fc.weight"]
        g[p + "mlp.c_fc.weight"] = dhpre.T @ c["a2"]
        g[p + "mlp.c_fc.bias"] = dhpre.sum(axis=0)
        dxl, g[p + "ln_2.weight"], g[p + "ln_2.bias"] = layernorm_bwd(da2, c["ln2"], params[p + "ln_2.weight"])
        dx = dx + dxl
        # attention branch: x_mid = x_in + attn(LN1(x_in)) Wproj^T + bproj
        do = dx @ params[p + "attn.c_proj.weight"]
        g[p + "attn.c_proj.weight"] = dx.T @ c["o"]
        g[p + "attn.c_proj.bias"] = dx.sum(axis=0)
        dq, dk, dv = attention_bwd(heads(do), c["q"], c["k"], c["v"], c["p"])
        if rope:
            dq, dk = rope_bwd(dq, cos, sin), rope_bwd(dk, cos, sin)
        if cfg.qk_rmsnorm:
            dq = rmsnorm_bwd(dq, c["qn"], c["rq"])
            dk = rmsnorm_bwd(dk, c["kn"], c["rk"])
        dqkv = np.concatenate([merge(dq), merge(dk), merge(dv)], axis=1)
        da1 = dqkv @ params[p + "attn.c_attn.weight"]
        g[p + "attn.c_attn.weight"] = dqkv.T @ c["a1"]
        g[p + "attn.c_attn.bias"] = dqkv.sum(axis=0)
        dxl, g[p + "ln_1.weight"], g[p + "ln_1.bias"] = layernorm_bwd(da1, c["ln1"], params[p + "ln_1.weight"])
        dx = dx + dxl
        if progress:
            progress(f"oracle backward layer {l}")

    # embeddings: the tied wte receives the lookup's gradient on top of the head's
    np.add.at(g["wte"], tokens.reshape(M), dx)
    if not rope:
        g["wpe"][:T] += dx.reshape(B, T, d).sum(axis=0)
    return loss, g, extras


# ----------------------------------------------------------------------------
# clip, AdamW, learning-rate schedule
# ----------------------------------------------------------------------------

def grad_norm(grads) -> float:
    """Global L2 norm over every (unique) parameter gradient."""
    return math.sqrt(sum(float(np.sum(g * g)) for g in grads.values()))


def clip_coefficient(norm: float, max_norm: float) -> float:
    """torch.nn.utils.clip_grad_norm_ semantics: min(1, max_norm / (norm + 1e-6))."""
    return min(1.0, max_norm / (norm + 1e-6))


def adamw_update(params, grads, m, v, lr, step, cfg, decay_flags, grad_coef=1.0):
    """AdamW with decoupled weight decay (the decay multiplies p by 1 - lr*wd
    for decayed tensors) and bias-corrected moments; eps outside the root.
    Returns new (params, m, v); inputs are not modified."""
    b1, b2, eps, wd = cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step
    P, Mn, Vn = {}, {}, {}
    for name, p in params.items():
        g = grads[name] * grad_coef
        mm = b1 * m[name] + (1.0 - b1) * g
        vv = b2 * v[name] + (1.0 - b2) * g * g
        pp = p * (1.0 - lr * wd) if decay_flags[name] else p.copy()
        pp = pp - lr * (mm / bc1) / (np.sqrt(vv / bc2) + eps)
        P[name], Mn[name], Vn[name] = pp, mm, vv
    return P, Mn, Vn


def get_lr(it, warmup_steps=715, max_steps=19073, max_lr=6e-4, min_lr=6e-5):
    """Linear warmup to max_lr over warmup_steps (lr = max_lr (it+1)/warmup),
    min_lr past max_steps, cosine decay in between (the lecture's final form)."""
    if it < warmup_steps:
        return max_lr * (it + 1) / warmup_steps
    if it > max_steps:
        return min_lr
    ratio = (it - warmup_steps) / (max_steps - warmup_steps)
    coeff = 0.5 * (1.0 + math.cos(math.pi * ratio))
    return min_lr + coeff * (max_lr - min_lr)


def decay_flags(cfg) -> Dict[str, bool]:
    return {name: dec for name, _s, dec, _k in param_table(cfg)}


def train_step(params, m, v, micro_batches, cfg, lr, step, progress=None, muon=None):
    """Full optimiser step: accumulate grads over the micro-batches with
    scale 1/k, clip at cfg.max_grad_norm, AdamW (or, with muon = (muon_lr,
    momentum), muon_update). Returns
    (mean loss, grad norm, grads (unclipped), new params, new m, new v)."""
    k = len(micro_batches)
    acc = zeros_like_params(params)
    loss_sum = 0.0
    for tok, tgt in micro_batches:
        loss, g, _ = forward_backward(params, tok, tgt, cfg, grad_scale=1.0 / k, progress=progress)
        loss_sum += loss
        for n in acc:
            acc[n] += g[n]
    norm = grad_norm(acc)
    coef = clip_coefficient(norm, cfg.max_grad_norm)
    if muon is None:
        P, Mn, Vn = adamw_update(params, acc, m, v, lr, step, cfg, decay_flags(cfg), grad_coef=coef)
    else:
        P, Mn, Vn = muon_update(params, acc, m, v, lr, step, cfg, muon[0], muon[1], grad_coef=coef)
    return loss_sum / k, norm, acc, P, Mn, Vn


# ----------------------------------------------------------------------------
# Muon for the hidden matrices
# ----------------------------------------------------------------------------

# Quintic Newton-Schulz coefficients of the Muon article (x -> a x + b x^3 + c x^5
# on the singular values), its five iterations and the normalisation epsilon.
MUON_NS_COEFFS = (3.4445, -4.7750, 2.0315)
MUON_NS_STEPS = 5
MUON_EPS = 1e-7


def newton_schulz5(G):
    """Approximate orthogonalisation (the U V^T of G = U S V^T) by the Muon
    article's iteration: G is taken wide (transposed when it has more rows than
    columns), divided by its Frobenius norm plus MUON_EPS, and then, five times,
    A = X X^T and X <- a X + (b A + c A A) X. The result is oriented back."""
    a, b, c = MUON_NS_COEFFS
    X = np.array(G, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X) + MUON_EPS)
    for _ in range(MUON_NS_STEPS):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def muon_tensors(cfg) -> List[str]:
    """The hidden matrices Muon updates: each block's qkv, attention-output,
    MLP-up and MLP-down weights. Embeddings (and the tied head), LayerNorm
    gains and biases keep AdamW."""
    out = []
    for l in range(cfg.n_layer):
        p = f"h.{l}."
        out += [p + "attn.c_attn.weight", p + "attn.c_proj.weight", p + "mlp.c_fc.weight", p + "mlp.c_proj.weight"]
    return out


def muon_update(params, grads, m, v, lr, step, cfg, muon_lr, muon_momentum, grad_coef=1.0):
    """One optimiser step with Muon on muon_tensors(cfg) and AdamW (adamw_update,
    learning rate lr) on the rest. For a hidden matrix W [r, c] with clipped
    gradient g and momentum buffer B (held where AdamW keeps its first moment):
        B <- mu B + g;   u = g + mu B   (Nesterov)
        W <- W - muon_lr sqrt(max(1, r / c)) NS5(u)
    with no weight decay; its second-moment buffer is left unchanged.
    Returns new (params, m, v); inputs are not modified."""
    hidden = set(muon_tensors(cfg))
    flags = decay_flags(cfg)
    rest = [n for n in params if n not in hidden]
    P, Mn, Vn = adamw_update({n: params[n] for n in rest}, grads, m, v, lr, step, cfg, flags, grad_coef=grad_coef)
    for n in hidden:
        g = grads[n] * grad_coef
        buf = muon_momentum * m[n] + g
        u = g + muon_momentum * buf
        r, c = params[n].shape
        P[n] = params[n] - muon_lr * math.sqrt(max(1.0, r / c)) * newton_schulz5(u)
        Mn[n] = buf
        Vn[n] = v[n].copy()
    return {n: P[n] for n in params}, {n: Mn[n] for n in params}, {n: Vn[n] for n in params}


# ----------------------------------------------------------------------------
# sampling (generate)
# ----------------------------------------------------------------------------

SAMPLE_STREAM = 0x73616D706C65   # Philox key word 1 of the sampling draws ("sample")


def sample_uniform(seed: int, step: int, row: int) -> float:
    """The uniform in (0, 1) of draw `step` of sequence `row`: word 0 of the
    Philox4x64-10 block with counter (step, row, 0, 0) and key
    (seed, SAMPLE_STREAM), top 53 bits mapped to the open interval."""
    w0, _, _, _ = philox4x64_10(np.array([step], dtype=np.uint64), np.array([row], dtype=np.uint64), 0, 0,
                                seed, SAMPLE_STREAM)
    return float(_unit_open(w0)[0])


def softcap(z, cap):
    """Speedrun logit softcap cap * tanh(z / cap) (cap 0: none)."""
    return cap * np.tanh(z / cap) if cap else z


def sample_next(z, temperature: float, top_k: int, u: float) -> int:
    """One draw from a row of logits z.

    temperature 0 is greedy (the first index of the maximum). Otherwise the
    probabilities are softmax(z / temperature); with 0 < top_k < len(z) only
    the top_k most probable tokens are kept (ties at the k-th value broken
    towards lower indices) and renormalised; the token is the first index i,
    in increasing token order, whose cumulative kept probability exceeds u.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if temperature == 0:
        return int(np.argmax(z))
    keep = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        order = np.lexsort((np.arange(V), -z))      # by value descending, then index ascending
        keep[:] = False
        keep[order[:top_k]] = True
    w = np.where(keep, np.exp((z - z.max()) / temperature), 0.0)
    c = np.cumsum(w)
    i = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(i, int(np.nonzero(keep)[0][-1]))


def generate(params, prompt, cfg, n_new: int, temperature: float, top_k: int, seed: int):
    """Autoregressive sampling with a full forward pass over the whole sequence
    at every step (no cache): returns (tokens [B, T0 + n_new], logits of each
    draw [n_new, B, Vp] after the softcap). The prompt plus the new tokens
    must fit in block_size (the pages crop longer contexts to block_size)."""
    seq = np.asarray(prompt, dtype=np.int64)
    B, T0 = seq.shape
    if T0 + n_new > cfg.block_size:
        raise ValueError("prompt + new tokens longer than block_size")
    logits = []
    for step in range(n_new):
        _, _, ex = forward_backward(params, seq, np.zeros_like(seq), cfg, want_grads=False, return_logits=True)
        z = ex["logits"][:, -1, :]          # the softcap is already applied
        logits.append(z)
        nxt = [sample_next(z[b], temperature, top_k, sample_uniform(seed, step, b)) for b in range(B)]
        seq = np.concatenate([seq, np.array(nxt, dtype=np.int64)[:, None]], axis=1)
    return seq.astype(np.int32), np.stack(logits) if logits else np.zeros((0, B, cfg.padded_vocab_size))

