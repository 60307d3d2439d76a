"""Kernel-level parity: each kernel family of the training step, called
through the test-only C entry points, against the CPU oracle's float64
pieces on the same seeded inputs (sizes span several tiles plus a ragged
tail)."""

import math
import sys

import numpy as np
import pytest

from oracle import gpt_oracle as O

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


def stream():
    return torch.cuda.current_stream().cuda_stream


def dev(a, bf):
    return torch.tensor(np.asarray(a), dtype=torch.bfloat16 if bf else torch.float32, device="cuda").contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def relmax(a, b, floor=1e-30):
    """max|a - b| / max|b|; `floor` bounds the denominator for references that
    are exactly zero (attention rows that only see themselves have dQ = 0)."""
    return float(np.abs(a - b).max() / max(np.abs(b).max(), floor))


# ---------------------------------------------------------------- GEMM

GEMM_CASES = [
    # (M, N, K, a_kc, b_kc): forward X W^T, dgrad dY W, wgrad dY^T X, plus the fourth orientation
    (77, 45, 133, 1, 1), (300, 200, 520, 1, 1), (130, 70, 96, 1, 0), (64, 96, 300, 0, 0), (45, 130, 77, 0, 1),
    (1, 1, 1, 1, 1), (257, 129, 1025, 1, 0), (128, 256, 512, 1, 1), (256, 128, 1024, 0, 0),
    # large enough for the 256x256 matrix-core tiles
    (4096, 4096, 64, 1, 1), (4096, 4096, 64, 1, 0), (4096, 4096, 64, 0, 0), (4000, 4104, 72, 1, 1),
    # few output tiles and a long K: split-K with a deterministic reduction
    (256, 384, 4096, 0, 0), (768, 768, 16384, 0, 0), (200, 136, 4104, 0, 0), (136, 200, 4104, 1, 0),
    # ragged rows/columns with K a multiple of 32 (matrix-core path, clamped edge loads)
    (300, 200, 512, 1, 1), (200, 136, 4096, 0, 0), (136, 200, 4096, 1, 0), (4000, 4104, 64, 1, 1),
    (1000, 72, 96, 1, 0), (72, 1000, 96, 0, 0), (33, 8, 64, 1, 0), (8, 40, 64, 0, 0), (5000, 65, 384, 1, 1),
]


def gemm_ref(A, B, a_kc, b_kc):
    Am = A if a_kc else A.T         # stored [M,K] or [K,M]
    Bm = B.T if b_kc else B         # stored [N,K] or [K,N]
    return Am @ Bm


def gemm_inputs(M, N, K, a_kc, b_kc, bf, rng):
    A = rng.normal(size=(M, K) if a_kc else (K, M))
    B = rng.normal(size=(N, K) if b_kc else (K, N))
    At, Bt = dev(A, bf), dev(B, bf)
    return At, Bt, host(At), host(Bt)


@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("case", GEMM_CASES)
def test_gemm_store(lib, case, bf):
    M, N, K, a_kc, b_kc = case
    say(f"gemm store bf={bf} M={M} N={N} K={K} a_kc={a_kc} b_kc={b_kc}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    At, Bt, A, B = gemm_inputs(M, N, K, a_kc, b_kc, bf, rng)
    ref = gemm_ref(A, B, a_kc, b_kc)
    for c_bf in ([0, 1] if bf else [0]):
        C = torch.zeros((M, N), dtype=torch.bfloat16 if c_bf else torch.float32, device="cuda")
        lda = K if a_kc else M
        ldb = K if b_kc else N
        scratch = torch.zeros(16 * M * N, dtype=torch.float32, device="cuda")
        st = lib.gptk_gemm(M, N, K, At.data_ptr(), lda, a_kc, Bt.data_ptr(), ldb, b_kc, C.data_ptr(), N, bf, c_bf,
                           0, 0, None, None, None, None, scratch.data_ptr(), scratch.numel(), stream())
        assert st == 0
        torch.cuda.synchronize()
        tol = 8e-3 if c_bf else 2e-5 * math.sqrt(K / 64 + 1)
        assert relmax(host(C), ref) < tol, (c_bf, relmax(host(C), ref))


CONFIG_CASES = [
    # (M, N, K, a_kc, b_kc) per orientation, with ragged rows and columns
    (1000, 776, 192, 1, 1), (1000, 776, 192, 1, 0), (776, 1000, 192, 0, 0),
    (520, 392, 1088, 1, 1), (520, 392, 1088, 1, 0), (392, 520, 1088, 0, 0),
    (300, 264, 1056, 1, 1), (300, 264, 1056, 1, 0), (264, 300, 1056, 0, 0),
    # more tiles than workgroup slots: persistent workgroups loop over several tiles
    (4000, 4104, 128, 1, 1), (4000, 4104, 128, 1, 0), (4104, 4000, 128, 0, 0),
]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("case", CONFIG_CASES)
def test_gemm_every_config(lib, case, splits):
    """Every matrix-core tile configuration, with and without split-K, on each
    operand orientation and ragged edges (bf16 inputs, fp32 and bf16 outputs)."""
    M, N, K, a_kc, b_kc = case
    rng = np.random.default_rng(M + N + K + 17 * splits)
    At, Bt, A, B = gemm_inputs(M, N, K, a_kc, b_kc, 1, rng)
    ref = gemm_ref(A, B, a_kc, b_kc)
    scratch = torch.zeros(4 * M * N, dtype=torch.float32, device="cuda")
    try:
        for cfg in range(lib.gptk_gemm_num_configs()):
            assert lib.gptk_gemm_force_config(cfg, splits) == 0
            for c_bf in (0, 1):
                say(f"gemm config {cfg} splits {splits} M={M} N={N} K={K} a_kc={a_kc} b_kc={b_kc} c_bf={c_bf}")
                C = torch.zeros((M, N), dtype=torch.bfloat16 if c_bf else torch.float32, device="cuda")
                st = lib.gptk_gemm(M, N, K, At.data_ptr(), K if a_kc else M, a_kc, Bt.data_ptr(), K if b_kc else N,
                                   b_kc, C.data_ptr(), N, 1, c_bf, 0, 0, None, None, None, None, scratch.data_ptr(),
                                   scratch.numel(), stream())
                assert st == 0
                torch.cuda.synchronize()
                err = relmax(host(C), ref)
                assert err < (8e-3 if c_bf else 2e-5 * math.sqrt(K / 64 + 1)), (cfg, c_bf, err)
    finally:
        assert lib.gptk_gemm_force_config(-1, 0) == 0


@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("epi", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("shape", [(200, 136, 264), (4096, 4096, 64), (256, 384, 4096)])
def test_gemm_epilogues(lib, epi, act, bf, shape):
    if act and epi not in (2, 4):
        pytest.skip("activation only matters for epilogues 2 and 4")
    M, N, K = shape
    say(f"gemm epilogue {epi} act {act} bf={bf}")
    rng = np.random.default_rng(epi * 10 + act)
    At, Bt, A, B = gemm_inputs(M, N, K, 1, 1, bf, rng)
    acc = gemm_ref(A, B, 1, 1) * 0.2
    At = At * 0.2 if not bf else dev(host(At) * 0.2, bf)
    A = host(At)
    acc = gemm_ref(A, B, 1, 1)
    bias = rng.normal(size=N)
    biast = torch.tensor(bias, dtype=torch.float32, device="cuda")
    act_f = O.relu2 if act else O.gelu_tanh
    actg = O.relu2_grad if act else O.gelu_tanh_grad
    c_bf = bf if epi in (1, 2, 4) else 0
    ctype = torch.bfloat16 if c_bf else torch.float32
    C = torch.zeros((M, N), dtype=ctype, device="cuda")
    C2 = torch.zeros((M, N), dtype=ctype, device="cuda")
    resid = rng.normal(size=(M, N))
    residt = torch.tensor(resid, dtype=torch.float32, device="cuda")
    aux = dev(rng.normal(size=(M, N)), c_bf)
    if epi == 5:
        C.copy_(residt)
    scratch = torch.zeros(8 * M * N, dtype=torch.float32, device="cuda")
    st = lib.gptk_gemm(M, N, K, At.data_ptr(), K, 1, Bt.data_ptr(), K, 1, C.data_ptr(), N, bf, c_bf, epi, act,
                       biast.data_ptr(), residt.data_ptr(), aux.data_ptr(), C2.data_ptr(), scratch.data_ptr(),
                       scratch.numel(), stream())
    assert st == 0
    torch.cuda.synchronize()
    tol = 1e-2 if c_bf else 3e-5
    if epi == 1:
        assert relmax(host(C), acc + bias) < tol
    elif epi == 2:
        pre = acc + bias
        assert relmax(host(C), actg(pre)) < tol
        assert relmax(host(C2), act_f(pre)) < tol
    elif epi == 3:
        assert relmax(host(C), resid + acc + bias) < tol
    elif epi == 4:
        assert relmax(host(C), acc * host(aux)) < tol
    else:
        assert relmax(host(C), resid + acc) < tol


def _gemm_colsum_case(lib, M, N, K, bf, seed):
    rng = np.random.default_rng(seed)
    At, Bt, A, B = gemm_inputs(M, N, K, 1, 0, bf, rng)
    acc = gemm_ref(A, B, 1, 0)
    aux = dev(rng.uniform(-1.0, 1.0, size=(M, N)), bf)
    C = torch.zeros((M, N), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    out0 = rng.normal(size=N)
    out = torch.tensor(out0, dtype=torch.float32, device="cuda")
    part = torch.zeros(int(lib.gptk_colsum_partial_floats(M, N)), dtype=torch.float32, device="cuda")
    scratch = torch.zeros(4 * M * N, dtype=torch.float32, device="cuda")
    st = lib.gptk_gemm_colsum(M, N, K, At.data_ptr(), K, 1, Bt.data_ptr(), N, 0, C.data_ptr(), N, bf, bf, 4, 0, None,
                              None, aux.data_ptr(), None, out.data_ptr(), part.data_ptr(), scratch.data_ptr(),
                              scratch.numel(), stream())
    assert st == 0
    torch.cuda.synchronize()
    ref = acc * host(aux)
    tol = 1e-2 if bf else 3e-5
    assert relmax(host(C), ref) < tol
    # fused sums add fp32 values before storage rounding; the separate pass adds the stored values
    assert relmax(host(out) - out0, ref.sum(0)) < (1e-2 if bf else 1e-5)


@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("shape", [(16384, 3072, 768), (1000, 200, 192), (300, 136, 64), (5000, 72, 384),
                                   (4096, 4096, 64), (33, 8, 64)])
def test_gemm_act_grad_colsum(lib, shape, bf):
    """ACT_GRAD product with the bias-gradient column sums (fused into the epilogue on the matrix-core path)."""
    M, N, K = shape
    say(f"gemm colsum {shape} bf={bf}")
    _gemm_colsum_case(lib, M, N, K, bf, M + N + K)


@pytest.mark.parametrize("cfg", list(range(27)))
def test_gemm_act_grad_colsum_every_config(lib, cfg):
    if cfg >= lib.gptk_gemm_num_configs():
        pytest.skip("no such configuration")
    say(f"gemm colsum cfg {cfg}")
    assert lib.gptk_gemm_force_config(cfg, 1) == 0
    try:
        _gemm_colsum_case(lib, 1000, 392, 192, 1, cfg)
    finally:
        lib.gptk_gemm_force_config(-1, 0)


# ---------------------------------------------------------------- attention

ATT_CASES = [
    # (B, T, H, hd, window)
    (2, 37, 3, 16, 0), (1, 130, 2, 32, 0), (2, 200, 2, 64, 0), (1, 257, 2, 128, 0),
    (2, 150, 2, 64, 17), (1, 300, 2, 128, 64), (1, 64, 4, 16, 1), (3, 1, 2, 64, 0),
    # the training step's head shapes at full length: GPT-2 (T 1024, hd 64) and
    # the speedrun block's short window (T 2048, hd 128, W 256)
    (2, 1024, 2, 64, 0), (2, 2048, 2, 128, 256),
]


def attn_case(B, T, H, hd, window, bf, seed):
    rng = np.random.default_rng(seed)
    d = H * hd
    qkv = rng.normal(size=(B * T, 3 * d))
    qkvt = dev(qkv, bf)
    qkv = host(qkvt)
    q = qkv[:, :d].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    k = qkv[:, d:2 * d].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    v = qkv[:, 2 * d:].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    return qkvt, q, k, v


@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("case", ATT_CASES)
def test_attention_fwd_bwd(lib, case, bf):
    B, T, H, hd, W = case
    d = H * hd
    say(f"attention B={B} T={T} H={H} hd={hd} W={W} bf={bf}")
    qkvt, q, k, v = attn_case(B, T, H, hd, W, bf, B * 1000 + T + hd)
    esz = qkvt.element_size()
    o = torch.zeros((B * T, d), dtype=qkvt.dtype, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    base = qkvt.data_ptr()
    st = lib.gptk_attention(0, B, T, H, hd, W, base, base + d * esz, base + 2 * d * esz, 3 * d, 3 * d, 3 * d,
                            o.data_ptr(), d, lse.data_ptr(), None, 0, None, None, None, None, 0, bf, stream())
    assert st == 0
    torch.cuda.synchronize()
    oref, p = O.attention_fwd(q, k, v, W)
    oref_m = oref.transpose(0, 2, 1, 3).reshape(B * T, d)
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    s = np.where(O.attention_mask(T, W), s, -np.inf)
    lse_ref = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    tol = 2e-2 if bf else 2e-5
    assert relmax(host(o), oref_m) < tol
    assert np.abs(host(lse) - lse_ref).max() < (2e-2 if bf else 1e-5)
    # backward
    rng = np.random.default_rng(7 + T)
    dO = rng.normal(size=(B * T, d))
    dOt = dev(dO, bf)
    dO = host(dOt)
    D = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    dqkv = torch.zeros((B * T, 3 * d), dtype=qkvt.dtype, device="cuda")
    g = dqkv.data_ptr()
    st = lib.gptk_attention(1, B, T, H, hd, W, base, base + d * esz, base + 2 * d * esz, 3 * d, 3 * d, 3 * d,
                            o.data_ptr(), d, lse.data_ptr(), dOt.data_ptr(), d, D.data_ptr(), g, g + d * esz,
                            g + 2 * d * esz, 3 * d, bf, stream())
    assert st == 0
    torch.cuda.synchronize()
    dO_h = dO.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    # the kernel uses its own stored O for D; the oracle's uses the exact P
    dq, dk, dv = O.attention_bwd(dO_h, q, k, v, p)
    ref = np.concatenate([a.transpose(0, 2, 1, 3).reshape(B * T, d) for a in (dq, dk, dv)], axis=1)
    got = host(dqkv)
    tol = 3e-2 if bf else 5e-5
    for j, name in enumerate(("dq", "dk", "dv")):
        assert relmax(got[:, j * d:(j + 1) * d], ref[:, j * d:(j + 1) * d], floor=1.0) < tol, name


@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("case", ATT_CASES + [(16, 1024, 12, 64, 0), (1, 4096, 2, 128, 0)])
def test_attention_bwd_bias_colsum(lib, case, bf):
    """qkv bias gradient (column sums of dq, dk, dv) fused into the attention backward,
    against the oracle's gradients summed over rows."""
    B, T, H, hd, W = case
    d = H * hd
    say(f"attention colsum B={B} T={T} H={H} hd={hd} W={W} bf={bf}")
    qkvt, q, k, v = attn_case(B, T, H, hd, W, bf, B * 1000 + T + hd + 5)
    esz = qkvt.element_size()
    o = torch.zeros((B * T, d), dtype=qkvt.dtype, device="cuda")
    lse = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    base = qkvt.data_ptr()
    assert lib.gptk_attention(0, B, T, H, hd, W, base, base + d * esz, base + 2 * d * esz, 3 * d, 3 * d, 3 * d,
                              o.data_ptr(), d, lse.data_ptr(), None, 0, None, None, None, None, 0, bf, stream()) == 0
    rng = np.random.default_rng(11 + T)
    dOt = dev(rng.normal(size=(B * T, d)), bf)
    D = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    dqkv = torch.zeros((B * T, 3 * d), dtype=qkvt.dtype, device="cuda")
    out0 = rng.normal(size=3 * d)
    out = torch.tensor(out0, dtype=torch.float32, device="cuda")
    part = torch.zeros(int(lib.gptk_attention_colsum_partial_floats(B, T, H, hd)), dtype=torch.float32, device="cuda")
    st = lib.gptk_attention_bwd_colsum(B, T, H, hd, W, base, base + d * esz, base + 2 * d * esz, 3 * d, 3 * d, 3 * d,
                                       o.data_ptr(), d, lse.data_ptr(), dOt.data_ptr(), d, D.data_ptr(),
                                       dqkv.data_ptr(), bf, out.data_ptr(), part.data_ptr(), stream())
    assert st == 0
    torch.cuda.synchronize()
    got = host(out) - out0
    # oracle column sums, one sequence at a time (bounded host memory)
    dO_h = host(dOt).reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    ref = np.zeros(3 * d)
    for b in range(B):
        sl = slice(b, b + 1)
        _, p = O.attention_fwd(q[sl], k[sl], v[sl], W)
        grads = O.attention_bwd(dO_h[sl], q[sl], k[sl], v[sl], p)
        ref += np.concatenate([a.transpose(0, 2, 1, 3).reshape(T, d).sum(0) for a in grads])
    assert relmax(got, ref, floor=1.0) < (3e-2 if bf else 1e-4)
    # the sums agree with the stored gradients (which the element-wise test checks)
    stored = host(dqkv).sum(0)
    assert relmax(got, stored, floor=1.0) < (1e-2 if bf else 1e-5)


# ---------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("M,d", [(7, 64), (130, 768), (65, 384), (33, 32), (200, 2048), (3000, 768), (70, 1000)])
def test_layernorm(lib, M, d, bf):
    say(f"layernorm M={M} d={d} bf={bf}")
    rng = np.random.default_rng(M + d)
    x = rng.normal(size=(M, d)) * 2 + 0.5
    g = 1 + 0.1 * rng.normal(size=d)
    b = 0.1 * rng.normal(size=d)
    xt, gt, bt = (torch.tensor(a, dtype=torch.float32, device="cuda") for a in (x, g, b))
    x, g, b = host(xt), host(gt), host(bt)
    y = torch.zeros((M, d), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    mean = torch.zeros(M, dtype=torch.float32, device="cuda")
    rstd = torch.zeros(M, dtype=torch.float32, device="cuda")
    s = stream()
    assert lib.gptk_layernorm(0, M, d, 1e-5, xt.data_ptr(), gt.data_ptr(), bt.data_ptr(), y.data_ptr(),
                              mean.data_ptr(), rstd.data_ptr(), None, None, None, 0, None, None, None, None, bf,
                              s) == 0
    yref, cache = O.layernorm_fwd(x, g, b, 1e-5)
    torch.cuda.synchronize()
    assert relmax(host(y), yref) < (8e-3 if bf else 1e-5)
    dy = rng.normal(size=(M, d))
    dyt = torch.tensor(dy, dtype=torch.float32, device="cuda")
    dres0 = rng.normal(size=(M, d))
    dres = torch.tensor(dres0, dtype=torch.float32, device="cuda")
    dlp = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
    dg = torch.full((d,), 0.5, dtype=torch.float32, device="cuda")
    db = torch.full((d,), -0.25, dtype=torch.float32, device="cuda")
    dcol = torch.full((d,), 0.125, dtype=torch.float32, device="cuda")
    part = torch.zeros(int(lib.gptk_layernorm_partial_floats(M, d)), dtype=torch.float32, device="cuda")
    assert lib.gptk_layernorm(1, M, d, 1e-5, xt.data_ptr(), gt.data_ptr(), None, None, mean.data_ptr(),
                              rstd.data_ptr(), dyt.data_ptr(), dres.data_ptr(), dlp.data_ptr() if bf else None, 0,
                              dg.data_ptr(), db.data_ptr(), dcol.data_ptr(), part.data_ptr(), bf, s) == 0
    torch.cuda.synchronize()
    dx, dgr, dbr = O.layernorm_bwd(host(dyt), cache, g)
    assert relmax(host(dres), dres0 + dx) < 1e-5
    assert relmax(host(dcol), 0.125 + (dres0 + dx).sum(0)) < 1e-5
    assert relmax(host(dg), 0.5 + dgr) < 1e-5
    assert relmax(host(db), -0.25 + dbr) < 1e-5
    if bf:
        assert relmax(host(dlp), dres0 + dx) < 8e-3


# ---------------------------------------------------------------- cross-entropy

@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("M,V,cap", [(9, 65, 0.0), (70, 1000, 0.0), (5, 50304, 0.0), (33, 777, 3.0), (4, 50304, 30.0)])
def test_cross_entropy(lib, M, V, cap, bf):
    say(f"cross entropy M={M} V={V} cap={cap} bf={bf}")
    rng = np.random.default_rng(M + V)
    z = rng.normal(size=(M, V)) * 3
    zt = dev(z, bf)
    z = host(zt)
    y = rng.integers(0, V, M).astype(np.int32)
    yt = torch.tensor(y, device="cuda")
    rl = torch.zeros(M, dtype=torch.float32, device="cuda")
    err = torch.zeros(4, dtype=torch.int32, device="cuda")
    scale = 0.37
    assert lib.gptk_cross_entropy(M, V, zt.data_ptr(), yt.data_ptr(), rl.data_ptr(), scale / M, cap,
                                  err.data_ptr(), bf, stream()) == 0
    torch.cuda.synchronize()
    if cap:
        th = np.tanh(z / cap)
        zc = cap * th
    else:
        zc = z
    losses, dz = O.cross_entropy_fwd_bwd(zc, y, scale)
    if cap:
        dz = dz * (1 - th * th)
    assert np.abs(host(rl) - losses).max() < 1e-4 * max(1, np.abs(losses).max())
    assert relmax(host(zt), dz) < (1e-2 if bf else 1e-5)
    assert int(err[0]) == 0


def test_cross_entropy_bad_target_flags(lib):
    M, V = 3, 17
    zt = dev(np.zeros((M, V)), 0)
    yt = torch.tensor([1, 17, -1], dtype=torch.int32, device="cuda")
    rl = torch.zeros(M, dtype=torch.float32, device="cuda")
    err = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert lib.gptk_cross_entropy(M, V, zt.data_ptr(), yt.data_ptr(), rl.data_ptr(), 1.0, 0.0, err.data_ptr(), 0,
                                  stream()) == 0
    torch.cuda.synchronize()
    assert int(err[0]) == 1
    assert float(rl[1]) == 0 and float(rl[2]) == 0 and abs(float(rl[0]) - math.log(17)) < 1e-5
    assert float(zt[1].abs().sum()) == 0


# ---------------------------------------------------------------- embedding backward, column sums

@pytest.mark.parametrize("B,T,V,kind", [(2, 37, 50, "uniform"), (4, 1024, 50304, "zipf"), (16, 1024, 50304, "zipf"),
                                        (3, 100, 65, "same"), (1, 1, 7, "uniform"), (8, 4096, 50304, "same")])
def test_embedding_backward(lib, B, T, V, kind):
    say(f"embedding backward B={B} T={T} V={V} {kind}")
    rng = np.random.default_rng(B * T)
    d = 64 if B * T < 30000 else 32
    if kind == "zipf":
        from transformer_lm_step_gpt_amd import inputs as I
        tok = I.ZipfEotStream(5).take(B * T)
    elif kind == "same":
        tok = np.full(B * T, V - 1, dtype=np.int32)
    else:
        tok = rng.integers(0, V, B * T).astype(np.int32)
    dx = rng.normal(size=(B * T, d)).astype(np.float32)
    wte0 = rng.normal(size=(V, d)).astype(np.float32)
    wpe0 = rng.normal(size=(T, d)).astype(np.float32)
    tt = torch.tensor(tok.astype(np.int32), device="cuda")
    dxt = torch.tensor(dx, device="cuda")
    dwte = torch.tensor(wte0, device="cuda")
    dwpe = torch.tensor(wpe0, device="cuda")
    scratch = torch.zeros(int(lib.gptk_embed_bwd_scratch_bytes(B * T, d)), dtype=torch.uint8, device="cuda")
    assert lib.gptk_embed_bwd(tt.data_ptr(), dxt.data_ptr(), dwte.data_ptr(), dwpe.data_ptr(), B, T, d, V,
                              scratch.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    ref = wte0.astype(np.float64)
    np.add.at(ref, tok, dx.astype(np.float64))
    refp = wpe0 + dx.reshape(B, T, d).astype(np.float64).sum(0)
    assert np.abs(host(dwte) - ref).max() < 1e-5 * max(1, np.abs(ref).max())
    assert np.abs(host(dwpe) - refp).max() < 1e-5 * max(1, np.abs(refp).max())
    # deterministic: a second run from the same start is bitwise identical
    dwte2 = torch.tensor(wte0, device="cuda")
    assert lib.gptk_embed_bwd(tt.data_ptr(), dxt.data_ptr(), dwte2.data_ptr(), None, B, T, d, V,
                              scratch.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dwte, dwte2)


@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("M,N", [(1, 5), (300, 768), (1000, 2304), (129, 3072), (5000, 3072), (77, 13)])
def test_colsum(lib, M, N, bf):
    rng = np.random.default_rng(M + N)
    Yt = dev(rng.normal(size=(M, N)), bf)
    out0 = rng.normal(size=N)
    out = torch.tensor(out0, dtype=torch.float32, device="cuda")
    part = torch.zeros(int(lib.gptk_colsum_partial_floats(M, N)), dtype=torch.float32, device="cuda")
    assert lib.gptk_colsum(M, N, Yt.data_ptr(), N, bf, out.data_ptr(), part.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert relmax(host(out), out0 + host(Yt).sum(0)) < 1e-5


# ---------------------------------------------------------------- QK-Norm and rotary positions

@pytest.mark.parametrize("bf", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("M,T,H,hd,norm,rope", [(300, 100, 3, 128, 1, 1), (260, 64, 4, 64, 1, 1), (70, 70, 2, 16, 1, 1),
                                                 (130, 65, 6, 128, 0, 1), (130, 65, 2, 32, 1, 0), (50, 50, 3, 24, 1, 1)])
def test_qk_prep(lib, M, T, H, hd, norm, rope, bf):
    """q/k RMS normalisation and rotary positions, forward and backward, against
    the oracle's rmsnorm / rope pieces (row m at position m % T); the value
    columns are left alone by the backward."""
    say(f"qk prep M={M} T={T} H={H} hd={hd} norm={norm} rope={rope} bf={bf}")
    rng = np.random.default_rng(M + 7 * hd + T)
    d = H * hd
    qt = dev(rng.normal(size=(M, 3 * d)) * 1.5, bf)
    qkv = host(qt)
    out = torch.zeros((M, 2 * d), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    tables = torch.zeros(T * hd, dtype=torch.float32, device="cuda")
    assert lib.gptk_qk_prep(0, M, T, H, hd, qt.data_ptr(), out.data_ptr(), tables.data_ptr(), 10000.0, norm, rope, 1e-6,
                            bf, stream()) == 0
    cos, sin = O.rope_tables(T, hd, 10000.0)
    pos = np.arange(M) % T
    c, s = cos[pos][:, None, :], sin[pos][:, None, :]
    gt = dev(rng.normal(size=(M, 3 * d)), bf)
    g = host(gt)
    ref_out, ref_g = [], g.copy()
    for which in (0, 1):
        x = qkv[:, which * d:(which + 1) * d].reshape(M, H, hd)
        y, r = O.rmsnorm_fwd(x, 1e-6) if norm else (x, None)
        ref_out.append((O.rope_fwd(y, c, s) if rope else y).reshape(M, d))
        dy = g[:, which * d:(which + 1) * d].reshape(M, H, hd)
        if rope:
            dy = O.rope_bwd(dy, c, s)
        if norm:
            dy = O.rmsnorm_bwd(dy, y, r)
        ref_g[:, which * d:(which + 1) * d] = dy.reshape(M, d)
    torch.cuda.synchronize()
    assert relmax(host(out), np.concatenate(ref_out, axis=1)) < (1e-2 if bf else 1e-5)
    assert lib.gptk_qk_prep(1, M, T, H, hd, qt.data_ptr(), gt.data_ptr(), tables.data_ptr(), 10000.0, norm, rope, 1e-6,
                            bf, stream()) == 0
    torch.cuda.synchronize()
    got = host(gt)
    assert relmax(got[:, :2 * d], ref_g[:, :2 * d]) < (1e-2 if bf else 1e-5)
    assert np.array_equal(got[:, 2 * d:], g[:, 2 * d:])


def test_qk_prep_rejects_bad_shapes(lib):
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    for hd in (0, 3, 130):
        assert lib.gptk_qk_prep(0, 2, 2, 1, hd, t.data_ptr(), t.data_ptr(), t.data_ptr(), 10000.0, 1, 1, 1e-6, 0,
                                stream()) == -1
