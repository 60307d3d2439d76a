"""gptk_layernorm_bwd_noalloc, the LayerNorm backward whose partial sums live
in the library's own device array (for callers that cannot allocate), against
the same backward through gptk_layernorm with a caller-provided partial-sum
buffer: bitwise-equal outputs (same kernels, same summation order) on calls in
a row, each later one smaller than the one before, plus the oversize rejection."""

import sys

import numpy as np
import pytest

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


def _f32(a):
    return torch.tensor(np.asarray(a), dtype=torch.float32, device="cuda").contiguous()


def _pair(lib, M, d, bf, seed):
    say(f"no-alloc LayerNorm backward M={M} d={d} bf={bf}")
    s = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(seed)
    x, g, b = _f32(rng.normal(size=(M, d)) * 2 + 0.3), _f32(1 + 0.1 * rng.normal(size=d)), _f32(0.1 * rng.normal(size=d))
    y = torch.zeros((M, d), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    mean = torch.zeros(M, dtype=torch.float32, device="cuda")
    rstd = torch.zeros(M, dtype=torch.float32, device="cuda")
    assert lib.gptk_layernorm(0, M, d, 1e-5, x.data_ptr(), g.data_ptr(), b.data_ptr(), y.data_ptr(), mean.data_ptr(),
                              rstd.data_ptr(), None, None, None, 0, None, None, None, None, bf, s) == 0
    dy = _f32(rng.normal(size=(M, d)))
    dres0, dg0, db0, dc0 = rng.normal(size=(M, d)), rng.normal(size=d), rng.normal(size=d), rng.normal(size=d)
    outs = []
    for noalloc in (False, True):
        dres, dg, db, dcol = _f32(dres0), _f32(dg0), _f32(db0), _f32(dc0)
        dlp = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
        lp = dlp.data_ptr() if bf else None
        if noalloc:
            st = lib.gptk_layernorm_bwd_noalloc(M, d, x.data_ptr(), g.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                                                dy.data_ptr(), dres.data_ptr(), lp, 0, dg.data_ptr(), db.data_ptr(),
                                                dcol.data_ptr(), bf, s)
        else:
            part = torch.zeros(int(lib.gptk_layernorm_partial_floats(M, d)), dtype=torch.float32, device="cuda")
            st = lib.gptk_layernorm(1, M, d, 1e-5, x.data_ptr(), g.data_ptr(), None, None, mean.data_ptr(),
                                    rstd.data_ptr(), dy.data_ptr(), dres.data_ptr(), lp, 0, dg.data_ptr(),
                                    db.data_ptr(), dcol.data_ptr(), part.data_ptr(), bf, s)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((dres, dg, db, dcol, dlp))
    for name, a, c in zip(("dres", "dg", "db", "dcol", "dres_lp"), outs[0], outs[1]):
        assert torch.equal(a, c), name


def test_noalloc_layernorm_bwd_matches_workspace_entry(lib):
    """Three calls in a row on the same array, each smaller than the last
    (the array keeps the earlier call's contents)."""
    _pair(lib, 16384, 768, 1, 1)
    _pair(lib, 3000, 768, 1, 2)
    _pair(lib, 70, 1000, 0, 3)


def test_noalloc_layernorm_bwd_rejects_oversize(lib):
    """A shape whose partial sums exceed the array is refused before any launch."""
    cap = int(lib.gptk_layernorm_noalloc_max_floats())
    M, d = 65536, 2048
    assert int(lib.gptk_layernorm_partial_floats(M, d)) > cap
    t = torch.zeros(16, dtype=torch.float32, device="cuda")
    p = t.data_ptr()
    st = lib.gptk_layernorm_bwd_noalloc(M, d, p, p, p, p, p, p, None, 0, p, p, None, 0,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == -1
    assert int(lib.gptk_layernorm_partial_floats(32768, 2048)) <= cap
