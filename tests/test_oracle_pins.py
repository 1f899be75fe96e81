"""The oracle's arithmetic against float64 brute force, closed forms and torch
library routines; and the recurrence properties every correct sweep has."""
import dataclasses

import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc

import pins

TINY_RESIDUAL = [ri.TINY_SWIGLU, ri.TINY_LLAMA, ri.TINY_LLAMA_HD128, ri.TINY_ENCODER,
                 ri.TINY_ENCODER_HD128, ri.TINY_ENCODER_POSTNORM, ri.TINY_ENCODER_POSTNORM_HD128,
                 ri.TINY_ENCODER_WIDE, ri.TINY_ENCODER_WIDE_POSTNORM]
# cells that compute Y = A exactly when the last projection of every branch is zero (a post-norm
# layer still normalises, so it has no such weights)
TINY_IDENTITY = [c for c in TINY_RESIDUAL if not c.post_norm]


def test_linear_gelu_bruteforce_fp32():
    pins.pin_linear_gelu_bruteforce(tol=1e-5)


def test_linear_gelu_bruteforce_fp64():
    fwd64 = lambda *a, **k: orc.forward_sequential(*a, dtype=np.float64, **k)  # noqa: E731
    pins.pin_linear_gelu_bruteforce(forward=fwd64, tol=1e-13)


def test_linear_gelu_bruteforce_diagonal():
    pins.pin_linear_gelu_bruteforce(forward=orc.forward_diagonal, tol=1e-5)


@pytest.mark.parametrize("cfg", TINY_IDENTITY, ids=lambda c: c.name)
def test_shift_register(cfg):
    pins.pin_shift_register(cfg)
    pins.pin_shift_register(cfg, forward=orc.forward_diagonal)


@pytest.mark.parametrize("cfg", TINY_RESIDUAL, ids=lambda c: c.name)
def test_single_segment_against_torch(cfg):
    pins.pin_single_segment_against_torch(cfg)


def test_single_segment_gqa_two_kv_heads():
    cfg = dataclasses.replace(ri.TINY_LLAMA, Hq=4, Hkv=2, hd=64, d=256)
    pins.pin_single_segment_against_torch(cfg)


def test_gelu():
    pins.pin_gelu()


def test_silu():
    pins.pin_silu()


def test_rms_norm():
    pins.pin_rms_norm()


def test_rope():
    pins.pin_rope()


def test_attention():
    pins.pin_attention()


def test_layer_norm():
    pins.pin_layer_norm()


def test_full_attention():
    pins.pin_full_attention()


# ---------------------------------------------------------------------------
# Recurrence properties
# ---------------------------------------------------------------------------

def _inputs(cfg, seed=0):
    w = ri.all_weights(cfg, seed)
    mem0 = ri.initial_memory(cfg, seed)
    if cfg.cell == ri.CELL_LLAMA:
        return w, ri.tokens(cfg, seed), mem0, ri.embedding(cfg, seed)
    return w, ri.input_embeddings(cfg, seed), mem0, None


@pytest.mark.parametrize("cfg", [ri.TINY_LINEAR_GELU] + TINY_RESIDUAL, ids=lambda c: c.name)
def test_diagonal_equals_sequential_bitwise(cfg):
    w, x, mem0, emb = _inputs(cfg)
    h1, m1 = orc.forward_sequential(cfg, w, x, mem0, emb)
    h2, m2 = orc.forward_diagonal(cfg, w, x, mem0, emb)
    assert h1.dtype == np.float32
    assert np.array_equal(h1, h2) and np.array_equal(m1, m2)


@pytest.mark.parametrize("cfg", [ri.TINY_LINEAR_GELU, ri.TINY_LLAMA], ids=lambda c: c.name)
def test_resume(cfg):
    """fwd(first a segments) then fwd(rest, mem0 = its memory) == fwd(all)."""
    w, x, mem0, emb = _inputs(cfg)
    a = 2
    h, mm = orc.forward_sequential(cfg, w, x, mem0, emb)
    h1, m1 = orc.forward_sequential(cfg, w, x[:a * cfg.n], mem0, emb)
    h2, m2 = orc.forward_diagonal(cfg, w, x[a * cfg.n:], m1, emb)
    assert np.array_equal(np.concatenate([h1, h2]), h) and np.array_equal(m2, mm)


def test_dependency_cone_segments():
    cfg = ri.TINY_LINEAR_GELU
    w, x, mem0, _ = _inputs(cfg)
    h, _ = orc.forward_sequential(cfg, w, x, mem0)
    s = 3
    x2 = x.copy()
    x2[s * cfg.n + 5] += 1.0
    h2, _ = orc.forward_sequential(cfg, w, x2, mem0)
    n = cfg.n
    assert np.array_equal(h[:s * n], h2[:s * n])
    # the change reaches some later output (each row-wise layer delays the
    # stream by m rows, so with L*m = n it lands one segment later)
    assert not np.array_equal(h[s * n:], h2[s * n:])


def test_dependency_cone_memory():
    cfg = ri.TINY_LLAMA
    w, tok, mem0, emb = _inputs(cfg)
    h, mm = orc.forward_sequential(cfg, w, tok, mem0, emb)
    l = 1
    mem2 = mem0.copy()
    mem2[l, 3, 7] += 0.5
    h2, mm2 = orc.forward_sequential(cfg, w, tok, mem2, emb)
    assert np.array_equal(mm[:l], mm2[:l])          # layers below l never see M(l, .)
    assert not np.array_equal(mm[l], mm2[l])
    assert not np.array_equal(h, h2)


def test_inplace_diagonal_sweep_is_wrong():
    """Negative control for the order test: a diagonal sweep that overwrites
    X(l-1, .) while walking the diagonal upward gives different results."""
    cfg = ri.TINY_LINEAR_GELU
    w, x, mem0, _ = _inputs(cfg)
    L, n = cfg.L, cfg.n
    M = [mem0[l].copy() for l in range(L)]
    X = [None] * L
    hidden = [None] * cfg.S
    for diag in orc.schedule(L, cfg.S):
        for (l, s) in diag:
            x_in = x[s * n:(s + 1) * n] if l == 0 else X[l - 1]
            Y = orc.cell(cfg, w[l], np.concatenate([M[l], x_in]))
            X[l], M[l] = Y[:n], Y[n:]
            if l == L - 1:
                hidden[s] = Y[:n]
    h_bad = np.concatenate(hidden)
    h, _ = orc.forward_sequential(cfg, w, x, mem0)
    assert not np.array_equal(h, h_bad)
    with pytest.raises(AssertionError):
        assert pins.normwise(h_bad, h) <= 1e-5


# ---- a short last segment ---------------------------------------------------

N_LG = ri.TINY_LINEAR_GELU.n     # 16 rows per segment, m = 4


@pytest.mark.parametrize("T", [5 * N_LG + 2, 5 * N_LG + 7, 5 * N_LG + 15, 9, 1])
def test_linear_gelu_bruteforce_ragged(T):
    """short tails with r < m, r >= m, r = n - 1, and sequences of one short segment"""
    pins.pin_linear_gelu_bruteforce_ragged(T)
    fwd = lambda *a, **k: orc.forward_diagonal(*a, **k)  # noqa: E731
    pins.pin_linear_gelu_bruteforce_ragged(T, forward=fwd)


@pytest.mark.parametrize("cfg", TINY_IDENTITY, ids=lambda c: c.name)
def test_shift_register_ragged(cfg):
    T = (cfg.S - 1) * cfg.n + cfg.n // 3
    pins.pin_shift_register_ragged(cfg, T)
    pins.pin_shift_register_ragged(cfg, T, forward=orc.forward_diagonal)


@pytest.mark.parametrize("cfg", TINY_RESIDUAL, ids=lambda c: c.name)
def test_short_single_segment_against_torch(cfg):
    pins.pin_short_single_segment_against_torch(cfg, cfg.n // 3 + 1)


@pytest.mark.parametrize("cfg", [ri.TINY_LINEAR_GELU, ri.TINY_LLAMA], ids=lambda c: c.name)
def test_ragged_run_extends_the_whole_segment_prefix(cfg):
    """Segments never read later ones: the whole segments of a ragged run
    equal the run over just those segments, bit for bit."""
    S_full = cfg.S - 1
    T = S_full * cfg.n + cfg.n // 2
    w, x, mem0, emb = pins.ragged_inputs(cfg, T)
    h, _ = orc.forward_sequential(cfg, w, x, mem0, emb)
    hp, _ = orc.forward_sequential(cfg, w, x[:S_full * cfg.n], mem0, emb)
    assert h.shape[0] == T
    assert np.array_equal(h[:S_full * cfg.n], hp)
    hd, md = orc.forward_diagonal(cfg, w, x, mem0, emb)
    hs, ms = orc.forward_sequential(cfg, w, x, mem0, emb)
    assert np.array_equal(hd, hs) and np.array_equal(md, ms)
