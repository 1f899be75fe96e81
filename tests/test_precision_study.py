"""The rounding-point emulation behind the precision figures of the design
notes (tests/precision_study.py), at the tiny grids' size.

The emulation must equal the oracle when nothing is rounded; rounding the
six 16-bit points must cost accuracy in the proportions a rounding model
predicts (fp16 rounds with an eighth of bf16's step, and independent
rounding errors add in quadrature); and the recurrence amplifies a small
change of the initial memory over the segments.  The full-size tables (1B
and 8B shapes) come from running the module as a script."""
import dataclasses
import math

import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc

import precision_study as ps


@pytest.mark.parametrize("norm_order", ps.NORM_ORDERS)
@pytest.mark.parametrize("cfg", [ri.TINY_LLAMA, ri.TINY_LLAMA_HD128], ids=lambda c: c.name)
def test_unrounded_emulation_is_the_oracle_cell(cfg, norm_order):
    """No point rounded: the oracle's cell, up to fp32 evaluation order (the
    emulation forms exponentials in base 2 from prescaled Q, as the GPU does,
    and, in the GPU's order, applies 1/rms to the GEMM's product rows)."""
    c1 = dataclasses.replace(cfg, L=1, S=1)
    w = [{k: np.asarray(v, np.float32) for k, v in d.items()} for d in ri.all_weights(c1)]
    tok, mem0, emb = ri.tokens(c1), ri.initial_memory(c1), ri.embedding(c1)
    A = np.concatenate([mem0[0], emb[tok]])
    y_em = ps.emulated_llama_cell(A, w[0], c1, points=(), norm_order=norm_order)
    y_or = orc.cell_llama(A, w[0], c1.Hq, c1.Hkv, c1.hd, c1.eps, c1.theta)
    err = np.max(np.abs(y_em - y_or)) / np.max(np.abs(y_or))
    assert err < 2e-6, err
    # and the sweep over the whole tiny grid
    h_em, m_em = ps.sweep(c1, w, tok, mem0, emb, 1, norm_order=norm_order)
    h_or, m_or = orc.forward_sequential(c1, w, tok, mem0, emb)
    assert ps.rel_l2(h_em, h_or) < 2e-6 and ps.rel_l2(m_em, m_or) < 2e-6


def test_round_helpers():
    x = np.array([1.0, 1.0 + 2.0 ** -9, 1.0 + 2.0 ** -8 + 2.0 ** -10, 3.0e-6, 7e4], np.float32)
    h = ps.round_fp16(x)
    assert h[0] == 1.0 and h[1] == 1.0 + 2.0 ** -9            # fp16 keeps 10 fraction bits
    assert ri.round_bf16(x)[1] == 1.0                          # bf16 keeps 7: ties to even
    assert np.isinf(h[4])                                      # above 65504
    assert abs(h[3] - 3.0e-6) <= 2.0 ** -25                    # subnormal grid 2^-24


@pytest.fixture(scope="module")
def tiny_table():
    cfg = ri.TINY_LLAMA
    return ps.rounding_table(cfg, cfg.S, ps.STANDARD_VARIANTS, log=lambda m: None)


def test_fp16_points_cost_a_fraction_of_bf16(tiny_table):
    e_bf = tiny_table["all six in bf16"]
    e_fp = tiny_table["all six in fp16"]
    for i in range(2):
        # one eighth of the rounding step; allow for chance
        assert e_fp[i] < e_bf[i] / 4, (e_fp, e_bf)
        assert e_fp[i] > e_bf[i] / 20, (e_fp, e_bf)


def test_rounding_errors_add_in_quadrature(tiny_table):
    e_all = tiny_table["all six in bf16"]
    for i in range(2):
        singles = [tiny_table[f"{p} only, bf16"][i] for p in ps.POINTS]
        assert min(singles) > 0
        q = math.sqrt(sum(e * e for e in singles))
        assert 0.7 * e_all[i] < q < 1.35 * e_all[i], (q, e_all[i])


def test_memory_perturbation_grows_over_segments():
    """A 1e-4 relative change of M(., -1) in the fp32 oracle: after the first
    segments it grows with every further segment (the chain runs through the
    memory rows and attention); at the 1B shape it grows about 1.3x per
    segment (script: --workload llama1b --chaos 12)."""
    cfg = dataclasses.replace(ri.TINY_LLAMA, S=12)
    d = ps.chaos_growth(cfg, cfg.S, log=lambda m: None)
    assert d[-1] > 2.0 * d[3], d
    assert all(x > 0 for x in d)


def test_two_term_split_value():
    """hi + lo with both terms bf16: exact for bf16 values, and within 2^-16
    relative of any other value (each term keeps 8 significant bits)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))).astype(np.float32)
    y = ps.round_bf16x2(x)
    assert np.all(np.abs(y - x) <= 2.0 ** -16 * np.abs(x))
    b = ri.round_bf16(x)
    assert np.array_equal(ps.round_bf16x2(b), b)


def test_two_term_split_removes_a_points_error():
    """A point carried as hi + lo costs a small fraction of its bf16 error
    (measured ~1/750 at Q/K/V), and each further split point lowers the
    error of the all-bf16 cell."""
    cfg = ri.TINY_LLAMA
    t = ps.rounding_table(cfg, cfg.S, list(ps.SPLIT_VARIANTS) + [
        ("qkv only, bf16", ("qkv",), "bf16"), ("qkv only, bf16x2", ("qkv",), "bf16x2")],
        log=lambda m: None)
    for i in range(2):
        assert t["qkv only, bf16x2"][i] < t["qkv only, bf16"][i] / 100
        chain = [t[label][i] for label, _, _ in ps.SPLIT_VARIANTS[:4]]
        assert all(a > b for a, b in zip(chain, chain[1:])), chain
