"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle (or a mutated
copy of one of its functions, see test_oracle_mutations.py) disagrees with
what the pages or the mathematics fix.  None of them re-types the oracle's own
formula: they use a hand-written fixture, closed forms, a different evaluation
order in float64, or torch library routines.
"""
from __future__ import annotations

import math
import os
import re

import numpy as np
import torch
import torch.nn.functional as F

import rmt_inputs as ri
from oracle import rmt_oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def normwise(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# Schedule
# ---------------------------------------------------------------------------

def load_golden_schedule(name="schedule_L4_S6.txt"):
    diags = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, rest = line.split(":", 1)
            cells = [tuple(int(v) for v in c.split(",")) for c in re.findall(r"\((\d+,\d+)\)", rest)]
            assert int(head) == len(diags)
            diags.append(cells)
    return diags


def pin_schedule_golden(schedule=orc.schedule):
    assert schedule(4, 6) == load_golden_schedule()


def pin_schedule_invariants(L, S, schedule=orc.schedule):
    diags = schedule(L, S)
    assert len(diags) == L + S - 1
    where = {}
    for d, diag in enumerate(diags):
        assert len(diag) == min(d + 1, L, S, L + S - 1 - d)
        layers = [l for l, _ in diag]
        assert layers == sorted(layers)
        for (l, s) in diag:
            assert 0 <= l < L and 0 <= s < S and l + s == d
            assert (l, s) not in where
            where[(l, s)] = d
    assert len(where) == L * S
    for (l, s), d in where.items():
        if l > 0:
            assert where[(l - 1, s)] == d - 1
        if s > 0:
            assert where[(l, s - 1)] == d - 1


# ---------------------------------------------------------------------------
# Linear-GELU stack: float64 whole-sequence evaluation
# ---------------------------------------------------------------------------

def tiny_linear_gelu_inputs(cfg=ri.TINY_LINEAR_GELU, seed=0):
    return (ri.all_weights(cfg, seed), ri.input_embeddings(cfg, seed), ri.initial_memory(cfg, seed))


def pin_linear_gelu_bruteforce(forward=orc.forward_sequential, cfg=ri.TINY_LINEAR_GELU, tol=1e-5):
    w, x0, mem0 = tiny_linear_gelu_inputs(cfg)
    hid, mem = forward(cfg, w, x0, mem0)
    hid_bf, mem_bf = orc.bruteforce_linear_gelu(cfg, w, x0, mem0)
    assert normwise(hid, hid_bf) <= tol, normwise(hid, hid_bf)
    assert normwise(mem, mem_bf) <= tol, normwise(mem, mem_bf)


# ---------------------------------------------------------------------------
# Identity cells: a closed form for the recurrence plumbing
# ---------------------------------------------------------------------------

def shift_register_closed_form(cfg, x_stream, mem0):
    """With cells that return their input (Y = A), layer l's output stream is
    its input stream delayed by m rows with M(l, -1) in front, and M(l, S-1)
    is the last m rows of its input stream."""
    m = cfg.m
    stream = np.asarray(x_stream, np.float64)
    mem_last = []
    for l in range(cfg.L):
        mem_last.append(stream[-m:])
        stream = np.concatenate([np.asarray(mem0[l], np.float64), stream[:-m]], axis=0)
    return stream, np.stack(mem_last)


def identity_weights(cfg, seed=0):
    """Weights under which the residual cells compute Y = A exactly: the last
    projection of every branch is zero."""
    ws = ri.all_weights(cfg, seed)
    for w in ws:
        for key in ("wd", "wo", "bo", "w2", "b2"):
            if key in w:
                w[key] = np.zeros_like(w[key])
    return ws


def pin_shift_register(cfg, forward=orc.forward_sequential, seed=0):
    ws = identity_weights(cfg, seed)
    mem0 = ri.initial_memory(cfg, seed)
    if cfg.cell == ri.CELL_LLAMA:
        emb = ri.embedding(cfg, seed)
        tok = ri.tokens(cfg, seed)
        hid, mem = forward(cfg, ws, tok, mem0, emb)
        x_stream = emb[tok]
    else:
        x0 = ri.input_embeddings(cfg, seed)
        hid, mem = forward(cfg, ws, x0, mem0)
        x_stream = x0
    exp_hid, exp_mem = shift_register_closed_form(cfg, x_stream, mem0)
    assert np.array_equal(hid.astype(np.float64), exp_hid)
    assert np.array_equal(mem.astype(np.float64), exp_mem)


# ---------------------------------------------------------------------------
# One cell against torch library routines (float64)
# ---------------------------------------------------------------------------

def torch_rope_complex(x, theta):
    """RoPE as a complex rotation: pair (x_i, x_{i+hd/2}) is the complex number
    x_i + i x_{i+hd/2}, multiplied by exp(i p theta^(-2i/hd)).  x: [H, R, hd]."""
    H, R, hd = x.shape
    half = hd // 2
    z = torch.complex(x[..., :half].contiguous(), x[..., half:].contiguous())
    freqs = theta ** (-(2.0 * torch.arange(half, dtype=torch.float64)) / hd)
    ang = torch.arange(R, dtype=torch.float64)[:, None] * freqs[None, :]
    z = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def torch_llama_block(A, w, cfg):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    A = t(A)
    R, d = A.shape
    Hq, Hkv, hd = cfg.Hq, cfg.Hkv, cfg.hd
    h = F.rms_norm(A, (d,), weight=t(w["g1"]), eps=cfg.eps)
    qkv = h @ t(w["wqkv"])
    nq, nk = Hq * hd, Hkv * hd
    q = qkv[:, :nq].reshape(R, Hq, hd).transpose(0, 1)
    k = qkv[:, nq:nq + nk].reshape(R, Hkv, hd).transpose(0, 1)
    v = qkv[:, nq + nk:].reshape(R, Hkv, hd).transpose(0, 1).contiguous()
    q = torch_rope_complex(q, cfg.theta)
    k = torch_rope_complex(k, cfg.theta)
    rep = Hq // Hkv
    k = k.repeat_interleave(rep, dim=0)
    v = v.repeat_interleave(rep, dim=0)
    att = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
    att = att.transpose(0, 1).reshape(R, Hq * hd)
    H = A + att @ t(w["wo"])
    hn = F.rms_norm(H, (d,), weight=t(w["g2"]), eps=cfg.eps)
    return (H + (F.silu(hn @ t(w["wg"])) * (hn @ t(w["wu"]))) @ t(w["wd"])).numpy()


def torch_norm_swiglu_block(A, w, cfg):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    A = t(A)
    hn = F.rms_norm(A, (A.shape[1],), weight=t(w["g2"]), eps=cfg.eps)
    return (A + (F.silu(hn @ t(w["wg"])) * (hn @ t(w["wu"]))) @ t(w["wd"])).numpy()


def torch_encoder_block(A, w, cfg):
    """One torch ``nn.TransformerEncoderLayer`` -- the module the skill page's
    Implementation sketch stacks -- with a ReLU feed-forward and no dropout,
    pre-norm or post-norm as the workload says, in float64, loaded with the
    cell's weights (torch keeps Linear weights as [out, in], hence the
    transposes)."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    layer = torch.nn.TransformerEncoderLayer(
        d_model=cfg.d, nhead=cfg.Hq, dim_feedforward=cfg.F, dropout=0.0, activation="relu",
        layer_norm_eps=cfg.eps, batch_first=True, norm_first=not cfg.post_norm, dtype=torch.float64)
    layer.eval()
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(t(w["wqkv"]).T)
        layer.self_attn.in_proj_bias.copy_(t(w["bqkv"]))
        layer.self_attn.out_proj.weight.copy_(t(w["wo"]).T)
        layer.self_attn.out_proj.bias.copy_(t(w["bo"]))
        layer.linear1.weight.copy_(t(w["w1"]).T)
        layer.linear1.bias.copy_(t(w["b1"]))
        layer.linear2.weight.copy_(t(w["w2"]).T)
        layer.linear2.bias.copy_(t(w["b2"]))
        layer.norm1.weight.copy_(t(w["ln1_g"]))
        layer.norm1.bias.copy_(t(w["ln1_b"]))
        layer.norm2.weight.copy_(t(w["ln2_g"]))
        layer.norm2.bias.copy_(t(w["ln2_b"]))
        return layer(t(A)[None])[0].numpy()


def torch_block(A, w, cfg):
    if cfg.cell == ri.CELL_LLAMA:
        return torch_llama_block(A, w, cfg)
    if cfg.cell == ri.CELL_ENCODER:
        return torch_encoder_block(A, w, cfg)
    return torch_norm_swiglu_block(A, w, cfg)


def pin_single_segment_against_torch(cfg, forward=orc.forward_sequential, seed=0, tol=1e-11):
    """S = 1 and L = 1: the whole sweep is one cell on [M(0,-1); X(-1,0)],
    i.e. one standard pre-norm block over R rows."""
    import dataclasses
    c1 = dataclasses.replace(cfg, L=1, S=1)
    w = ri.all_weights(c1, seed)
    mem0 = ri.initial_memory(c1, seed)
    if c1.cell == ri.CELL_LLAMA:
        emb = ri.embedding(c1, seed)
        tok = ri.tokens(c1, seed)
        hid, mem = forward(c1, w, tok, mem0, emb, dtype=np.float64)
        A = np.concatenate([mem0[0], emb[tok]], axis=0)
        Y = torch_llama_block(A, w[0], c1)
    else:
        x0 = ri.input_embeddings(c1, seed)
        hid, mem = forward(c1, w, x0, mem0, dtype=np.float64)
        A = np.concatenate([mem0[0], x0], axis=0)
        Y = torch_block(A, w[0], c1)
    assert normwise(hid, Y[:c1.n]) <= tol, normwise(hid, Y[:c1.n])
    assert normwise(mem[0], Y[c1.n:]) <= tol, normwise(mem[0], Y[c1.n:])


# ---------------------------------------------------------------------------
# Elementwise pieces
# ---------------------------------------------------------------------------

def pin_gelu(gelu=orc.gelu_erf):
    x = np.linspace(-8, 8, 4001)
    ref = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.max(np.abs(gelu(x) - ref)) <= 1e-14
    # GELU(x) - GELU(-x) = x since Phi(x) + Phi(-x) = 1
    assert np.max(np.abs(gelu(x) - gelu(-x) - x)) <= 1e-14
    assert gelu(np.zeros(1))[0] == 0.0


def pin_silu(silu=orc.silu):
    x = np.linspace(-30, 30, 3001)
    ref = F.silu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(silu(x) - ref)) <= 1e-13
    assert np.max(np.abs(silu(x) - silu(-x) - x)) <= 1e-13


def pin_rms_norm(rms_norm=orc.rms_norm):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 33)) * 3.0
    g = rng.standard_normal(33)
    ref = F.rms_norm(torch.from_numpy(x), (33,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    assert np.max(np.abs(rms_norm(x, g, 1e-5) - ref)) <= 1e-13
    # with g = 1 and eps -> 0 every row has unit root-mean-square
    y = rms_norm(x, np.ones(33), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)


def pin_layer_norm(layer_norm=orc.layer_norm):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((7, 33)) * 3.0 + 1.5
    g = rng.standard_normal(33)
    b = rng.standard_normal(33)
    ref = F.layer_norm(torch.from_numpy(x), (33,), weight=torch.from_numpy(g),
                       bias=torch.from_numpy(b), eps=1e-5).numpy()
    assert np.max(np.abs(layer_norm(x, g, b, 1e-5) - ref)) <= 1e-13
    # with g = 1, b = 0 and eps -> 0 every row has mean 0 and (population) variance 1
    y = layer_norm(x, np.ones(33), np.zeros(33), 0.0)
    assert np.allclose(np.mean(y, axis=1), 0.0, atol=1e-14)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, atol=1e-13)
    # a constant added to a row leaves its normalised values unchanged (unlike RMSNorm)
    shifted = layer_norm(x + rng.standard_normal((7, 1)) * 10.0, g, b, 1e-5)
    assert np.allclose(shifted, layer_norm(x, g, b, 1e-5), atol=1e-12)


def pin_rope(rope=orc.rope_rotate_half, theta=500000.0):
    rng = np.random.default_rng(6)
    R, H, hd = 37, 3, 64
    x = rng.standard_normal((R, H, hd))
    pos = np.arange(R)
    y = rope(x, pos, theta)
    ref = torch_rope_complex(torch.from_numpy(x).transpose(0, 1), theta).transpose(0, 1).numpy()
    assert np.max(np.abs(y - ref)) <= 1e-12
    assert np.array_equal(rope(x[:1], np.zeros(1, int), theta), x[:1])      # p = 0 is the identity
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    assert np.allclose(rope(y, -pos, theta), x, atol=1e-12)               # R_{-p} R_p = I
    # <R_p q, R_r k> depends only on p - r
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    dots = [float(np.sum(rope(q, np.array([p + 5]), theta) * rope(k, np.array([p]), theta)))
            for p in (0, 11, 300)]
    assert np.allclose(dots, dots[0], atol=1e-12)


def attention_bruteforce(q, k, v):
    """Per query, per key, with math.exp: plain softmax-weighted sums."""
    R, Hq, hd = q.shape
    Hkv = k.shape[1]
    out = np.zeros((R, Hq, hd))
    for h in range(Hq):
        j = h * Hkv // Hq
        for i in range(R):
            scores = [sum(q[i, h, c] * k[t, j, c] for c in range(hd)) / math.sqrt(hd)
                      for t in range(i + 1)]
            mx = max(scores)
            e = [math.exp(sc - mx) for sc in scores]
            z = sum(e)
            for c in range(hd):
                out[i, h, c] = sum(e[t] * v[t, j, c] for t in range(i + 1)) / z
    return out.reshape(R, Hq * hd)


def pin_attention(attn=orc.causal_gqa_attention):
    rng = np.random.default_rng(7)
    R, Hq, Hkv, hd = 6, 4, 2, 4
    q = rng.standard_normal((R, Hq, hd))
    k = rng.standard_normal((R, Hkv, hd))
    v = rng.standard_normal((R, Hkv, hd))
    assert np.max(np.abs(attn(q, k, v) - attention_bruteforce(q, k, v))) <= 1e-13
    # constant values come back unchanged (softmax rows sum to one)
    vc = np.full_like(v, 0.375)
    assert np.allclose(attn(q, k, vc), 0.375, atol=1e-14)
    # row 0 attends only to itself
    out = attn(q, k, v).reshape(R, Hq, hd)
    for h in range(Hq):
        assert np.allclose(out[0, h], v[0, h * Hkv // Hq], atol=1e-14)


def full_attention_bruteforce(q, k, v):
    """Per query, per key, with math.exp, every key visible."""
    R, H, hd = q.shape
    out = np.zeros((R, H, hd))
    for h in range(H):
        for i in range(R):
            scores = [sum(q[i, h, c] * k[t, h, c] for c in range(hd)) / math.sqrt(hd)
                      for t in range(R)]
            mx = max(scores)
            e = [math.exp(sc - mx) for sc in scores]
            z = sum(e)
            for c in range(hd):
                out[i, h, c] = sum(e[t] * v[t, h, c] for t in range(R)) / z
    return out.reshape(R, H * hd)


def pin_full_attention(attn=orc.full_mha):
    rng = np.random.default_rng(9)
    R, H, hd = 6, 3, 4
    q = rng.standard_normal((R, H, hd))
    k = rng.standard_normal((R, H, hd))
    v = rng.standard_normal((R, H, hd))
    out = attn(q, k, v)
    assert np.max(np.abs(out - full_attention_bruteforce(q, k, v))) <= 1e-13
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a).transpose(0, 1)[None] for a in (q, k, v)),
                                         is_causal=False)[0].transpose(0, 1).reshape(R, H * hd).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-13
    # no mask: permuting the rows of q, k and v together permutes the output rows
    perm = rng.permutation(R)
    assert np.allclose(attn(q[perm], k[perm], v[perm]), out[perm], atol=1e-13)
    # constant values come back unchanged
    assert np.allclose(attn(q, k, np.full_like(v, -0.625)), -0.625, atol=1e-14)


# ---------------------------------------------------------------------------
# A short last segment (T not a multiple of n)
# ---------------------------------------------------------------------------

def ragged_inputs(cfg, T, seed=0):
    """The first T rows (or ids) of the workload's draw, with its weights,
    initial memory and embedding."""
    w = ri.all_weights(cfg, seed)
    mem0 = ri.initial_memory(cfg, seed)
    if cfg.cell == ri.CELL_LLAMA:
        return w, ri.tokens(cfg, seed)[:T].copy(), mem0, ri.embedding(cfg, seed)
    return w, ri.input_embeddings(cfg, seed)[:T].copy(), mem0, None


def pin_linear_gelu_bruteforce_ragged(T, forward=orc.forward_sequential, tol=1e-13):
    """fp64 sweep against the fp64 whole-sequence products with a short tail."""
    cfg = ri.TINY_LINEAR_GELU
    w, x0, mem0, _ = ragged_inputs(cfg, T)
    hid, mem = forward(cfg, w, x0, mem0, dtype=np.float64)
    hid_bf, mem_bf = orc.bruteforce_linear_gelu(cfg, w, x0, mem0)
    assert hid.shape == (T, cfg.d)
    assert normwise(hid, hid_bf) <= tol, normwise(hid, hid_bf)
    assert normwise(mem, mem_bf) <= tol, normwise(mem, mem_bf)


def pin_shift_register_ragged(cfg, T, forward=orc.forward_sequential):
    """Identity cells: the closed form holds for any segment lengths (the
    concatenated [M(l,-1); input stream] is cut into consecutive pieces)."""
    ws = identity_weights(cfg)
    _, x, mem0, emb = ragged_inputs(cfg, T)
    hid, mem = forward(cfg, ws, x, mem0, emb)
    x_stream = emb[x] if cfg.cell == ri.CELL_LLAMA else x
    exp_hid, exp_mem = shift_register_closed_form(cfg, x_stream, mem0)
    assert np.array_equal(hid.astype(np.float64), exp_hid)
    assert np.array_equal(mem.astype(np.float64), exp_mem)


def pin_short_single_segment_against_torch(cfg, n_short, forward=orc.forward_sequential, tol=1e-11):
    """S = 1, L = 1 with n' < n input rows: one pre-norm block over m + n' rows."""
    import dataclasses
    c1 = dataclasses.replace(cfg, L=1, S=1)
    w, x, mem0, emb = ragged_inputs(c1, n_short)
    hid, mem = forward(c1, w, x, mem0, emb, dtype=np.float64)
    rows = emb[x] if c1.cell == ri.CELL_LLAMA else x
    A = np.concatenate([mem0[0], rows], axis=0)
    Y = torch_block(A, w[0], c1)
    assert hid.shape[0] == n_short
    assert normwise(hid, Y[:n_short]) <= tol, normwise(hid, Y[:n_short])
    assert normwise(mem[0], Y[n_short:]) <= tol, normwise(mem[0], Y[n_short:])
