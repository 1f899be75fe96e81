"""CPU oracle for diagonal-batched recurrent-memory-transformer (RMT) inference.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg may call
it.  It shares no code with the HIP library; the only thing both sides use is
the seeded input generator in ``rmt_inputs``.

What it computes, and where the pages say so
--------------------------------------------
Sources: "Diagonal Batching for Recurrent Memory Transformers" (skill page
summarising arXiv 2506.05229: sections *Core Concept*, *Architecture
Overview*, *Implementation*) and "Diagonal Batching Unlocks Parallelism in
Recurrent Memory Transformers for Long Contexts" (catalogue record, abstract).

* An RMT splits one long sequence into S segments of n tokens.  Layer l keeps
  m memory rows that carry state from segment s to segment s+1 (abstract:
  linear time, constant memory).  Cell (l, s) consumes
  ``A = [M(l, s-1); X(l-1, s)]`` (memory rows first) and produces R = m + n
  rows Y; the first n rows become X(l, s), the last m rows become M(l, s).
* The (layer, segment) grid is swept along anti-diagonals d = l + s
  (*Implementation*, the scheduler's diagonal enumeration; *Architecture
  Overview*, Diagonal Reorganization).  Every cell of a diagonal depends
  only on (l-1, s) and (l, s-1), so the reordering is exact (*Architecture
  Overview*, Dependency Preservation; the abstract states that the
  recurrence stays exact and only the run-time order of the computation
  changes).
* A sequence whose length T is not a multiple of n ends in a shorter
  segment of n' = T - (S-1) n rows (the *Implementation* sketch rounds the
  segment count up): its cells have m + n' rows, the first n' become X and
  the last m become M, the same split rule as every other cell.

Readings where the pages are silent (the design notes list each one):
  - the cell function is the one each workload defines: linear+GELU (tiny
    grid), RMSNorm+SwiGLU with residual (attention-free), or a pre-norm
    LLaMA block (RMSNorm, QKV, RoPE, causal GQA, O, RMSNorm, SwiGLU);
  - RMSNorm is ``x * rsqrt(mean(x^2) + eps) * g``;
  - RoPE is the rotate-half form with positions 0..R-1 local to the cell,
    memory rows included;
  - attention is causal over all R rows of the cell, scale 1/sqrt(hd),
    query head h reads KV head h // (Hq / Hkv);
  - GELU is the exact erf form;
  - the encoder-layer cell of the *Implementation* sketch (a stack of
    PyTorch ``nn.TransformerEncoderLayer`` modules whose argument values are
    stripped from the page) is read as the pre-norm layer with a 4x
    feed-forward: ``H = A + MHA(LN1(A))``, ``Y = H + FFN(LN2(H))``, where
    LayerNorm is ``(x - mean) / sqrt(var + eps) * g + b`` (biased variance),
    MHA projects with biases, attends over all R rows of the cell without a
    mask (scale 1/sqrt(hd), one KV head per query head) and projects out with
    a bias, and FFN is ``relu(z W1 + b1) W2 + b2``.  Dropout is the identity
    at inference.  The post-norm order (torch's default, ``norm_first=False``)
    is also provided: ``H = LN1(A + MHA(A))``, ``Y = LN2(H + FFN(H))``.

Arithmetic is in the dtype of the inputs (float32 by default, float64 for
the pins).  There is no blocking, fusion or reordering beyond the per-cell
definition: every product is one ``numpy.matmul`` call.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

CELL_LINEAR_GELU = 0
CELL_NORM_SWIGLU = 1
CELL_LLAMA = 2
CELL_ENCODER = 3


# ---------------------------------------------------------------------------
# Schedule.  Cell (l, s) needs (l-1, s) and (l, s-1) and nothing else
# (skill page, *Architecture Overview*, Dependency Preservation), so every
# cell can run one step after both of them: on anti-diagonal l + s
# (*Architecture Overview*, Diagonal Reorganization).  The grid has L + S - 1
# anti-diagonals, none of them empty.
# ---------------------------------------------------------------------------

def schedule(L: int, S: int) -> List[List[Tuple[int, int]]]:
    """Every cell of the L x S grid, grouped by its anti-diagonal l + s.
    Within a diagonal the cells are listed layer-ascending (the order is
    immaterial to the result; fixing it makes tables comparable)."""
    by_diagonal: List[List[Tuple[int, int]]] = [[] for _ in range(L + S - 1)]
    for l in range(L):
        for s in range(S):
            by_diagonal[l + s].append((l, s))
    return by_diagonal


def schedule_table(L: int, S: int) -> Tuple[np.ndarray, np.ndarray]:
    """CSR form of ``schedule``: ``diag_ptr[k]..diag_ptr[k+1]`` index the cells
    of diagonal k; each cell row is (layer, segment, slot), slot being the
    cell's position within its diagonal."""
    diags = schedule(L, S)
    diag_ptr = np.zeros(len(diags) + 1, np.int32)
    cells = np.zeros((L * S, 3), np.int32)
    k = 0
    for i, diag in enumerate(diags):
        for slot, (l, s) in enumerate(diag):
            cells[k] = (l, s, slot)
            k += 1
        diag_ptr[i + 1] = k
    return diag_ptr, cells


# ---------------------------------------------------------------------------
# Elementwise pieces of the cells.
# ---------------------------------------------------------------------------

def gelu_erf(z: np.ndarray) -> np.ndarray:
    """GELU, exact form: z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2))."""
    one = z.dtype.type(1.0)
    half = z.dtype.type(0.5)
    return half * z * (one + _erf(z / z.dtype.type(math.sqrt(2.0))))


def silu(t: np.ndarray) -> np.ndarray:
    """SiLU t * sigmoid(t)."""
    one = t.dtype.type(1.0)
    return t / (one + np.exp(-t))


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm: x * rsqrt(mean(x^2) + eps) * g."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * (x.dtype.type(1.0) / np.sqrt(ms + x.dtype.type(eps))) * g.astype(x.dtype)


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise LayerNorm: (x - mean) / sqrt(var + eps) * g + b, with the
    biased (population) variance of each row."""
    mu = np.mean(x, axis=-1, keepdims=True)
    xc = x - mu
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    return xc / np.sqrt(var + x.dtype.type(eps)) * g.astype(x.dtype) + b.astype(x.dtype)


def relu(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, z.dtype.type(0.0))


def rope_rotate_half(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding in the rotate-half layout.

    x: [R, H, hd].  Element i of the first half pairs with element i + hd/2;
    the pair turns by angle pos * theta**(-2i/hd).  Angles are formed in
    float64 and the cos/sin cast to x's dtype.
    """
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = pos.astype(np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang).astype(x.dtype)[:, None, :]
    sin = np.sin(ang).astype(x.dtype)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q_h k_j^T / sqrt(hd) + causal mask) v_j per query head h, with
    j = h // (Hq / Hkv).  q: [R, Hq, hd]; k, v: [R, Hkv, hd] -> [R, Hq*hd]."""
    R, Hq, hd = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    future = np.triu(np.ones((R, R), dtype=bool), k=1)
    out = np.empty((R, Hq, hd), dtype=q.dtype)
    for h in range(Hq):
        j = h // rep
        s = (q[:, h, :] @ k[:, j, :].T) * scale
        s[future] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, j, :]
    return out.reshape(R, Hq * hd)


def full_mha(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(q_h k_h^T / sqrt(hd)) v_h per head h, every row attending to
    every row (no mask).  q, k, v: [R, H, hd] -> [R, H*hd]."""
    R, H, hd = q.shape
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    out = np.empty((R, H, hd), dtype=q.dtype)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out.reshape(R, H * hd)


def swiglu(z: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """(silu(z Wg) * (z Wu)) Wd."""
    return (silu(z @ wg) * (z @ wu)) @ wd


# ---------------------------------------------------------------------------
# Cells.  A is [R, d] = [M(l, s-1); X(l-1, s)]; the result is Y [R, d].
# ---------------------------------------------------------------------------

def cell_linear_gelu(A: np.ndarray, w: Dict[str, np.ndarray]) -> np.ndarray:
    """Y = GELU(A W_l + b_l)."""
    return gelu_erf(A @ w["w"] + w["b"])


def cell_norm_swiglu(A: np.ndarray, w: Dict[str, np.ndarray], eps: float) -> np.ndarray:
    """Y = A + SwiGLU(RMSNorm(A))."""
    return A + swiglu(rms_norm(A, w["g2"], eps), w["wg"], w["wu"], w["wd"])


def cell_llama(A: np.ndarray, w: Dict[str, np.ndarray], Hq: int, Hkv: int, hd: int,
               eps: float, theta: float) -> np.ndarray:
    """Pre-norm LLaMA block over the cell's R rows:
    H = A + Attn(RMSNorm1(A)) Wo;  Y = H + SwiGLU(RMSNorm2(H))."""
    R = A.shape[0]
    h = rms_norm(A, w["g1"], eps)
    qkv = h @ w["wqkv"]
    nq, nk = Hq * hd, Hkv * hd
    q = qkv[:, :nq].reshape(R, Hq, hd)
    k = qkv[:, nq:nq + nk].reshape(R, Hkv, hd)
    v = qkv[:, nq + nk:nq + 2 * nk].reshape(R, Hkv, hd)
    pos = np.arange(R)
    q = rope_rotate_half(q, pos, theta)
    k = rope_rotate_half(k, pos, theta)
    att = causal_gqa_attention(q, k, v)
    H = A + att @ w["wo"]
    return H + swiglu(rms_norm(H, w["g2"], eps), w["wg"], w["wu"], w["wd"])


def _encoder_mha(z: np.ndarray, w: Dict[str, np.ndarray], H: int, hd: int) -> np.ndarray:
    """Biased Q/K/V projection, unmasked multi-head attention, biased output
    projection, on rows z [R, d]."""
    R = z.shape[0]
    qkv = z @ w["wqkv"] + w["bqkv"]
    nq = H * hd
    q = qkv[:, :nq].reshape(R, H, hd)
    k = qkv[:, nq:2 * nq].reshape(R, H, hd)
    v = qkv[:, 2 * nq:3 * nq].reshape(R, H, hd)
    return full_mha(q, k, v) @ w["wo"] + w["bo"]


def _encoder_ffn(z: np.ndarray, w: Dict[str, np.ndarray]) -> np.ndarray:
    return relu(z @ w["w1"] + w["b1"]) @ w["w2"] + w["b2"]


def cell_encoder(A: np.ndarray, w: Dict[str, np.ndarray], H: int, hd: int,
                 eps: float, post_norm: bool = False) -> np.ndarray:
    """Encoder layer over the cell's R rows.
    Pre-norm:  H = A + MHA(LN1(A));    Y = H + FFN(LN2(H)).
    Post-norm: H = LN1(A + MHA(A));    Y = LN2(H + FFN(H)).
    FFN(z) = relu(z W1 + b1) W2 + b2."""
    if post_norm:
        Hs = layer_norm(A + _encoder_mha(A, w, H, hd), w["ln1_g"], w["ln1_b"], eps)
        return layer_norm(Hs + _encoder_ffn(Hs, w), w["ln2_g"], w["ln2_b"], eps)
    Hs = A + _encoder_mha(layer_norm(A, w["ln1_g"], w["ln1_b"], eps), w, H, hd)
    return Hs + _encoder_ffn(layer_norm(Hs, w["ln2_g"], w["ln2_b"], eps), w)


def cell(cfg, w: Dict[str, np.ndarray], A: np.ndarray) -> np.ndarray:
    if cfg.cell == CELL_LINEAR_GELU:
        return cell_linear_gelu(A, w)
    if cfg.cell == CELL_NORM_SWIGLU:
        return cell_norm_swiglu(A, w, cfg.eps)
    if cfg.cell == CELL_LLAMA:
        return cell_llama(A, w, cfg.Hq, cfg.Hkv, cfg.hd, cfg.eps, cfg.theta)
    if cfg.cell == CELL_ENCODER:
        return cell_encoder(A, w, cfg.Hq, cfg.hd, cfg.eps, getattr(cfg, "post_norm", False))
    raise ValueError(f"unknown cell kind {cfg.cell}")


# ---------------------------------------------------------------------------
# Sweeps.
# ---------------------------------------------------------------------------

def _cast_weights(weights: Sequence[Dict[str, np.ndarray]], dtype) -> List[Dict[str, np.ndarray]]:
    return [{k: np.asarray(v, dtype=dtype) for k, v in w.items()} for w in weights]


def segment_input(cfg, inputs: np.ndarray, s: int, embed, dtype) -> np.ndarray:
    """X(-1, s): the segment's input rows -- n of them, fewer for a short last
    segment.  For the LLaMA cell ``inputs`` are token ids looked up in
    ``embed``; otherwise they are rows [T, d]."""
    n = cfg.n
    if cfg.cell == CELL_LLAMA:
        return np.asarray(embed[inputs[s * n:(s + 1) * n]], dtype=dtype)
    return np.asarray(inputs[s * n:(s + 1) * n], dtype=dtype)


def _num_segments(cfg, inputs) -> int:
    """ceil(T / n): a length that is not a multiple of n ends in a short segment."""
    T = inputs.shape[0]
    if T < 1:
        raise ValueError("empty sequence")
    return -(-T // cfg.n)


def forward_sequential(cfg, weights, inputs, mem0, embed=None, dtype=np.float32):
    """Segment by segment, then layer by layer.

    Returns (hidden [T, d] = X(L-1, .), memory [L, m, d] = M(., S-1)).
    The number of segments, ceil(T / n), is taken from ``inputs``."""
    S = _num_segments(cfg, inputs)
    L, n = cfg.L, cfg.n
    ws = _cast_weights(weights, dtype)
    M = [np.array(mem0[l], dtype=dtype) for l in range(L)]
    hidden = []
    for s in range(S):
        x = segment_input(cfg, inputs, s, embed, dtype)
        ns = x.shape[0]                      # n, or n' for a short last segment
        for l in range(L):
            A = np.concatenate([M[l], x], axis=0)
            Y = cell(cfg, ws[l], A)
            x, M[l] = Y[:ns], Y[ns:]
        hidden.append(x)
    return np.concatenate(hidden, axis=0), np.stack(M)


def forward_diagonal(cfg, weights, inputs, mem0, embed=None, dtype=np.float32):
    """The same recurrence swept along anti-diagonals d = l + s.

    Every cell of a diagonal reads its inputs as they stood at the end of the
    previous diagonal: all inputs of a diagonal are gathered first, then the
    cells run, and their X outputs go to a fresh buffer.  (Writing X in place
    while walking the diagonal would let cell (l-1, s+1) overwrite X(l-1, s)
    before cell (l, s) reads it.)"""
    S = _num_segments(cfg, inputs)
    L, n = cfg.L, cfg.n
    ws = _cast_weights(weights, dtype)
    M = [np.array(mem0[l], dtype=dtype) for l in range(L)]
    hidden = [None] * S
    prev_x: Dict[Tuple[int, int], np.ndarray] = {}
    for diag in schedule(L, S):
        A_list = []
        for (l, s) in diag:
            x_in = segment_input(cfg, inputs, s, embed, dtype) if l == 0 else prev_x[(l - 1, s)]
            A_list.append(np.concatenate([M[l], x_in], axis=0))
        next_x = {}
        for (l, s), A in zip(diag, A_list):
            Y = cell(cfg, ws[l], A)
            ns = A.shape[0] - cfg.m          # the segment's rows: n, or n' at the end
            next_x[(l, s)] = Y[:ns]
            M[l] = Y[ns:]
            if l == L - 1:
                hidden[s] = Y[:ns]
        prev_x = next_x
    return np.concatenate(hidden, axis=0), np.stack(M)


# ---------------------------------------------------------------------------
# Whole-sequence evaluation of the linear-GELU stack (no segment loop, no
# schedule), in float64.  The cell is row-wise, so the last m output rows of
# cell (l, s) depend only on input rows n..R-1, i.e. on X(l-1, s) rows
# n-m..n-1: M(l, s) = f_l(X(l-1, s)[n-m:n]).  Each layer is then two
# whole-sequence products: all memory rows first, then every cell's
# [M(l, s-1); X(l-1, s)] stacked into one [S*R, d] matrix.
# ---------------------------------------------------------------------------

def bruteforce_linear_gelu(cfg, weights, x0, mem0):
    """As above, for T = S_full * n + r rows: the r < n rows of a short last
    segment form one more, smaller product per layer.  Its memory comes from
    rows r .. r+m-1 of that cell's [M(l, S-2); X(l-1, S-1)], i.e. the last
    m - r rows of M(l, S-2) followed by its r input rows when r < m."""
    assert cfg.cell == CELL_LINEAR_GELU and cfg.m <= cfg.n
    L, n, m, d = cfg.L, cfg.n, cfg.m, cfg.d
    T = x0.shape[0]
    S, r = T // n, T % n                     # whole segments, rows of the short one
    x0 = np.asarray(x0, np.float64)
    X = x0[:S * n].reshape(S, n, d)
    Xr = x0[S * n:]                          # [r, d]
    mem_last = []
    for l in range(L):
        W = np.asarray(weights[l]["w"], np.float64)
        b = np.asarray(weights[l]["b"], np.float64)
        f = lambda rows: gelu_erf(rows @ W + b)  # noqa: E731
        last = np.asarray(mem0[l], np.float64)
        if S:
            M_all = f(X[:, n - m:, :].reshape(S * m, d)).reshape(S, m, d)
            M_prev = np.concatenate([last[None], M_all[:-1]], axis=0)
            A = np.concatenate([M_prev, X], axis=1).reshape(S * (m + n), d)
            X = f(A).reshape(S, m + n, d)[:, :n, :]
            last = M_all[-1]
        if r:
            Yr = f(np.concatenate([last, Xr], axis=0))   # the short cell, m + r rows
            Xr, last = Yr[:r], Yr[r:]
        mem_last.append(last)
    return np.concatenate([X.reshape(S * n, d), Xr], axis=0), np.stack(mem_last)
