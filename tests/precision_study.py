"""Where the 16-bit path's error comes from, measured on the CPU.

TEST INFRASTRUCTURE (a study, not the product).  The LLaMA-shaped cell is
evaluated in fp32 exactly as the oracle defines it, except that the values the
GPU path stores in a 16-bit type -- each of them an MFMA operand -- can be
rounded at their point of the dataflow:

  norm1     the 16-bit operand of the Q/K/V product: y * g with 1/rms applied
            to the product's rows (the GPU's dataflow), or the normalised
            row itself (the oracle's order; --norm-order normalised)
  qkv       Q (after RoPE, carrying the softmax scale log2(e)/sqrt(hd)), K
            (after RoPE) and V, operands of the two attention products
  probs     the softmax probabilities, operand of P V (the row sums are taken
            over the rounded values, as on the GPU)
  attn_out  the attention output, operand of the O product
  norm2     the same for H, operand of the gate/up product
  u         silu(gate) * up, operand of the down product

to bf16 or to fp16 (round to nearest even), or to the value of a two-term
bf16 split (bf16x2: hi + lo, both bf16).  With no point rounded the cell
equals the oracle's ``cell_llama`` up to fp32 rounding order (pinned by
``tests/test_precision_study.py``).  The weights are bf16 values in both
cases; fp16 holds every one of them exactly except magnitudes below 2^-17
(about 0.03% of N(0, 0.02^2) draws), which round to fp16's 2^-24 grid.

Run as a script for the full-size tables quoted in the design notes, e.g.

    python tests/precision_study.py --workload llama8b --segments 2
    python tests/precision_study.py --workload llama1b --chaos 12
    python tests/precision_study.py --workload llama8b --segments 2 --split

(minutes of CPU time and tens of GB of memory at the 8B shape).
"""
from __future__ import annotations

import argparse
import math
import os
import sys
import time
from typing import Dict, Iterable, Tuple

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import rmt_inputs as ri  # noqa: E402
from oracle import rmt_oracle as orc  # noqa: E402

POINTS = ("norm1", "qkv", "probs", "attn_out", "norm2", "u")


def round_fp16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even fp16 value (numpy's conversion), back in fp32;
    magnitudes beyond 65504 become infinite."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def round_bf16x2(x: np.ndarray) -> np.ndarray:
    """The value of a two-term bf16 split, hi + lo with hi = bf16(x) and
    lo = bf16(x - hi): what an operand carries when each product is formed
    from both terms (hi W + lo W, or for Q K^T the three products qh kh +
    qh kl + ql kh, which drop only the ql kl term), accumulated in fp32."""
    x = np.asarray(x, np.float32)
    hi = ri.round_bf16(x)
    return (hi + ri.round_bf16((x - hi).astype(np.float32))).astype(np.float32)


ROUND = {"bf16": ri.round_bf16, "fp16": round_fp16, "bf16x2": round_bf16x2}


NORM_ORDERS = ("scaled_after", "normalised")


def emulated_llama_cell(A: np.ndarray, w: Dict[str, np.ndarray], cfg, points: Iterable[str],
                        fmt: str = "bf16", norm_order: str = "scaled_after") -> np.ndarray:
    """The pre-norm LLaMA cell in fp32 with the named points rounded to `fmt`
    (one format for every point, or a dict of per-point formats, bf16 for the
    points it does not name).

    norm_order says where an RMSNorm's 1/rms enters its GEMM, which decides
    what the norm1 / norm2 points round:
      scaled_after  the GPU's dataflow: the 16-bit operand is y * g, and the
                    product's rows are multiplied by 1/rms afterwards (in fp32)
      normalised    the oracle's order: the operand is rms_norm(y) * g itself
    Both equal rms_norm(y, g) @ W up to fp32 rounding when nothing is rounded.
    """
    pts = set(points)
    unknown = pts - set(POINTS)
    assert not unknown, unknown
    assert norm_order in NORM_ORDERS, norm_order
    fmts = fmt if isinstance(fmt, dict) else {}
    assert set(fmts) <= pts, (fmts, pts)

    def at(name, x):
        return ROUND[fmts.get(name, fmt if isinstance(fmt, str) else "bf16")](x) if name in pts else x

    def normed_product(name, y, g, Ws):
        """rms_norm(y, g) @ W for each W in Ws, with the rounding point `name`."""
        if norm_order == "normalised":
            z = at(name, orc.rms_norm(y, g, cfg.eps))
            return [z @ W for W in Ws]
        rinv = (np.float32(1.0) / np.sqrt(np.mean(y * y, axis=1, dtype=np.float32)
                                          + np.float32(cfg.eps))).astype(np.float32)
        z = at(name, (y * g).astype(np.float32))
        return [(z @ W) * rinv[:, None] for W in Ws]

    R = A.shape[0]
    Hq, Hkv, hd = cfg.Hq, cfg.Hkv, cfg.hd
    c = np.float32(math.log2(math.e) / math.sqrt(hd))
    (qkv,) = normed_product("norm1", A, w["g1"], [w["wqkv"]])
    nq, nk = Hq * hd, Hkv * hd
    pos = np.arange(R)
    q = orc.rope_rotate_half(qkv[:, :nq].reshape(R, Hq, hd), pos, cfg.theta) * c
    k = orc.rope_rotate_half(qkv[:, nq:nq + nk].reshape(R, Hkv, hd), pos, cfg.theta)
    v = qkv[:, nq + nk:].reshape(R, Hkv, hd)
    q, k, v = at("qkv", q), at("qkv", k), at("qkv", v)
    future = np.triu(np.ones((R, R), dtype=bool), k=1)
    att = np.empty((R, Hq, hd), np.float32)
    rep = Hq // Hkv
    for h in range(Hq):
        j = h // rep
        s2 = q[:, h, :] @ k[:, j, :].T          # scores in the base-2 domain
        s2[future] = -np.inf
        p = at("probs", np.exp2(s2 - s2.max(axis=1, keepdims=True)))
        att[:, h, :] = (p @ v[:, j, :]) / p.sum(axis=1, keepdims=True)
    att = at("attn_out", att.reshape(R, nq))
    H = A + att @ w["wo"]
    gate, up = normed_product("norm2", H, w["g2"], [w["wg"], w["wu"]])
    u = at("u", orc.silu(gate) * up)
    return H + u @ w["wd"]


def sweep(cfg, layers, tokens, mem0, embed, S: int, points=(), fmt="bf16", cell=None,
          norm_order="scaled_after"):
    """Segment by segment, layer by layer (the oracle's sequential order) over
    the first S segments with the emulated cell.  Returns (hidden, memory)."""
    cell = cell or (lambda A, w: emulated_llama_cell(A, w, cfg, points, fmt, norm_order))
    n = cfg.n
    M = [np.array(mem0[l], np.float32) for l in range(cfg.L)]
    hidden = []
    for s in range(S):
        x = np.asarray(embed[tokens[s * n:(s + 1) * n]], np.float32)
        for l in range(cfg.L):
            Y = cell(np.concatenate([M[l], x]), layers[l])
            x, M[l] = Y[:n], Y[n:]
        hidden.append(x)
    return np.concatenate(hidden), np.stack(M)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def load(cfg, S: int, seed: int = 0):
    layers = [{k: np.asarray(v, np.float32) for k, v in w.items()}
              for w in ri.all_weights(cfg, seed, workers=8)]
    return layers, ri.tokens(cfg, seed, S=S), ri.initial_memory(cfg, seed), ri.embedding(cfg, seed)


def rounding_table(cfg, S: int, variants, seed: int = 0, log=print,
                   norm_order: str = "scaled_after") -> Dict[str, Tuple[float, float]]:
    """Relative L2 error of hidden and memory after S segments, for each
    (label, points, fmt) variant, against the unrounded sweep (the oracle's
    cell up to fp32 rounding order)."""
    layers, tok, mem0, embed = load(cfg, S, seed)
    t0 = time.perf_counter()
    h_ref, m_ref = sweep(cfg, layers, tok, mem0, embed, S)
    log(f"reference sweep: {time.perf_counter() - t0:.1f} s")
    out = {}
    for label, points, fmt in variants:
        h, m = sweep(cfg, layers, tok, mem0, embed, S, points, fmt, norm_order=norm_order)
        out[label] = (rel_l2(h, h_ref), rel_l2(m, m_ref))
        log(f"{label:40s} hidden {out[label][0]:.3e}  mem {out[label][1]:.3e}")
    return out


def chaos_growth(cfg, S: int, rel: float = 1e-4, seed: int = 0, log=print):
    """Per-segment relative L2 difference of the hidden rows between the fp32
    oracle's sweep from M(., -1) and from M(., -1) perturbed by `rel` (relative,
    a seeded random direction)."""
    layers, tok, mem0, embed = load(cfg, S, seed)
    noise = np.random.default_rng(1234).standard_normal(mem0.shape).astype(np.float32)
    mem1 = (mem0 + rel * np.abs(mem0).mean() * noise).astype(np.float32)
    h0, _ = orc.forward_sequential(cfg, layers, tok, mem0, embed)
    h1, _ = orc.forward_sequential(cfg, layers, tok, mem1, embed)
    n = cfg.n
    diffs = [rel_l2(h1[s * n:(s + 1) * n], h0[s * n:(s + 1) * n]) for s in range(S)]
    for s, d in enumerate(diffs):
        log(f"segment {s:3d}: hidden difference {d:.3e}")
    return diffs


STANDARD_VARIANTS = (
    [("all six in bf16", POINTS, "bf16")]
    + [(f"{p} only, bf16", (p,), "bf16") for p in POINTS]
    + [("all six in fp16", POINTS, "fp16")]
)

# bf16 everywhere except two-term splits at the largest contributors: the
# Q/K/V product's A operand (norm1), then Q, K and V (qkv), then the gate/up
# product's A operand (norm2)
SPLIT_VARIANTS = (
    [("all six in bf16", POINTS, "bf16"),
     ("qkv as hi+lo, rest bf16", POINTS, {"qkv": "bf16x2"}),
     ("norm1 and qkv as hi+lo, rest bf16", POINTS, {"norm1": "bf16x2", "qkv": "bf16x2"}),
     ("norm1, qkv, norm2 as hi+lo, rest bf16", POINTS, {"norm1": "bf16x2", "qkv": "bf16x2",
                                                         "norm2": "bf16x2"}),
     ("all six in fp16", POINTS, "fp16")]
)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b", choices=["llama1b", "llama8b", "tiny_llama"])
    ap.add_argument("--segments", type=int, default=1)
    ap.add_argument("--chaos", type=int, default=0, help="segments of the perturbation study instead")
    ap.add_argument("--quick", action="store_true", help="only all-bf16 and all-fp16")
    ap.add_argument("--split", action="store_true",
                    help="two-term bf16 splits at the largest contributors instead")
    ap.add_argument("--norm-order", default="scaled_after", choices=NORM_ORDERS,
                    help="where 1/rms enters the GEMMs after the RMSNorms (what norm1/norm2 round)")
    args = ap.parse_args()
    cfg = {"llama1b": ri.LLAMA_1B, "llama8b": ri.LLAMA_8B, "tiny_llama": ri.TINY_LLAMA}[args.workload]
    print(f"{cfg.name}: L={cfg.L} d={cfg.d} R={cfg.R}", flush=True)
    if args.chaos:
        chaos_growth(cfg, args.chaos, log=lambda m: print(m, flush=True))
        return
    variants = STANDARD_VARIANTS if not args.quick else [STANDARD_VARIANTS[0], STANDARD_VARIANTS[-1]]
    if args.split:
        variants = SPLIT_VARIANTS
    print(f"norm order: {args.norm_order}", flush=True)
    rounding_table(cfg, args.segments, variants, log=lambda m: print(m, flush=True), norm_order=args.norm_order)


if __name__ == "__main__":
    main()
