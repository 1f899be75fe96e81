"""Seeded synthetic inputs and workload presets for diagonal-batched RMT inference.

This module is shared by the CPU oracle and by the HIP path's tests and bench.
It holds shapes and random draws only: no step of the method's arithmetic lives
here.  Every tensor is drawn from its own counter-style seed
``SeedSequence([seed, workload_id, tensor_kind, layer])`` so that any tensor
(one layer's weights, say) can be regenerated alone.

Conventions (the pages print no values, so these are readings):
  * weights are given in the mathematical layout ``W[d_in, d_out]`` so that a
    cell computes ``Y = A @ W``;
  * ``N(0, x)`` in the 1B/8B-shaped workloads means standard deviation ``x``;
    in the tiny linear-GELU workload and the isolated grouped GEMM it means
    variance ``x`` (the variance-preserving ``1/d`` initialisation);
  * bf16 workloads round every drawn tensor to bf16 (round to nearest even)
    and hand it out as float32 holding bf16-representable values, so both
    sides consume identical numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

CELL_LINEAR_GELU = 0
CELL_NORM_SWIGLU = 1
CELL_LLAMA = 2
CELL_ENCODER = 3

F32 = "f32"
BF16 = "bf16"

# Tensor kinds: part of each tensor's seed.
_KIND = {
    "w": 1, "b": 2, "x0": 3, "mem0": 4, "wqkv": 5, "wo": 6, "wg": 7, "wu": 8,
    "wd": 9, "embed": 10, "tokens": 11, "gemm_a": 12, "gemm_b": 13,
    "bqkv": 14, "bo": 15, "w1": 16, "b1": 17, "w2": 18, "b2": 19,
    "ln1_g": 20, "ln1_b": 21, "ln2_g": 22, "ln2_b": 23, "g1": 24, "g2": 25,
}


@dataclasses.dataclass(frozen=True)
class RMTConfig:
    """One recurrent-memory-transformer workload.

    L layers, S segments of n tokens, m memory rows per layer, width d.
    A cell (l, s) works on R = m + n rows: [M(l, s-1); X(l-1, s)].
    """
    name: str
    wid: int                  # workload id, part of every seed
    cell: int
    dtype: str
    L: int
    S: int
    n: int
    m: int
    d: int
    Hq: int = 0
    Hkv: int = 0
    hd: int = 0
    F: int = 0
    V: int = 0
    eps: float = 1e-5
    theta: float = 500000.0
    w_std: float = 0.02       # weight / embedding std (1B/8B-shaped cells)
    x_std: float = 1.0        # input-embedding std (cells that take rows directly)
    mem_std: float = 1.0      # initial memory std
    b_std: float = 0.02       # encoder cell: bias std
    ln_std: float = 0.1       # encoder cell: LayerNorm gain spread around 1, and shift std
    post_norm: bool = False   # encoder cell: LayerNorm after each residual add (torch's default)
    gain_std: float = 0.0     # RMSNorm gains: 1 (LLaMA initialisation) when 0, else 1 + N(0, gain_std)

    @property
    def R(self) -> int:
        return self.n + self.m

    @property
    def T(self) -> int:
        return self.S * self.n

    @property
    def n_qkv(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.hd

    def with_segments(self, S: int) -> "RMTConfig":
        return dataclasses.replace(self, S=S)


@dataclasses.dataclass(frozen=True)
class GemmConfig:
    """Isolated grouped GEMM: G groups of C_g = A_g @ B_{layer(g)}."""
    name: str
    wid: int
    M: int
    K: int
    N: int
    G_max: int
    G_sweep: Tuple[int, ...]


# The five workloads.  Sizes follow the diagonal-batching abstract's LLaMA-1B
# setting (131,072-token sequences) and an 8B-shaped variant.
TINY_LINEAR_GELU = RMTConfig(
    name="tiny_linear_gelu_L4_S6", wid=0, cell=CELL_LINEAR_GELU, dtype=F32,
    L=4, S=6, n=16, m=4, d=32, mem_std=1.0)
GROUPED_GEMM_1B = GemmConfig(
    name="grouped_gemm_1152x2048x8192", wid=1, M=1152, K=2048, N=8192,
    G_max=16, G_sweep=(1, 4, 8, 16))
NORM_SWIGLU_1B = RMTConfig(
    name="norm_swiglu_1b_L16_S32", wid=2, cell=CELL_NORM_SWIGLU, dtype=BF16,
    L=16, S=32, n=1024, m=128, d=2048, F=8192, w_std=0.02, x_std=1.0,
    mem_std=1.0)
LLAMA_1B = RMTConfig(
    name="llama1b_rmt_L16_S128", wid=3, cell=CELL_LLAMA, dtype=BF16,
    L=16, S=128, n=1024, m=128, d=2048, Hq=32, Hkv=8, hd=64, F=8192,
    V=32000, w_std=0.02, mem_std=0.02)
LLAMA_8B = RMTConfig(
    name="llama8b_rmt_L32_S64", wid=4, cell=CELL_LLAMA, dtype=BF16,
    L=32, S=64, n=2048, m=128, d=4096, Hq=32, Hkv=8, hd=128, F=14336,
    V=128000, w_std=0.02, mem_std=0.02)

# Small grids that still span several GEMM/attention tiles with ragged tails
# (R = 240 rows: 128 + 112; widths that are not multiples of 256).  Their
# RMSNorm gains are drawn around 1, so that the two norms of a cell differ and
# a dropped or exchanged gain changes the result.
TINY_SWIGLU = RMTConfig(
    name="tiny_norm_swiglu", wid=20, cell=CELL_NORM_SWIGLU, dtype=BF16,
    L=3, S=5, n=200, m=40, d=192, F=320, w_std=0.05, x_std=1.0, mem_std=1.0, gain_std=0.1)
TINY_LLAMA = RMTConfig(
    name="tiny_llama", wid=30, cell=CELL_LLAMA, dtype=BF16,
    L=3, S=4, n=200, m=40, d=256, Hq=4, Hkv=1, hd=64, F=384, V=1000,
    w_std=0.05, mem_std=0.05, gain_std=0.1)
TINY_LLAMA_HD128 = RMTConfig(
    name="tiny_llama_hd128", wid=31, cell=CELL_LLAMA, dtype=BF16,
    L=2, S=3, n=136, m=24, d=512, Hq=4, Hkv=1, hd=128, F=448, V=777,
    w_std=0.04, mem_std=0.04, gain_std=0.1)

# The encoder-layer cell of the skill page's Implementation sketch
# (nn.TransformerEncoderLayer with a 4x feed-forward), at the 1B width and
# 131,072 tokens, and two small grids (64- and 128-wide heads).
ENCODER_1B = RMTConfig(
    name="encoder1b_rmt_L16_S128", wid=5, cell=CELL_ENCODER, dtype=BF16,
    L=16, S=128, n=1024, m=128, d=2048, Hq=32, Hkv=32, hd=64, F=8192,
    w_std=0.02, x_std=1.0, mem_std=1.0)
TINY_ENCODER = RMTConfig(
    name="tiny_encoder", wid=40, cell=CELL_ENCODER, dtype=BF16,
    L=3, S=4, n=200, m=40, d=256, Hq=4, Hkv=4, hd=64, F=1024,
    w_std=0.05, x_std=1.0, mem_std=1.0)
TINY_ENCODER_HD128 = RMTConfig(
    name="tiny_encoder_hd128", wid=41, cell=CELL_ENCODER, dtype=BF16,
    L=2, S=3, n=136, m=24, d=512, Hq=4, Hkv=4, hd=128, F=2048,
    w_std=0.04, x_std=1.0, mem_std=1.0)

# The same encoder layer in the post-norm order (norm_first=False, torch's default).
ENCODER_1B_POSTNORM = dataclasses.replace(ENCODER_1B, name="encoder1b_postnorm_rmt_L16_S128", wid=6,
                                          post_norm=True)
TINY_ENCODER_POSTNORM = dataclasses.replace(TINY_ENCODER, name="tiny_encoder_postnorm", wid=42,
                                            post_norm=True)
TINY_ENCODER_POSTNORM_HD128 = dataclasses.replace(TINY_ENCODER_HD128, name="tiny_encoder_postnorm_hd128",
                                                  wid=43, post_norm=True)

# Rows wider than 2048 (the norm kernels' wide-row variant), in both norm orders.
TINY_ENCODER_WIDE = RMTConfig(
    name="tiny_encoder_wide", wid=44, cell=CELL_ENCODER, dtype=BF16,
    L=2, S=2, n=100, m=20, d=2560, Hq=20, Hkv=20, hd=128, F=10240,
    w_std=0.02, x_std=1.0, mem_std=1.0)
TINY_ENCODER_WIDE_POSTNORM = dataclasses.replace(TINY_ENCODER_WIDE, name="tiny_encoder_wide_postnorm",
                                                 wid=45, post_norm=True)

PRESETS: Dict[str, RMTConfig] = {
    c.name: c for c in (TINY_LINEAR_GELU, NORM_SWIGLU_1B, LLAMA_1B, LLAMA_8B,
                        TINY_SWIGLU, TINY_LLAMA, TINY_LLAMA_HD128, ENCODER_1B,
                        TINY_ENCODER, TINY_ENCODER_HD128, ENCODER_1B_POSTNORM,
                        TINY_ENCODER_POSTNORM, TINY_ENCODER_POSTNORM_HD128, TINY_ENCODER_WIDE,
                        TINY_ENCODER_WIDE_POSTNORM)
}


def rng_for(seed: int, wid: int, kind: str, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), int(wid), _KIND[kind], int(layer)])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16 value, returned as fp32 (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable fp32 array -> its uint16 bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def normal(shape, std: float, seed: int, wid: int, kind: str, layer: int = 0,
           bf16: bool = False) -> np.ndarray:
    x = rng_for(seed, wid, kind, layer).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_bf16(x) if bf16 else x


# ---------------------------------------------------------------------------
# Per-workload tensors.  Each function returns float32 arrays (bf16-valued for
# bf16 workloads) in the mathematical layout.
# ---------------------------------------------------------------------------

def layer_weights(cfg: RMTConfig, layer: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """Weights of one layer, W[d_in, d_out]."""
    bf = cfg.dtype == BF16
    d = cfg.d
    if cfg.cell == CELL_LINEAR_GELU:
        return {
            "w": normal((d, d), 1.0 / math.sqrt(d), seed, cfg.wid, "w", layer, bf),
            "b": normal((d,), 0.1, seed, cfg.wid, "b", layer, bf),
        }
    if cfg.cell == CELL_ENCODER:
        # gains 1 + N(0, ln_std), shifts and biases drawn too, so that no term
        # of the cell is zero
        F, hd3 = cfg.F, 3 * cfg.Hq * cfg.hd
        return {
            "ln1_g": 1.0 + normal((d,), cfg.ln_std, seed, cfg.wid, "ln1_g", layer, bf),
            "ln1_b": normal((d,), cfg.ln_std, seed, cfg.wid, "ln1_b", layer, bf),
            "wqkv": normal((d, hd3), cfg.w_std, seed, cfg.wid, "wqkv", layer, bf),
            "bqkv": normal((hd3,), cfg.b_std, seed, cfg.wid, "bqkv", layer, bf),
            "wo": normal((cfg.Hq * cfg.hd, d), cfg.w_std, seed, cfg.wid, "wo", layer, bf),
            "bo": normal((d,), cfg.b_std, seed, cfg.wid, "bo", layer, bf),
            "ln2_g": 1.0 + normal((d,), cfg.ln_std, seed, cfg.wid, "ln2_g", layer, bf),
            "ln2_b": normal((d,), cfg.ln_std, seed, cfg.wid, "ln2_b", layer, bf),
            "w1": normal((d, F), cfg.w_std, seed, cfg.wid, "w1", layer, bf),
            "b1": normal((F,), cfg.b_std, seed, cfg.wid, "b1", layer, bf),
            "w2": normal((F, d), cfg.w_std, seed, cfg.wid, "w2", layer, bf),
            "b2": normal((d,), cfg.b_std, seed, cfg.wid, "b2", layer, bf),
        }
    def gain(kind):
        if cfg.gain_std == 0.0:
            return np.ones((d,), np.float32)
        return (1.0 + normal((d,), cfg.gain_std, seed, cfg.wid, kind, layer, bf)).astype(np.float32)

    out = {
        "g2": gain("g2"),
        "wg": normal((d, cfg.F), cfg.w_std, seed, cfg.wid, "wg", layer, bf),
        "wu": normal((d, cfg.F), cfg.w_std, seed, cfg.wid, "wu", layer, bf),
        "wd": normal((cfg.F, d), cfg.w_std, seed, cfg.wid, "wd", layer, bf),
    }
    if cfg.cell == CELL_LLAMA:
        out["g1"] = gain("g1")
        out["wqkv"] = normal((d, cfg.n_qkv), cfg.w_std, seed, cfg.wid, "wqkv", layer, bf)
        out["wo"] = normal((cfg.Hq * cfg.hd, d), cfg.w_std, seed, cfg.wid, "wo", layer, bf)
    return out


def all_weights(cfg: RMTConfig, seed: int = 0, layers: Optional[range] = None, workers: int = 1):
    """Per-layer weights.  `workers` > 1 draws layers on a thread pool (each
    layer has its own generator, so the values do not depend on it)."""
    layers = range(cfg.L) if layers is None else layers
    if workers <= 1:
        return [layer_weights(cfg, l, seed) for l in layers]
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda l: layer_weights(cfg, l, seed), layers))


def embedding(cfg: RMTConfig, seed: int = 0) -> np.ndarray:
    assert cfg.cell == CELL_LLAMA
    return normal((cfg.V, cfg.d), cfg.w_std, seed, cfg.wid, "embed", 0, cfg.dtype == BF16)


def tokens(cfg: RMTConfig, seed: int = 0, S: Optional[int] = None) -> np.ndarray:
    """Token ids, uniform over the vocabulary.  A prefix of S segments is the
    first S*n ids of the full draw."""
    assert cfg.cell == CELL_LLAMA
    ids = rng_for(seed, cfg.wid, "tokens").integers(0, cfg.V, size=cfg.T, dtype=np.int64)
    ids = ids.astype(np.int32)
    return ids if S is None else ids[: S * cfg.n].copy()


def input_embeddings(cfg: RMTConfig, seed: int = 0, S: Optional[int] = None) -> np.ndarray:
    """Segment inputs X(-1, s) as rows [T, d] for the cells that take
    embeddings directly.  A prefix is the first S*n rows of the full draw."""
    assert cfg.cell in (CELL_LINEAR_GELU, CELL_NORM_SWIGLU, CELL_ENCODER)
    x = normal((cfg.T, cfg.d), cfg.x_std, seed, cfg.wid, "x0", 0, cfg.dtype == BF16)
    return x if S is None else x[: S * cfg.n].copy()


def initial_memory(cfg: RMTConfig, seed: int = 0) -> np.ndarray:
    """M(l, -1) for every layer, [L, m, d]."""
    return np.stack([
        normal((cfg.m, cfg.d), cfg.mem_std, seed, cfg.wid, "mem0", l, cfg.dtype == BF16)
        for l in range(cfg.L)
    ])


def gemm_operands(gc: GemmConfig, seed: int = 0, G: Optional[int] = None):
    """A_g [M, K] ~ N(0, 1) and B_g [K, N] with variance 1/K, bf16-valued."""
    G = gc.G_max if G is None else G
    A = np.stack([normal((gc.M, gc.K), 1.0, seed, gc.wid, "gemm_a", g, True) for g in range(G)])
    B = np.stack([normal((gc.K, gc.N), 1.0 / math.sqrt(gc.K), seed, gc.wid, "gemm_b", g, True)
                  for g in range(G)])
    return A, B
