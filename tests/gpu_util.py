"""Helpers shared by the GPU tests: run a workload through the C ABI and
through the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import rmt_inputs as ri
from rmt_inputs import device as rdev


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


needs_gpu = pytest.mark.skipif(not gpu_available(), reason="no GPU in this environment")


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def inputs(cfg, S=None, seed=0):
    """Seeded weights, segment inputs, initial memory and embedding of a
    workload prefix of S segments."""
    S = cfg.S if S is None else S
    w = ri.all_weights(cfg, seed, workers=8)
    mem0 = ri.initial_memory(cfg, seed)
    if cfg.cell == ri.CELL_LLAMA:
        return w, ri.tokens(cfg, seed, S=S), mem0, ri.embedding(cfg, seed)
    return w, ri.input_embeddings(cfg, seed, S=S), mem0, None


class GpuRun:
    """A model built from seeded weights, with device inputs for S segments."""

    def __init__(self, cfg, S=None, seed=0, layers=None, embed=None, x=None, mem0=None, dtype=None):
        """dtype: the model's 16-bit type (RMT_BF16 or RMT_F16) when it is not
        the workload's own."""
        import torch
        import long_context_anti_amd as rmt
        self.cfg = cfg
        self.S = cfg.S if S is None else S
        if layers is None:
            layers, x, mem0, embed = inputs(cfg, self.S, seed)
        self.layers, self.x, self.mem0, self.embed = layers, x, mem0, embed
        dw = rdev.device_weights(cfg, layers, embed)
        kw = rdev.model_kwargs(cfg, self.S)
        if dtype is not None:
            kw["dtype"] = dtype
        self.model = rmt.RMTModel(**kw, weights=dw)
        self.embed_dev = dw.get("embed")
        del dw
        self.tokens = rdev.segment_inputs(cfg, x)
        self.mem0_dev = rdev.f32_tensor(mem0)
        T = self.S * cfg.n
        self.hidden = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
        self.mem = torch.empty((cfg.L, cfg.m, cfg.d), dtype=torch.float32, device="cuda")

    def run(self, path="diagonal"):
        import torch
        self.hidden.fill_(float("nan"))
        self.mem.fill_(float("nan"))
        fn = self.model.forward_diagonal if path == "diagonal" else self.model.forward_sequential
        fn(self.tokens, self.mem0_dev, self.hidden, self.mem)
        torch.cuda.synchronize()
        return self.hidden.cpu().numpy().copy(), self.mem.cpu().numpy().copy()

    def close(self):
        self.model.close()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def normwise(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
