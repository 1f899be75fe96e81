"""Diagonal-batched recurrent-memory-transformer inference on AMD MI355X.

Thin Python binding over librmt.so (C ABI in include/rmt.h): it only
marshals arguments.  Every step of the forward pass runs in the library's HIP
kernels; torch provides device memory and the stream.  There is no fallback:
if librmt.so is missing or fails to load, these calls raise.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional

import numpy as np

from . import _lib
from ._lib import (RMT_BF16, RMT_CELL_ENCODER, RMT_CELL_LINEAR_GELU, RMT_CELL_LLAMA,
                   RMT_CELL_NORM_SWIGLU, RMT_F32, STAGES, RmtConfig, RmtError, RmtOutput, RmtWeights,
                   check, lib)

__all__ = [
    "RMTModel", "RmtError", "diag_schedule", "grouped_gemm", "pack_weight", "causal_attention",
    "attention", "STAGES",
    "RMT_CELL_LINEAR_GELU", "RMT_CELL_NORM_SWIGLU", "RMT_CELL_LLAMA", "RMT_CELL_ENCODER", "RMT_F32",
    "RMT_BF16",
]


def _ptr(t) -> Optional[C.c_void_p]:
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def diag_schedule(L: int, S: int):
    """Anti-diagonal schedule as CSR arrays (diag_ptr [L+S], cells [L*S, 3])."""
    ndiag = check(lib().rmt_diag_schedule(L, S, None, None))
    diag_ptr = np.zeros(ndiag + 1, np.int32)
    cells = np.zeros((L * S, 3), np.int32)
    check(lib().rmt_diag_schedule(L, S, diag_ptr.ctypes.data_as(C.c_void_p),
                                  cells.ctypes.data_as(C.c_void_p)))
    return diag_ptr, cells


def pack_weight(src, dst, stream=None) -> None:
    """src [L, K, N] (fp32 or bf16, device) -> dst [L, N, K] bf16 (device)."""
    import torch
    L, K, N = src.shape
    assert dst.shape == (L, N, K) and dst.dtype == torch.bfloat16
    assert src.is_contiguous() and dst.is_contiguous()
    dt = RMT_BF16 if src.dtype == torch.bfloat16 else RMT_F32
    assert dt == RMT_BF16 or src.dtype == torch.float32
    check(lib().rmt_pack_weight(L, K, N, _ptr(src), dt, _ptr(dst), _stream(stream)))


def grouped_gemm(A, B, group_layer, C_out, stream=None) -> None:
    """C_out[g] = A[g] @ B[group_layer[g]]^T with A [G, M, K], B [Lw, N, K],
    C_out [G, M, N], all bf16 device tensors; group_layer a host int sequence."""
    import torch
    G, M, K = A.shape
    N = B.shape[1]
    assert B.shape[2] == K and C_out.shape == (G, M, N)
    for t in (A, B, C_out):
        assert t.dtype == torch.bfloat16 and t.is_contiguous()
    gl = (C.c_int32 * G)(*[int(x) for x in group_layer])
    check(lib().rmt_grouped_gemm(G, M, N, K, _ptr(A), _ptr(B), gl, _ptr(C_out), _stream(stream)))


def attention(qkv, out, n_heads: int, n_kv_heads: int, head_dim: int, causal: bool = True,
              stream=None) -> None:
    """Attention over G cells, causal or unmasked: qkv [G, R, (Hq+2Hkv)*hd] ->
    out [G, R, Hq*hd], both bf16 device tensors."""
    import torch
    G, R, W = qkv.shape
    assert W == (n_heads + 2 * n_kv_heads) * head_dim
    assert out.shape == (G, R, n_heads * head_dim)
    for t in (qkv, out):
        assert t.dtype == torch.bfloat16 and t.is_contiguous()
    check(lib().rmt_attention(G, R, n_heads, n_kv_heads, head_dim, int(bool(causal)), _ptr(qkv),
                              _ptr(out), _stream(stream)))


def causal_attention(qkv, out, n_heads: int, n_kv_heads: int, head_dim: int, stream=None) -> None:
    """Causal GQA attention over G cells (rmt_causal_attention): qkv
    [G, R, (Hq+2Hkv)*hd] -> out [G, R, Hq*hd], both bf16 device tensors."""
    import torch
    G, R, W = qkv.shape
    assert W == (n_heads + 2 * n_kv_heads) * head_dim
    assert out.shape == (G, R, n_heads * head_dim)
    for t in (qkv, out):
        assert t.dtype == torch.bfloat16 and t.is_contiguous()
    check(lib().rmt_causal_attention(G, R, n_heads, n_kv_heads, head_dim, _ptr(qkv), _ptr(out),
                                     _stream(stream)))


class RMTModel:
    """A model handle (rmt_model_create).  `weights` maps the rmt_weights field
    names (w, b, g1, wqkv, wo, g2, wg, wu, wd, embed, and for the encoder cell
    beta1, bqkv, bo, beta2, w1, b1, w2, b2) to contiguous device tensors in the
    mathematical layout, stacked over layers."""

    _FIELDS = ("w", "b", "g1", "wqkv", "wo", "g2", "wg", "wu", "wd", "embed",
               "beta1", "bqkv", "bo", "beta2", "w1", "b1", "w2", "b2")

    def __init__(self, *, cell: int, dtype: int, L: int, S: int, n: int, m: int, d: int,
                 n_heads: int = 0, n_kv_heads: int = 0, head_dim: int = 0, ffn: int = 0,
                 vocab: int = 0, eps: float = 1e-5, rope_theta: float = 500000.0,
                 post_norm: bool = False, weights: Dict[str, object], stream=None):
        import torch
        self.cfg = RmtConfig(cell, dtype, L, S, n, m, d, n_heads, n_kv_heads, head_dim, ffn, vocab,
                             eps, rope_theta, int(bool(post_norm)))
        big = [weights[k] for k in ("w", "wqkv", "wo", "wg", "wu", "wd", "w1", "w2")
               if weights.get(k) is not None]
        wdt = RMT_BF16 if big and big[0].dtype == torch.bfloat16 else RMT_F32
        for t in weights.values():
            if t is not None:
                assert t.is_contiguous() and t.is_cuda
        w = RmtWeights(wdt, *[_ptr(weights.get(k)) for k in self._FIELDS])
        self._embed = weights.get("embed")     # borrowed by the library: keep it alive
        self._handle = C.c_void_p()
        check(lib().rmt_model_create(C.byref(self.cfg), C.byref(w), _stream(stream),
                                     C.byref(self._handle)))

    # -- configuration -----------------------------------------------------
    def set_segments(self, S: int) -> None:
        check(lib().rmt_model_set_segments(self._handle, S))
        self.cfg.S = S

    def set_tokens(self, T: int) -> None:
        """T tokens per sequence: ceil(T / n) segments, the last one short when
        T is not a multiple of n."""
        check(lib().rmt_model_set_tokens(self._handle, T))
        self.cfg.S = -(-T // self.cfg.n)

    def set_batch(self, B: int) -> None:
        """B sequences per forward call: inputs and outputs gain a leading [B]."""
        check(lib().rmt_model_set_batch(self._handle, B))
        self.batch = B

    def set_stream(self, stream=None) -> None:
        check(lib().rmt_model_set_stream(self._handle, _stream(stream)))

    def device_bytes(self) -> int:
        v = C.c_size_t()
        check(lib().rmt_model_device_bytes(self._handle, C.byref(v)))
        return v.value

    # -- forward -----------------------------------------------------------
    def _fwd(self, fn, tokens, mem0, hidden, mem) -> None:
        out = RmtOutput(_ptr(hidden), _ptr(mem))
        check(fn(self._handle, _ptr(tokens), _ptr(mem0), C.byref(out)))

    def forward_diagonal(self, tokens, mem0, hidden, mem) -> None:
        self._fwd(lib().rmt_forward_diagonal, tokens, mem0, hidden, mem)

    def forward_sequential(self, tokens, mem0, hidden, mem) -> None:
        self._fwd(lib().rmt_forward_sequential, tokens, mem0, hidden, mem)

    def bad_tokens(self) -> bool:
        v = C.c_int32()
        check(lib().rmt_model_check(self._handle, C.byref(v)))
        return bool(v.value)

    # -- timing ------------------------------------------------------------
    def enable_timing(self, on: bool = True) -> None:
        check(lib().rmt_model_enable_timing(self._handle, 1 if on else 0))

    def stage_times(self, groups=None) -> Dict[str, dict]:
        """Per-stage totals of the timed launches since timing was enabled.
        With groups=(lo, hi), only launches that covered lo..hi cells, and the
        totals are kept; without, all launches, and the totals are cleared."""
        n = len(STAGES)
        ms = (C.c_double * n)()
        nl = (C.c_int64 * n)()
        fl = (C.c_double * n)()
        by = (C.c_double * n)()
        if groups is None:
            check(lib().rmt_model_stage_times(self._handle, ms, nl, fl, by))
        else:
            lo, hi = groups
            check(lib().rmt_model_stage_times_groups(self._handle, int(lo), int(hi), ms, nl, fl, by))
        return {name: {"ms": ms[i], "launches": nl[i], "flops": fl[i], "bytes": by[i]}
                for i, name in enumerate(STAGES)}

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            check(lib().rmt_model_destroy(self._handle))
            self._handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
