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
from ._lib import (RMT_BF16, RMT_F16, RMT_BUF_WEIGHTS, RMT_BUF_WORKSPACE, RMT_CELL_ENCODER,
                   RMT_CELL_LINEAR_GELU, RMT_CELL_LLAMA, RMT_CELL_NORM_SWIGLU, RMT_F32, STAGES,
                   RmtConfig, RmtError, RmtOutput, RmtWeights, check, lib)

__all__ = [
    "RMTModel", "RmtError", "diag_schedule", "grouped_gemm", "pack_weight", "causal_attention",
    "attention", "STAGES",
    "RMT_CELL_LINEAR_GELU", "RMT_CELL_NORM_SWIGLU", "RMT_CELL_LLAMA", "RMT_CELL_ENCODER", "RMT_F32",
    "RMT_BF16", "RMT_F16",
]


def _ptr(t) -> Optional[C.c_void_p]:
    return None if t is None else C.c_void_p(t.data_ptr())


def _require(t, name: str, dtypes, shape, device: bool = True) -> None:
    """Raise ValueError unless `t` is a contiguous tensor of one of `dtypes`
    and of `shape` (a tuple; None matches any extent), on the GPU unless
    `device` is False."""
    if t is None:
        raise ValueError(f"{name} is required")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if len(t.shape) != len(shape) or any(w is not None and int(v) != w for v, w in zip(t.shape, shape)):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) device tensor")


def _require_all(specs) -> None:
    """_require over (tensor, name, dtypes, shape) specs: every dtype and shape
    first, then placement, so that the message names the first real mismatch."""
    for spec in specs:
        _require(*spec, device=False)
    for spec in specs:
        _require(*spec)


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
    _require_all([(src, "src", (torch.bfloat16, torch.float32), (L, K, N)),
                  (dst, "dst", torch.bfloat16, (L, N, K))])
    dt = RMT_BF16 if src.dtype == torch.bfloat16 else RMT_F32
    check(lib().rmt_pack_weight(L, K, N, _ptr(src), dt, _ptr(dst), _stream(stream)))


def grouped_gemm(A, B, group_layer, C_out, stream=None) -> None:
    """C_out[g] = A[g] @ B[group_layer[g]]^T with A [G, M, K], B [Lw, N, K],
    C_out [G, M, N], all bf16 or all fp16 device tensors; group_layer a host
    int sequence with every entry in [0, Lw)."""
    import torch
    G, M, K = A.shape
    Lw, N = B.shape[0], B.shape[1]
    layers = [int(x) for x in group_layer]
    if len(layers) != G:
        raise ValueError(f"group_layer has {len(layers)} entries, A has {G} groups")
    if any(not 0 <= x < Lw for x in layers):
        raise ValueError(f"group_layer entries must lie in [0, {Lw})")
    dt = A.dtype if A.dtype in (torch.bfloat16, torch.float16) else torch.bfloat16
    _require_all([(A, "A", dt, (G, M, K)), (B, "B", dt, (Lw, N, K)), (C_out, "C_out", dt, (G, M, N))])
    gl = (C.c_int32 * G)(*layers)
    check(lib().rmt_grouped_gemm(G, M, N, K, Lw, _ptr(A), _ptr(B), gl, _ptr(C_out),
                                 RMT_F16 if dt == torch.float16 else RMT_BF16, _stream(stream)))


def attention(qkv, out, n_heads: int, n_kv_heads: int, head_dim: int, causal: bool = True,
              stream=None) -> None:
    """Attention over G cells, causal or unmasked: qkv [G, R, (Hq+2Hkv)*hd] ->
    out [G, R, Hq*hd], both bf16 device tensors."""
    import torch
    G, R = qkv.shape[0], qkv.shape[1]
    _require_all([(qkv, "qkv", torch.bfloat16, (G, R, (n_heads + 2 * n_kv_heads) * head_dim)),
                  (out, "out", torch.bfloat16, (G, R, n_heads * head_dim))])
    check(lib().rmt_attention(G, R, n_heads, n_kv_heads, head_dim, int(bool(causal)), _ptr(qkv),
                              _ptr(out), _stream(stream)))


def causal_attention(qkv, out, n_heads: int, n_kv_heads: int, head_dim: int, stream=None) -> None:
    """Causal GQA attention over G cells (rmt_causal_attention): qkv
    [G, R, (Hq+2Hkv)*hd] -> out [G, R, Hq*hd], both bf16 device tensors."""
    import torch
    G, R = qkv.shape[0], qkv.shape[1]
    _require_all([(qkv, "qkv", torch.bfloat16, (G, R, (n_heads + 2 * n_kv_heads) * head_dim)),
                  (out, "out", torch.bfloat16, (G, R, n_heads * head_dim))])
    check(lib().rmt_causal_attention(G, R, n_heads, n_kv_heads, head_dim, _ptr(qkv), _ptr(out),
                                     _stream(stream)))


class RMTModel:
    """A model handle (rmt_model_create).  `weights` maps the rmt_weights field
    names (w, b, g1, wqkv, wo, g2, wg, wu, wd, embed, and for the encoder cell
    beta1, bqkv, bo, beta2, w1, b1, w2, b2) to contiguous device tensors in the
    mathematical layout, stacked over layers.

    The library allocates no device memory: this wrapper allocates the packed
    weight buffer and the activation workspace as torch tensors, of the sizes
    rmt_workspace_bytes reports, and binds them (rmt_model_bind).  Packing
    happens at construction, after which only `embed` of `weights` is still
    read (the wrapper keeps a reference to it)."""

    _FIELDS = ("w", "b", "g1", "wqkv", "wo", "g2", "wg", "wu", "wd", "embed",
               "beta1", "bqkv", "bo", "beta2", "w1", "b1", "w2", "b2")
    _FP32_FIELDS = ("b", "g1", "g2", "beta1", "bqkv", "bo", "beta2", "b1", "b2")

    def __init__(self, *, cell: int, dtype: int, L: int, S: int, n: int, m: int, d: int,
                 n_heads: int = 0, n_kv_heads: int = 0, head_dim: int = 0, ffn: int = 0,
                 vocab: int = 0, eps: float = 1e-5, rope_theta: float = 500000.0,
                 post_norm: bool = False, weights: Dict[str, object], stream=None):
        import torch
        self.cfg = RmtConfig(cell, dtype, L, S, n, m, d, n_heads, n_kv_heads, head_dim, ffn, vocab,
                             eps, rope_theta, int(bool(post_norm)))
        self.batch = 1
        self.T = S * n
        self._handle = C.c_void_p()
        self.weight_buffer = None
        self.workspace = None
        wdt = self._check_weights(weights)
        w = RmtWeights(wdt, *[_ptr(weights.get(k)) for k in self._FIELDS])
        self._embed = weights.get("embed")     # borrowed by the library: keep it alive
        check(lib().rmt_model_create(C.byref(self.cfg), C.byref(w), _stream(stream),
                                     C.byref(self._handle)))
        nbytes = self.buffer_bytes(RMT_BUF_WEIGHTS)
        self.weight_buffer = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        check(lib().rmt_model_bind(self._handle, RMT_BUF_WEIGHTS, _ptr(self.weight_buffer), nbytes))
        self._ensure_workspace()

    def _check_weights(self, weights) -> int:
        """Dtypes and shapes of the weights the cell reads; returns weight_dtype."""
        import torch
        c = self.cfg
        L, d, F = c.L, c.d, c.ffn
        hq = c.n_heads * c.head_dim
        nq = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim
        if c.cell == RMT_CELL_LINEAR_GELU:
            shapes = {"w": (L, d, d), "b": (L, d)}
        elif c.cell == RMT_CELL_ENCODER:
            shapes = {"g1": (L, d), "beta1": (L, d), "wqkv": (L, d, nq), "bqkv": (L, nq),
                      "wo": (L, hq, d), "bo": (L, d), "g2": (L, d), "beta2": (L, d),
                      "w1": (L, d, F), "b1": (L, F), "w2": (L, F, d), "b2": (L, d)}
        else:
            shapes = {"g2": (L, d), "wg": (L, d, F), "wu": (L, d, F), "wd": (L, F, d)}
            if c.cell == RMT_CELL_LLAMA:
                shapes.update({"g1": (L, d), "wqkv": (L, d, nq), "wo": (L, hq, d),
                               "embed": (c.vocab, d)})
        mats = [k for k in shapes if k not in self._FP32_FIELDS and k != "embed"]
        if c.cell == RMT_CELL_LINEAR_GELU:
            mat_dtype = torch.float32
        else:
            first = weights.get(mats[0])
            mat_dtype = first.dtype if first is not None else torch.bfloat16
            if mat_dtype not in (torch.bfloat16, torch.float32):
                raise ValueError(f"{mats[0]}: dtype {mat_dtype}, expected torch.bfloat16 or torch.float32")
        specs = []
        for k, shape in shapes.items():
            if k in self._FP32_FIELDS:
                dt = torch.float32
            elif k == "embed":
                dt = torch.bfloat16
            else:
                dt = mat_dtype
            specs.append((weights.get(k), k, dt, shape))
        _require_all(specs)
        return RMT_BF16 if mat_dtype == torch.bfloat16 else RMT_F32

    def buffer_bytes(self, kind: int) -> int:
        """rmt_workspace_bytes: bytes the weight buffer (RMT_BUF_WEIGHTS) or the
        workspace for the current batch (RMT_BUF_WORKSPACE) needs."""
        v = C.c_size_t()
        check(lib().rmt_workspace_bytes(self._handle, kind, C.byref(v)))
        return v.value

    def _ensure_workspace(self) -> None:
        import torch
        need = self.buffer_bytes(RMT_BUF_WORKSPACE)
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
            check(lib().rmt_model_bind(self._handle, RMT_BUF_WORKSPACE, _ptr(self.workspace), need))

    # -- configuration -----------------------------------------------------
    def set_segments(self, S: int) -> None:
        check(lib().rmt_model_set_segments(self._handle, S))
        self.cfg.S = S
        self.T = S * self.cfg.n

    def set_tokens(self, T: int) -> None:
        """T tokens per sequence: ceil(T / n) segments, the last one short when
        T is not a multiple of n."""
        check(lib().rmt_model_set_tokens(self._handle, T))
        self.cfg.S = -(-T // self.cfg.n)
        self.T = T

    def set_batch(self, B: int) -> None:
        """B sequences per forward call: inputs and outputs gain a leading [B].
        A larger workspace is allocated and bound when the batch needs one."""
        check(lib().rmt_model_set_batch(self._handle, B))
        self.batch = B
        self._ensure_workspace()

    def set_stream(self, stream=None) -> None:
        check(lib().rmt_model_set_stream(self._handle, _stream(stream)))

    def device_bytes(self) -> int:
        v = C.c_size_t()
        check(lib().rmt_model_device_bytes(self._handle, C.byref(v)))
        return v.value

    # -- forward -----------------------------------------------------------
    def _check_io(self, tokens, mem0, hidden, mem) -> None:
        """Dtypes, shapes and placement of a forward call's buffers: [B, ...]
        with B sequences, or without the leading B when B = 1."""
        import torch
        c, B, T = self.cfg, self.batch, self.T

        def shaped(t, rest):
            if B == 1 and t is not None and len(t.shape) == len(rest) + 1:
                return (1,) + rest
            return ((B,) if B > 1 else ()) + rest
        if c.cell == RMT_CELL_LLAMA:
            tok = (tokens, "tokens", torch.int32, shaped(tokens, (T,)))
        else:
            dt = torch.float32 if c.dtype == RMT_F32 else torch.bfloat16
            tok = (tokens, "tokens", dt, shaped(tokens, (T, c.d)))
        _require_all([tok,
                      (mem0, "mem0", torch.float32, shaped(mem0, (c.L, c.m, c.d))),
                      (hidden, "hidden", torch.float32, shaped(hidden, (T, c.d))),
                      (mem, "mem", torch.float32, shaped(mem, (c.L, c.m, c.d)))])

    def _fwd(self, fn, tokens, mem0, hidden, mem) -> None:
        self._check_io(tokens, mem0, hidden, mem)
        out = RmtOutput(_ptr(hidden), _ptr(mem))
        check(fn(self._handle, _ptr(tokens), _ptr(mem0), C.byref(out)))

    def forward_diagonal(self, tokens, mem0, hidden, mem) -> None:
        self._fwd(lib().rmt_forward_diagonal, tokens, mem0, hidden, mem)

    def forward_sequential(self, tokens, mem0, hidden, mem) -> None:
        self._fwd(lib().rmt_forward_sequential, tokens, mem0, hidden, mem)

    def forward_diagonal_static(self, tokens, mem0, hidden, mem) -> None:
        """rmt_forward_diagonal with the library's static 64 MiB workspace
        instead of the bound one: allocates nothing (for callers that cannot);
        overlapping calls on one device race."""
        self._fwd(lib().rmt_forward_diagonal_static, tokens, mem0, hidden, mem)

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
