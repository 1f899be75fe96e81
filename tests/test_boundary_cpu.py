"""The memory contract of the C ABI, checked on the CPU: a model handle is
created without any device call, the library sizes the caller's buffers
(rmt_workspace_bytes) from the configuration alone, refuses buffers that are
missing, misaligned or too small, and refuses a forward call before both
buffers are bound.  Also the Python binding's argument checks, which raise
before anything reaches the library."""
import ctypes as C
import dataclasses

import numpy as np
import pytest
import torch

import rmt_inputs as ri

FAKE = 1 << 20        # an aligned stand-in address; never dereferenced on these paths


def _L():
    from long_context_anti_amd import _lib
    return _lib


def _config(cfg):
    L = _L()
    dtype = L.RMT_F32 if cfg.dtype == ri.F32 else L.RMT_BF16
    return L.RmtConfig(cfg.cell, dtype, cfg.L, cfg.S, cfg.n, cfg.m, cfg.d, cfg.Hq, cfg.Hkv, cfg.hd,
                       cfg.F, cfg.V, cfg.eps, cfg.theta, int(cfg.post_norm))


def _fake_weights(cfg):
    """Non-NULL stand-ins for every field (the create call only records them)."""
    L = _L()
    w = L.RmtWeights()
    w.weight_dtype = L.RMT_F32 if cfg.dtype == ri.F32 else L.RMT_BF16
    for name, _ in L.RmtWeights._fields_[1:]:
        setattr(w, name, FAKE)
    return w


def _create(cfg):
    L = _L()
    c = _config(cfg)
    w = _fake_weights(cfg)
    h = C.c_void_p()
    assert L.lib().rmt_model_create(C.byref(c), C.byref(w), None, C.byref(h)) == L.RMT_OK, \
        L.lib().rmt_last_error()
    return h


def _bytes(h, kind):
    L = _L()
    v = C.c_size_t()
    assert L.lib().rmt_workspace_bytes(h, kind, C.byref(v)) == L.RMT_OK
    return v.value


def _al(x):
    return (x + 255) // 256 * 256


def _layout(sizes):
    off = 0
    for b in sizes:
        off = _al(off) + b
    return _al(off)


def test_create_makes_no_device_call():
    """This container has no GPU: a create that touched the device would fail."""
    L = _L()
    for cfg in (ri.TINY_LINEAR_GELU, ri.TINY_SWIGLU, ri.LLAMA_1B, ri.LLAMA_8B, ri.ENCODER_1B_POSTNORM):
        h = _create(cfg)
        v = C.c_size_t()
        assert L.lib().rmt_model_device_bytes(h, C.byref(v)) == L.RMT_OK and v.value == 0
        assert L.lib().rmt_model_destroy(h) == L.RMT_OK


def test_weight_buffer_size_llama1b():
    """Packed bf16 matrices [L][N][K] (gate/up interleaved, so 2F rows), fp32
    gains, the RoPE table [R][hd/2] of (cos, sin) and a 256-byte flag, each at
    a 256-byte boundary."""
    c = ri.LLAMA_1B
    L_, d, F, R = c.L, c.d, c.F, c.R
    nq, hq = c.n_qkv, c.Hq * c.hd
    want = _layout([L_ * 2 * F * d * 2, L_ * d * F * 2, L_ * d * 4, L_ * nq * d * 2, L_ * d * hq * 2,
                    L_ * d * 4, R * (c.hd // 2) * 8, 256])
    h = _create(c)
    assert _bytes(h, _L().RMT_BUF_WEIGHTS) == want
    _L().lib().rmt_model_destroy(h)


def test_workspace_size_llama1b_and_batch():
    """Per-launch buffers for min(32, B L) cells plus per-sequence X pairs and
    memory copies; the segment count does not enter."""
    c = ri.LLAMA_1B
    Lib = _L()

    def want(B):
        cells = min(32, B * c.L)
        rows = cells * c.R
        nc = c.d // 64          # 64-column chunk sums per row (RMSNorm inputs)
        # X slots' 16-bit copies and chunk sums (L + 1 slots: the last is a discard area), the same for
        # the memory rows, twice (ping-pong), then the launch's H chunk sums and 1/rms per row
        norm_inputs = [B * (c.L + 1) * c.n * c.d * 2, B * (c.L + 1) * c.n * nc * 4,
                       B * c.L * c.m * c.d * 2, B * c.L * c.m * nc * 4] * 2 + [rows * nc * 4, rows * 4]
        return _layout([rows * c.d * 2, rows * c.F * 2, rows * c.n_qkv * 2, rows * c.Hq * c.hd * 2,
                        rows * c.d * 4, B * c.L * c.n * c.d * 4, B * c.L * c.n * c.d * 4,
                        B * c.L * c.m * c.d * 4] + norm_inputs)
    h = _create(c)
    ws1 = _bytes(h, Lib.RMT_BUF_WORKSPACE)
    assert ws1 == want(1)
    assert Lib.lib().rmt_model_set_segments(h, 3) == Lib.RMT_OK
    assert _bytes(h, Lib.RMT_BUF_WORKSPACE) == ws1
    for B in (2, 3, 5):
        assert Lib.lib().rmt_model_set_batch(h, B) == Lib.RMT_OK
        assert _bytes(h, Lib.RMT_BUF_WORKSPACE) == want(B)
    Lib.lib().rmt_model_destroy(h)


def test_forward_needs_bound_buffers():
    Lib = _L()
    h = _create(ri.TINY_LLAMA)
    out = Lib.RmtOutput(FAKE, FAKE)
    p = C.c_void_p(FAKE)
    assert Lib.lib().rmt_forward_diagonal(h, p, p, C.byref(out)) == Lib.RMT_EWORKSPACE
    assert b"weight buffer" in Lib.lib().rmt_last_error()
    assert Lib.lib().rmt_forward_sequential(h, p, p, C.byref(out)) == Lib.RMT_EWORKSPACE
    flag = C.c_int32()
    assert Lib.lib().rmt_model_check(h, C.byref(flag)) == Lib.RMT_EWORKSPACE
    Lib.lib().rmt_model_destroy(h)


def test_bind_rejects_bad_buffers():
    Lib = _L()
    lib = Lib.lib()
    h = _create(ri.TINY_LLAMA)
    need_w = _bytes(h, Lib.RMT_BUF_WEIGHTS)
    need_ws = _bytes(h, Lib.RMT_BUF_WORKSPACE)
    assert lib.rmt_model_bind(None, Lib.RMT_BUF_WORKSPACE, FAKE, need_ws) == Lib.RMT_EINVAL
    assert lib.rmt_model_bind(h, Lib.RMT_BUF_WORKSPACE, None, need_ws) == Lib.RMT_EINVAL
    assert lib.rmt_model_bind(h, 7, FAKE, need_ws) == Lib.RMT_EINVAL
    assert lib.rmt_model_bind(h, Lib.RMT_BUF_WORKSPACE, FAKE + 64, need_ws) == Lib.RMT_EINVAL
    assert b"aligned" in lib.rmt_last_error()
    assert lib.rmt_model_bind(h, Lib.RMT_BUF_WORKSPACE, FAKE, need_ws - 1) == Lib.RMT_EWORKSPACE
    assert lib.rmt_model_bind(h, Lib.RMT_BUF_WEIGHTS, FAKE, need_w - 1) == Lib.RMT_EWORKSPACE
    v = C.c_size_t()
    assert lib.rmt_workspace_bytes(h, 9, C.byref(v)) == Lib.RMT_EINVAL
    assert lib.rmt_workspace_bytes(None, 0, C.byref(v)) == Lib.RMT_EINVAL
    lib.rmt_model_destroy(h)


def test_workspace_too_small_after_batch_grows():
    """Binding a workspace involves no device call; a larger batch then needs a
    larger one, and binding the old size again is refused."""
    Lib = _L()
    lib = Lib.lib()
    h = _create(ri.TINY_LLAMA)
    need1 = _bytes(h, Lib.RMT_BUF_WORKSPACE)
    assert lib.rmt_model_bind(h, Lib.RMT_BUF_WORKSPACE, FAKE, need1) == Lib.RMT_OK
    v = C.c_size_t()
    assert lib.rmt_model_device_bytes(h, C.byref(v)) == Lib.RMT_OK and v.value == need1
    assert lib.rmt_model_set_batch(h, 4) == Lib.RMT_OK
    need4 = _bytes(h, Lib.RMT_BUF_WORKSPACE)
    assert need4 > need1
    assert lib.rmt_model_bind(h, Lib.RMT_BUF_WORKSPACE, FAKE, need1) == Lib.RMT_EWORKSPACE
    assert lib.rmt_model_set_batch(h, 1) == Lib.RMT_OK
    lib.rmt_model_destroy(h)


def test_static_forward_refuses_models_beyond_its_scratch():
    """rmt_forward_diagonal_static compares the workspace a model needs with
    its 64 MiB array before any device call."""
    Lib = _L()
    h = _create(ri.LLAMA_1B)
    need = _bytes(h, Lib.RMT_BUF_WORKSPACE)
    assert need > Lib.STATIC_SCRATCH_BYTES
    out = Lib.RmtOutput(FAKE, FAKE)
    p = C.c_void_p(FAKE)
    assert Lib.lib().rmt_forward_diagonal_static(h, p, p, C.byref(out)) == Lib.RMT_EWORKSPACE
    assert b"static scratch" in Lib.lib().rmt_last_error()
    assert Lib.lib().rmt_forward_diagonal_static(None, p, p, C.byref(out)) == Lib.RMT_EINVAL
    Lib.lib().rmt_model_destroy(h)
    # the tiny grids fit
    for cfg in (ri.TINY_LLAMA, ri.TINY_ENCODER_POSTNORM, ri.TINY_LINEAR_GELU):
        h = _create(cfg)
        assert _bytes(h, Lib.RMT_BUF_WORKSPACE) <= Lib.STATIC_SCRATCH_BYTES
        Lib.lib().rmt_model_destroy(h)


# ---------------------------------------------------------------------------
# The Python binding's own checks (no library call is reached)
# ---------------------------------------------------------------------------

def _bare_model(cfg, B=1):
    import long_context_anti_amd as rmt
    m = object.__new__(rmt.RMTModel)
    m.cfg = _config(cfg)
    m.batch = B
    m.T = cfg.S * cfg.n
    m._handle = C.c_void_p()
    return m


def _io(cfg, B=1, tok_dtype=None):
    lead = (B,) if B > 1 else ()
    if cfg.cell == ri.CELL_LLAMA:
        tok = torch.zeros(lead + (cfg.T,), dtype=tok_dtype or torch.int32)
    else:
        tok = torch.zeros(lead + (cfg.T, cfg.d), dtype=tok_dtype or torch.bfloat16)
    mem0 = torch.zeros(lead + (cfg.L, cfg.m, cfg.d))
    hidden = torch.zeros(lead + (cfg.T, cfg.d))
    return tok, mem0, hidden, mem0.clone()


def test_wrapper_rejects_int64_token_ids():
    m = _bare_model(ri.TINY_LLAMA)
    tok, mem0, hidden, mem = _io(ri.TINY_LLAMA, tok_dtype=torch.int64)
    with pytest.raises(ValueError, match="tokens: dtype torch.int64"):
        m.forward_diagonal(tok, mem0, hidden, mem)


@pytest.mark.parametrize("which", ["mem0", "hidden", "mem"])
def test_wrapper_rejects_undersized_outputs(which):
    cfg = ri.TINY_LLAMA
    m = _bare_model(cfg)
    tok, mem0, hidden, mem = _io(cfg)
    bufs = {"mem0": mem0, "hidden": hidden, "mem": mem}
    bufs[which] = bufs[which][:-1]
    with pytest.raises(ValueError, match=f"{which}: shape"):
        m.forward_sequential(tok, bufs["mem0"], bufs["hidden"], bufs["mem"])


def test_wrapper_rejects_bf16_memory_and_batch_shape():
    cfg = ri.TINY_SWIGLU
    m = _bare_model(cfg, B=2)
    tok, mem0, hidden, mem = _io(cfg, B=2)
    with pytest.raises(ValueError, match="mem0: dtype"):
        m.forward_diagonal(tok, mem0.to(torch.bfloat16), hidden, mem)
    tok1, _, _, _ = _io(cfg, B=1)
    with pytest.raises(ValueError, match="tokens: shape"):
        m.forward_diagonal(tok1, mem0, hidden, mem)


def test_wrapper_rejects_host_tensors():
    cfg = ri.TINY_LLAMA
    m = _bare_model(cfg)
    with pytest.raises(ValueError, match="CUDA"):
        m.forward_diagonal(*_io(cfg))


def test_wrapper_accepts_a_leading_batch_of_one():
    cfg = ri.TINY_LLAMA
    m = _bare_model(cfg)
    tok, mem0, hidden, mem = _io(cfg, B=1)
    with pytest.raises(ValueError, match="CUDA"):       # shapes pass, placement does not
        m.forward_diagonal(tok[None], mem0[None], hidden[None], mem[None])


def test_wrapper_checks_weights():
    import long_context_anti_amd as rmt
    cfg = dataclasses.replace(ri.TINY_LLAMA, L=1, S=1)
    m = _bare_model(cfg)
    w = {"g1": torch.ones(1, cfg.d), "g2": torch.ones(1, cfg.d),
         "wqkv": torch.zeros(1, cfg.d, cfg.n_qkv, dtype=torch.bfloat16),
         "wo": torch.zeros(1, cfg.Hq * cfg.hd, cfg.d, dtype=torch.bfloat16),
         "wg": torch.zeros(1, cfg.d, cfg.F, dtype=torch.bfloat16),
         "wu": torch.zeros(1, cfg.d, cfg.F, dtype=torch.bfloat16),
         "wd": torch.zeros(1, cfg.F, cfg.d, dtype=torch.bfloat16),
         "embed": torch.zeros(cfg.V, cfg.d)}           # fp32: the library reads bf16
    with pytest.raises(ValueError, match="embed: dtype"):
        rmt.RMTModel._check_weights(m, w)
    w["embed"] = w["embed"].to(torch.bfloat16)
    w["wo"] = torch.zeros(1, cfg.d, cfg.Hq * cfg.hd + 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="wo: shape"):
        rmt.RMTModel._check_weights(m, w)
    w["wo"] = torch.zeros(1, cfg.Hq * cfg.hd, cfg.d, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):      # everything else is right
        rmt.RMTModel._check_weights(m, w)


def test_wrapper_grouped_gemm_layer_range():
    import long_context_anti_amd as rmt
    A = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    B = torch.zeros(3, 64, 64, dtype=torch.bfloat16)
    Cm = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"\[0, 3\)"):
        rmt.grouped_gemm(A, B, [0, 3], Cm)
    with pytest.raises(ValueError, match="entries"):
        rmt.grouped_gemm(A, B, [0], Cm)


def test_llama_memory_rows_must_be_whole_loads():
    """The LLaMA cell's QKV product reads the memory rows and the segment
    rows from separate buffers in 8-row loads: m must be a multiple of 8."""
    L = _L()
    bad = dataclasses.replace(ri.TINY_LLAMA, m=36)
    c = _config(bad)
    w = _fake_weights(bad)
    h = C.c_void_p()
    assert L.lib().rmt_model_create(C.byref(c), C.byref(w), None, C.byref(h)) == L.RMT_EUNSUPPORTED
    assert b"multiple of 8" in L.lib().rmt_last_error()
    ok = dataclasses.replace(ri.TINY_LLAMA, m=32)
    h = _create(ok)
    L.lib().rmt_model_destroy(h)
