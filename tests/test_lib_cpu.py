"""librmt.so on the CPU: it loads, exports every symbol include/rmt.h
declares, its host schedule matches the oracle's table bit for bit, and its
argument checks fire before any device call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmt.h")


def _lib():
    from long_context_anti_amd import _lib as L
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rmt_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("rmt_diag_schedule", "rmt_forward_diagonal", "rmt_forward_sequential",
                     "rmt_grouped_gemm", "rmt_model_create", "rmt_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    h = C.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name
    # the binding declares a signature for each of them
    assert set(declared_functions()) == set(L.SIGNATURES)


def _schedule_lib(L_, S):
    import long_context_anti_amd as rmt
    return rmt.diag_schedule(L_, S)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8, 12])
@pytest.mark.parametrize("S", [1, 2, 4, 7, 12])
def test_schedule_matches_oracle(L, S):
    dp, cells = _schedule_lib(L, S)
    dp_o, cells_o = orc.schedule_table(L, S)
    assert dp.dtype == np.int32 and np.array_equal(dp, dp_o)
    assert np.array_equal(cells, cells_o)


@pytest.mark.parametrize("cfg", [ri.TINY_LINEAR_GELU, ri.NORM_SWIGLU_1B, ri.LLAMA_1B, ri.LLAMA_8B],
                         ids=lambda c: c.name)
def test_schedule_matches_oracle_workloads(cfg):
    dp, cells = _schedule_lib(cfg.L, cfg.S)
    dp_o, cells_o = orc.schedule_table(cfg.L, cfg.S)
    assert np.array_equal(dp, dp_o) and np.array_equal(cells, cells_o)


def test_schedule_errors():
    L = _lib()
    h = L.lib()
    assert h.rmt_diag_schedule(4, 6, None, None) == 9
    assert h.rmt_diag_schedule(0, 6, None, None) == L.RMT_EINVAL
    assert b"L and S" in h.rmt_last_error()
    assert h.rmt_diag_schedule(4, -1, None, None) == L.RMT_EINVAL
    buf = (C.c_int32 * 16)()
    assert h.rmt_diag_schedule(4, 6, buf, None) == L.RMT_EINVAL
    assert h.rmt_diag_schedule(1 << 20, 1 << 20, None, None) == L.RMT_EINVAL


def _cfg(**kw):
    L = _lib()
    base = dict(cell=L.RMT_CELL_LLAMA, dtype=L.RMT_BF16, L=2, S=3, n=64, m=16, d=256, n_heads=4,
                n_kv_heads=1, head_dim=64, ffn=256, vocab=100, eps=1e-5, rope_theta=5e5)
    base.update(kw)
    return L.RmtConfig(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), -1), (dict(n=0), -1), (dict(head_dim=96, n_heads=2, d=192), -2),
    (dict(n_heads=6, n_kv_heads=2, d=384), -2), (dict(d=200), -2), (dict(ffn=100), -2), (dict(dtype=0), -2),
    (dict(cell=7), -1), (dict(vocab=0), -1), (dict(n_heads=3, n_kv_heads=2), -1),
])
def test_model_create_rejects_bad_configs(kw, code):
    L = _lib()
    cfg = _cfg(**kw)
    w = L.RmtWeights()
    handle = C.c_void_p()
    rc = L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(handle))
    assert rc == code, L.lib().rmt_last_error()
    assert not handle.value


def test_fp16_operands_are_a_llama_cell_option():
    """RMT_F16 (fp16 operands) is accepted for LLAMA cells and refused for the
    others; create makes no device call, so this runs on the CPU."""
    L = _lib()
    w = L.RmtWeights()
    for name, _ in L.RmtWeights._fields_[1:]:
        setattr(w, name, 1 << 20)
    h = C.c_void_p()
    cfg = _cfg(dtype=L.RMT_F16)
    assert L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(h)) == L.RMT_OK
    assert L.lib().rmt_model_destroy(h) == L.RMT_OK
    for cell, extra in ((L.RMT_CELL_NORM_SWIGLU, {}), (L.RMT_CELL_ENCODER, dict(n_kv_heads=4, ffn=1024))):
        cfg = _cfg(cell=cell, dtype=L.RMT_F16, **extra)
        h = C.c_void_p()
        assert L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(h)) == L.RMT_EUNSUPPORTED
        assert b"fp16" in L.lib().rmt_last_error()


def test_model_create_rejects_missing_weights():
    L = _lib()
    cfg = _cfg()
    w = L.RmtWeights()     # all NULL
    handle = C.c_void_p()
    assert L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(handle)) == L.RMT_EINVAL
    assert b"LLAMA needs" in L.lib().rmt_last_error() or b"required" in L.lib().rmt_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv_heads=2), -2),                       # one KV head per query head
    (dict(n_heads=4, n_kv_heads=4, head_dim=96, d=384), -2),
    (dict(ffn=100), -2), (dict(dtype=0), -2), (dict(n_heads=3, n_kv_heads=3, d=256), -2),
    (dict(post_norm=2), -1),
])
def test_encoder_create_rejects_bad_configs(kw, code):
    L = _lib()
    base = dict(cell=L.RMT_CELL_ENCODER, n_heads=4, n_kv_heads=4, ffn=1024)
    base.update(kw)
    cfg = _cfg(**base)
    w = L.RmtWeights()
    handle = C.c_void_p()
    rc = L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(handle))
    assert rc == code, L.lib().rmt_last_error()
    assert not handle.value


def test_post_norm_only_for_encoder_cells():
    L = _lib()
    w = L.RmtWeights()
    handle = C.c_void_p()
    cfg = _cfg(post_norm=1)       # a LLaMA cell
    assert L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(handle)) == L.RMT_EINVAL
    assert b"post_norm" in L.lib().rmt_last_error()


def test_encoder_create_rejects_missing_weights():
    L = _lib()
    cfg = _cfg(cell=L.RMT_CELL_ENCODER, n_heads=4, n_kv_heads=4, ffn=1024)
    w = L.RmtWeights()
    handle = C.c_void_p()
    assert L.lib().rmt_model_create(C.byref(cfg), C.byref(w), None, C.byref(handle)) == L.RMT_EINVAL
    assert b"ENCODER needs" in L.lib().rmt_last_error()


def test_attention_rejects_bad_arguments():
    L = _lib()
    h = L.lib()
    p = C.c_void_p(16)
    assert h.rmt_attention(0, 64, 4, 4, 64, 0, p, p, None) == L.RMT_EINVAL
    assert h.rmt_attention(1, 0, 4, 4, 64, 0, p, p, None) == L.RMT_EINVAL
    assert h.rmt_attention(1, 64, 4, 3, 64, 0, p, p, None) == L.RMT_EINVAL      # 4 % 3 != 0
    assert h.rmt_attention(1, 64, 6, 2, 64, 0, p, p, None) == L.RMT_EUNSUPPORTED  # ratio 3
    assert h.rmt_attention(1, 64, 4, 4, 96, 0, p, p, None) == L.RMT_EUNSUPPORTED
    assert h.rmt_attention(1, 64, 4, 4, 64, 0, None, p, None) == L.RMT_EINVAL
    assert h.rmt_causal_attention(1, 64, 6, 2, 64, p, p, None) == L.RMT_EUNSUPPORTED
    # one cell's qkv rows above 2 GiB: 65,536 rows x (64 + 2 * 64) heads x 128 x 2 bytes = 3 GiB
    assert h.rmt_attention(1, 65536, 64, 64, 128, 0, p, p, None) == L.RMT_EINVAL


def test_grouped_gemm_rejects_bad_shapes():
    L = _lib()
    h = L.lib()
    gl = (C.c_int32 * 1)(0)
    p = C.c_void_p(16)
    bf = L.RMT_BF16
    assert h.rmt_grouped_gemm(0, 128, 256, 64, 1, p, p, gl, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_grouped_gemm(33, 128, 256, 64, 1, p, p, gl, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_grouped_gemm(1, 128, 250, 64, 1, p, p, gl, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_grouped_gemm(1, 128, 256, 60, 1, p, p, gl, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_grouped_gemm(1, 128, 256, 64, 1, None, p, gl, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_grouped_gemm(1, 128, 256, 64, 0, p, p, gl, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_grouped_gemm(1, 128, 256, 64, 1, p, p, gl, p, L.RMT_F32, None) == L.RMT_EUNSUPPORTED
    # a layer index outside [0, Lw) is refused before any device work
    g3 = (C.c_int32 * 2)(0, 3)
    assert h.rmt_grouped_gemm(2, 128, 256, 64, 3, p, p, g3, p, bf, None) == L.RMT_EINVAL
    assert b"group_layer[1] = 3" in h.rmt_last_error()
    gneg = (C.c_int32 * 1)(-1)
    assert h.rmt_grouped_gemm(1, 128, 256, 64, 3, p, p, gneg, p, bf, None) == L.RMT_EINVAL
    assert h.rmt_pack_weight(1, 60, 64, p, 0, p, None) == L.RMT_EINVAL


def test_forward_rejects_null_model():
    L = _lib()
    out = L.RmtOutput(None, None)
    assert L.lib().rmt_forward_diagonal(None, None, None, C.byref(out)) == L.RMT_EINVAL
    assert L.lib().rmt_forward_sequential(None, None, None, C.byref(out)) == L.RMT_EINVAL
    assert L.lib().rmt_model_destroy(None) == L.RMT_OK
    assert L.lib().rmt_model_stage_times_groups(None, 1, 2, None, None, None, None) == L.RMT_EINVAL
    assert L.lib().rmt_model_set_batch(None, 2) == L.RMT_EINVAL
    assert L.lib().rmt_model_set_tokens(None, 100) == L.RMT_EINVAL
