"""A short last segment (rmt_model_set_tokens with T not a multiple of n):
the GPU against the oracle (fp32: normwise <= 1e-4; bf16: relative L2 <=
2e-2 on hidden and memory), diagonal equal to sequential bit for bit, the
whole segments equal to a run over just those segments, and a batch of two
short-tailed sequences equal to its single runs."""
import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc
from rmt_inputs import device as rdev

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]


def _inputs(cfg, T, seed=0):
    layers = ri.all_weights(cfg, seed, workers=8)
    mem0 = ri.initial_memory(cfg, seed)
    if cfg.cell == ri.CELL_LLAMA:
        return layers, ri.tokens(cfg, seed)[:T].copy(), mem0, ri.embedding(cfg, seed)
    return layers, ri.input_embeddings(cfg, seed)[:T].copy(), mem0, None


def _run(model, x_d, mem0_d, T, cfg, path="diagonal", B=None):
    import torch
    shape_h = (T, cfg.d) if B is None else (B, T, cfg.d)
    shape_m = (cfg.L, cfg.m, cfg.d) if B is None else (B, cfg.L, cfg.m, cfg.d)
    hidden = torch.full(shape_h, float("nan"), dtype=torch.float32, device="cuda")
    mem = torch.full(shape_m, float("nan"), dtype=torch.float32, device="cuda")
    fn = model.forward_diagonal if path == "diagonal" else model.forward_sequential
    fn(x_d, mem0_d, hidden, mem)
    torch.cuda.synchronize()
    return hidden.cpu().numpy(), mem.cpu().numpy()


CASES = [(ri.TINY_LINEAR_GELU, 5 * 16 + 7), (ri.TINY_LINEAR_GELU, 5 * 16 + 2), (ri.TINY_LINEAR_GELU, 9),
         (ri.TINY_SWIGLU, 4 * 200 + 67), (ri.TINY_LLAMA, 3 * 200 + 66), (ri.TINY_LLAMA, 3 * 200 + 1),
         (ri.TINY_LLAMA_HD128, 2 * 136 + 45), (ri.TINY_ENCODER, 3 * 200 + 33),
         (ri.TINY_ENCODER_HD128, 2 * 136 + 1), (ri.TINY_ENCODER_POSTNORM, 3 * 200 + 77)]


@pytest.mark.parametrize("cfg,T", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_short_last_segment(cfg, T):
    import long_context_anti_amd as rmt
    gu.say(f"[ragged] {cfg.name} T={T} (n={cfg.n})")
    layers, x, mem0, embed = _inputs(cfg, T)
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=dw)
    model.set_tokens(T)
    x_d, mem0_d = rdev.segment_inputs(cfg, x), rdev.f32_tensor(mem0)
    hd, md = _run(model, x_d, mem0_d, T, cfg)
    hs, ms = _run(model, x_d, mem0_d, T, cfg, "sequential")
    assert np.array_equal(hd, hs) and np.array_equal(md, ms)
    ho, mo = orc.forward_sequential(cfg, layers, x, mem0, embed)
    assert ho.shape == hd.shape
    if cfg.dtype == ri.F32:
        assert gu.normwise(hd, ho) <= 1e-4 and gu.normwise(md, mo) <= 1e-4
    else:
        e_h, e_m = gu.rel_l2(hd, ho), gu.rel_l2(md, mo)
        gu.say(f"  rel L2 hidden {e_h:.3e} mem {e_m:.3e}")
        assert e_h <= 2e-2 and e_m <= 2e-2
    # the whole segments alone give the same rows, bit for bit
    S_full = T // cfg.n
    if S_full:
        model.set_segments(S_full)
        hp, _ = _run(model, x_d[:S_full * cfg.n], mem0_d, S_full * cfg.n, cfg)
        assert np.array_equal(hd[:S_full * cfg.n], hp)
    model.close()


def test_batch_of_short_tailed_sequences():
    import torch
    import long_context_anti_amd as rmt
    cfg = ri.TINY_LLAMA
    T = 3 * cfg.n + 90
    gu.say(f"[ragged] {cfg.name} T={T} B=2")
    layers, _, _, embed = _inputs(cfg, T)
    xs = [ri.tokens(cfg, 50 + b)[:T].copy() for b in range(2)]
    mems = [ri.initial_memory(cfg, 50 + b) for b in range(2)]
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=dw)
    model.set_tokens(T)
    singles = [_run(model, rdev.segment_inputs(cfg, xs[b]), rdev.f32_tensor(mems[b]), T, cfg)
               for b in range(2)]
    model.set_batch(2)
    tok = torch.stack([rdev.segment_inputs(cfg, x) for x in xs]).contiguous()
    hb, mb = _run(model, tok, rdev.f32_tensor(np.stack(mems)), T, cfg, B=2)
    for b in range(2):
        assert np.array_equal(hb[b], singles[b][0]) and np.array_equal(mb[b], singles[b][1])
    model.close()


def test_set_tokens_rejects_bad_lengths():
    from long_context_anti_amd import _lib
    run = gu.GpuRun(ri.TINY_LLAMA, S=1)
    assert _lib.lib().rmt_model_set_tokens(run.model._handle, 0) == _lib.RMT_EINVAL
    assert _lib.lib().rmt_model_set_tokens(run.model._handle, -5) == _lib.RMT_EINVAL
    run.close()


def test_llama1b_width_short_tail():
    """All 16 layers at full width, one whole segment and one of 500 tokens
    (a 628-row cell: its third 288-row tile holds 52 rows)."""
    import long_context_anti_amd as rmt
    cfg = ri.LLAMA_1B
    T = cfg.n + 500
    gu.say(f"[ragged] {cfg.name} T={T}")
    layers, x, mem0, embed = _inputs(cfg, T)
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg, 2), weights=dw)
    del dw
    model.set_tokens(T)
    x_d, mem0_d = rdev.segment_inputs(cfg, x), rdev.f32_tensor(mem0)
    hd, md = _run(model, x_d, mem0_d, T, cfg)
    hs, ms = _run(model, x_d, mem0_d, T, cfg, "sequential")
    assert np.array_equal(hd, hs) and np.array_equal(md, ms)
    ho, mo = orc.forward_sequential(cfg, layers, x, mem0, embed)
    e_h, e_m = gu.rel_l2(hd, ho), gu.rel_l2(md, mo)
    gu.say(f"  rel L2 hidden {e_h:.3e} mem {e_m:.3e}")
    assert e_h <= 2e-2 and e_m <= 2e-2
    model.close()
