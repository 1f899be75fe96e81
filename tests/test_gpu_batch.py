"""B sequences through the same diagonals (rmt_model_set_batch): each
sequence's hidden states and memory equal a B = 1 run on its own inputs bit
for bit, the batched sequential sweep equals the batched diagonal one, and
every sequence agrees with the oracle (fp32: normwise <= 1e-4; bf16: relative
L2 <= 2e-2 on hidden and on memory).  B = 12 on the three-layer grid puts 36
cells on a full diagonal, more than one launch holds."""
import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc
from rmt_inputs import device as rdev

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]


def _run(model, tok_d, mem0_d, B, cfg, path="diagonal"):
    import torch
    hidden = torch.full((B, cfg.S * cfg.n, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    mem = torch.full((B, cfg.L, cfg.m, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    fn = model.forward_diagonal if path == "diagonal" else model.forward_sequential
    fn(tok_d, mem0_d, hidden, mem)
    torch.cuda.synchronize()
    return hidden.cpu().numpy(), mem.cpu().numpy()


@pytest.mark.parametrize("cfg,B", [(ri.TINY_LINEAR_GELU, 2), (ri.TINY_SWIGLU, 2), (ri.TINY_LLAMA, 3),
                                   (ri.TINY_LLAMA, 12), (ri.TINY_ENCODER, 3), (ri.TINY_ENCODER_POSTNORM, 2)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_batch_matches_single_sequences(cfg, B):
    import torch
    import long_context_anti_amd as rmt
    gu.say(f"[batch] {cfg.name} B={B}")
    layers = ri.all_weights(cfg, 0, workers=8)
    embed = ri.embedding(cfg, 0) if cfg.cell == ri.CELL_LLAMA else None
    # sequence b: inputs and initial memory from seed 100 + b
    xs = [ri.tokens(cfg, 100 + b) if cfg.cell == ri.CELL_LLAMA else ri.input_embeddings(cfg, 100 + b)
          for b in range(B)]
    mems = [ri.initial_memory(cfg, 100 + b) for b in range(B)]
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=dw)
    # one sequence at a time
    singles = []
    for b in range(B):
        h, m = _run(model, rdev.segment_inputs(cfg, xs[b]), rdev.f32_tensor(mems[b]), 1, cfg)
        singles.append((h[0], m[0]))
    # all B together
    model.set_batch(B)
    tok_d = torch.stack([rdev.segment_inputs(cfg, x) for x in xs]).contiguous()
    mem0_d = rdev.f32_tensor(np.stack(mems))
    hb, mb = _run(model, tok_d, mem0_d, B, cfg)
    hs, ms = _run(model, tok_d, mem0_d, B, cfg, "sequential")
    assert np.array_equal(hb, hs) and np.array_equal(mb, ms)
    for b in range(B):
        assert np.array_equal(hb[b], singles[b][0]), f"hidden of sequence {b}"
        assert np.array_equal(mb[b], singles[b][1]), f"memory of sequence {b}"
        if b < 3:
            ho, mo = orc.forward_sequential(cfg, layers, xs[b], mems[b], embed)
            if cfg.dtype == ri.F32:
                assert gu.normwise(hb[b], ho) <= 1e-4 and gu.normwise(mb[b], mo) <= 1e-4
            else:
                assert gu.rel_l2(hb[b], ho) <= 2e-2 and gu.rel_l2(mb[b], mo) <= 2e-2
    # back to one sequence
    model.set_batch(1)
    h1, m1 = _run(model, rdev.segment_inputs(cfg, xs[0]), rdev.f32_tensor(mems[0]), 1, cfg)
    assert np.array_equal(h1[0], singles[0][0]) and np.array_equal(m1[0], singles[0][1])
    model.close()


def test_set_batch_rejects_bad_sizes():
    from long_context_anti_amd import _lib
    cfg = ri.TINY_LLAMA
    run = gu.GpuRun(cfg, S=1)
    assert _lib.lib().rmt_model_set_batch(run.model._handle, 0) == _lib.RMT_EINVAL
    assert _lib.lib().rmt_model_set_batch(run.model._handle, -3) == _lib.RMT_EINVAL
    run.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", [2, 3])
def test_full_width_batch_fills_the_largest_launch(B):
    """The LLaMA-1B width over 16 segments: with B = 2 every full diagonal
    holds 2 x 16 = 32 cells, the most one launch's group table carries; with
    B = 3 its 48 cells take a launch of 32 and one of 16.  Each sequence
    equals its own single-sequence run bit for bit (the oracle's agreement
    at this width is covered by the prefix and teacher-forced tests)."""
    import torch
    import long_context_anti_amd as rmt
    cfg = ri.LLAMA_1B.with_segments(16)
    gu.say(f"[batch] {cfg.name} S=16 B={B} at full width")
    layers = ri.all_weights(cfg, 0, workers=8)
    embed = ri.embedding(cfg, 0)
    xs = [ri.tokens(cfg, 200 + b) for b in range(B)]
    mems = [ri.initial_memory(cfg, 200 + b) for b in range(B)]
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=dw)
    singles = [_run(model, rdev.segment_inputs(cfg, xs[b]), rdev.f32_tensor(mems[b]), 1, cfg)
               for b in range(B)]
    model.set_batch(B)
    tok_d = torch.stack([rdev.segment_inputs(cfg, x) for x in xs]).contiguous()
    hb, mb = _run(model, tok_d, rdev.f32_tensor(np.stack(mems)), B, cfg)
    for b in range(B):
        assert np.array_equal(hb[b], singles[b][0][0]), f"hidden of sequence {b}"
        assert np.array_equal(mb[b], singles[b][1][0]), f"memory of sequence {b}"
        assert np.isfinite(hb[b]).all()
    model.close()


@pytest.mark.timeout(900)
def test_batch_outputs_past_int32_offsets():
    """The LLaMA-1B-shaped workload at full length (128 segments, 131,072
    tokens) with B = 9: the hidden output holds 9 x 131,072 x 2,048 = 2.42e9
    elements, and sequence 8 starts at element 2^31, past INT32_MAX.  Its
    hidden states and memory, and those of sequence 0, equal their own B = 1
    runs bit for bit, and no element of the batched outputs is left unwritten
    (compared on the device: the batched hidden states alone are 9.7 GB)."""
    import torch
    import long_context_anti_amd as rmt
    cfg, B = ri.LLAMA_1B, 9
    T = cfg.S * cfg.n
    assert (B - 1) * T * cfg.d > 2**31 - 1     # INT32_MAX
    gu.say(f"[batch] {cfg.name} full length B={B}")
    layers = ri.all_weights(cfg, 0, workers=8)
    embed = ri.embedding(cfg, 0)
    xs = [ri.tokens(cfg, 300 + b) for b in range(B)]
    mems = [ri.initial_memory(cfg, 300 + b) for b in range(B)]
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=dw)
    del dw, layers
    tok_d = torch.stack([rdev.segment_inputs(cfg, x) for x in xs]).contiguous()
    mem0_d = rdev.f32_tensor(np.stack(mems))
    singles = {}
    for b in (0, B - 1):
        h = torch.full((1, T, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((1, cfg.L, cfg.m, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        model.forward_diagonal(tok_d[b:b + 1].contiguous(), mem0_d[b:b + 1].contiguous(), h, m)
        torch.cuda.synchronize()
        singles[b] = (h, m)
    model.set_batch(B)
    hb = torch.full((B, T, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    mb = torch.full((B, cfg.L, cfg.m, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    model.forward_diagonal(tok_d, mem0_d, hb, mb)
    torch.cuda.synchronize()
    gu.say("  batched sweep done")
    for b, (h, m) in singles.items():
        assert torch.equal(hb[b], h[0]), f"hidden of sequence {b}"
        assert torch.equal(mb[b], m[0]), f"memory of sequence {b}"
    assert bool(torch.isfinite(hb).all()) and bool(torch.isfinite(mb).all())
    model.close()
