"""The caller-owned workspace (rmt_model_bind, RMT_BUF_WORKSPACE) through
the C ABI on the GPU.  Every forward call must write each workspace byte
before it reads it: with the workspace filled with all-ones bytes (NaN in
fp32 and bf16) before every call, the outputs equal those of a zero-filled
workspace bit for bit, on both paths.  A kernel that read a row it had not
written (past a cell's end, a stale X slot, the memory copy) would carry the
NaN into the outputs."""
import dataclasses

import numpy as np
import pytest

import rmt_inputs as ri

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]


def _run(run, path, fill):
    import torch
    run.model.workspace.fill_(fill)
    run.hidden.fill_(float("nan"))
    run.mem.fill_(float("nan"))
    fn = run.model.forward_diagonal if path == "diagonal" else run.model.forward_sequential
    fn(run.tokens, run.mem0_dev, run.hidden, run.mem)
    torch.cuda.synchronize()
    return run.hidden.cpu().numpy().copy(), run.mem.cpu().numpy().copy()


CASES = [(ri.TINY_LINEAR_GELU, None), (ri.TINY_SWIGLU, None), (ri.TINY_LLAMA, None),
         (ri.TINY_LLAMA_HD128, None), (ri.TINY_ENCODER, None), (ri.TINY_ENCODER_POSTNORM, None),
         (ri.LLAMA_1B, 2), (ri.ENCODER_1B, 2)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg,S", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_poisoned_workspace(cfg, S):
    gu.say(f"[workspace] {cfg.name} S={S or cfg.S}: all-ones workspace vs zeroed")
    run = gu.GpuRun(cfg, S=S)
    for path in ("diagonal", "sequential"):
        h0, m0 = _run(run, path, 0)
        h1, m1 = _run(run, path, 255)
        assert np.isfinite(h1).all() and np.isfinite(m1).all(), path
        assert np.array_equal(h0, h1) and np.array_equal(m0, m1), path
    run.close()


def test_poisoned_workspace_short_tail_and_batch():
    """A short last segment and a batch of three, which change the cell row
    counts and the per-sequence slots."""
    import torch
    import long_context_anti_amd as rmt
    from rmt_inputs import device as rdev
    cfg = ri.TINY_LLAMA
    T = 3 * cfg.n + 41
    gu.say(f"[workspace] {cfg.name} T={T} B=3 poisoned")
    layers = ri.all_weights(cfg, 0)
    embed = ri.embedding(cfg, 0)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=rdev.device_weights(cfg, layers, embed))
    model.set_tokens(T)
    model.set_batch(3)
    tok = torch.stack([rdev.segment_inputs(cfg, ri.tokens(cfg, 7 + b)[:T].copy()) for b in range(3)]).contiguous()
    mem0 = rdev.f32_tensor(np.stack([ri.initial_memory(cfg, 7 + b) for b in range(3)]))
    outs = []
    for fill in (0, 255):
        model.workspace.fill_(fill)
        h = torch.full((3, T, cfg.d), float("nan"), device="cuda")
        m = torch.full((3, cfg.L, cfg.m, cfg.d), float("nan"), device="cuda")
        model.forward_diagonal(tok, mem0, h, m)
        torch.cuda.synchronize()
        outs.append((h.cpu().numpy(), m.cpu().numpy()))
    assert np.isfinite(outs[1][0]).all() and np.isfinite(outs[1][1]).all()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    model.close()


def test_workspace_rebind_and_weights_freed():
    """The mathematical-layout weights may be freed once packed; a fresh
    workspace bound between two calls gives the same result."""
    import torch
    import long_context_anti_amd as rmt
    from rmt_inputs import device as rdev
    cfg = dataclasses.replace(ri.TINY_LLAMA, S=2)
    gu.say(f"[workspace] {cfg.name}: weights freed after packing, workspace re-bound")
    layers, x, mem0, embed = gu.inputs(cfg)
    dw = rdev.device_weights(cfg, layers, embed)
    model = rmt.RMTModel(**rdev.model_kwargs(cfg), weights=dw)
    emb = dw["embed"]
    for k in list(dw):
        if k != "embed":
            dw[k].fill_(float("nan"))     # the packed copy must not read these again
    del dw
    tok, m0 = rdev.segment_inputs(cfg, x), rdev.f32_tensor(mem0)
    h1 = torch.empty((cfg.T, cfg.d), device="cuda")
    mm1 = torch.empty((cfg.L, cfg.m, cfg.d), device="cuda")
    model.forward_diagonal(tok, m0, h1, mm1)
    model.workspace = None
    model._ensure_workspace()
    h2, mm2 = torch.empty_like(h1), torch.empty_like(mm1)
    model.forward_diagonal(tok, m0, h2, mm2)
    torch.cuda.synchronize()
    assert torch.isfinite(h1).all() and torch.equal(h1, h2) and torch.equal(mm1, mm2)
    model.close()
    del emb
