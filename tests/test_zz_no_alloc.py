"""rmt_forward_diagonal_static -- the forward entry point for callers that
cannot allocate device memory -- through the C ABI, against
rmt_forward_diagonal on the same model.  Both run the same kernels in the same
order on workspaces of the same layout (the static one is the library's own
device array), so the results must agree bit for bit: stronger than the
parity bar (fp32 normwise 1e-4, bf16 relative L2 2e-2) that the bound-workspace
path is held to against the oracle.  Two calls in a row, the second on a
smaller input (fewer segments, or one sequence after two): the array keeps
the first call's contents, which the second must not read."""
import numpy as np
import pytest

import rmt_inputs as ri

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]


def _call(run, fn, T):
    import torch
    cfg = run.cfg
    h = torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((cfg.L, cfg.m, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    fn(run.tokens[:T], run.mem0_dev, h, m)
    torch.cuda.synchronize()
    return h.cpu().numpy(), m.cpu().numpy()


@pytest.mark.parametrize("cfg", [ri.TINY_LINEAR_GELU, ri.TINY_SWIGLU, ri.TINY_LLAMA, ri.TINY_LLAMA_HD128,
                                 ri.TINY_ENCODER, ri.TINY_ENCODER_POSTNORM], ids=lambda c: c.name)
def test_static_workspace_matches_bound_workspace(cfg):
    gu.say(f"[no-alloc] {cfg.name}: static-scratch forward vs bound workspace, S={cfg.S} then smaller")
    run = gu.GpuRun(cfg)
    model = run.model
    for S in (cfg.S, max(1, cfg.S // 2)):
        model.set_segments(S)
        T = S * cfg.n
        # the bound workspace is poisoned, so a static call that touched it could not go unseen
        model.workspace.fill_(255)
        hs, ms = _call(run, model.forward_diagonal_static, T)
        model.workspace.fill_(0)
        hb, mb = _call(run, model.forward_diagonal, T)
        gu.say(f"  S={S}: finite {np.isfinite(hs).all()} equal {np.array_equal(hs, hb) and np.array_equal(ms, mb)}")
        assert np.isfinite(hs).all() and np.isfinite(ms).all()
        assert np.array_equal(hs, hb) and np.array_equal(ms, mb)
    run.close()


def test_static_workspace_batch_then_single():
    """A batch of two sequences, then one sequence with a short last segment."""
    import torch
    cfg = ri.TINY_LLAMA
    gu.say(f"[no-alloc] {cfg.name}: B=2, then B=1 with a short tail")
    run = gu.GpuRun(cfg)
    model = run.model
    toks = torch.stack([run.tokens, run.tokens.flip(0)]).contiguous()
    mem0 = torch.stack([run.mem0_dev, run.mem0_dev * 0.5]).contiguous()
    model.set_batch(2)
    outs = []
    for fn in (model.forward_diagonal_static, model.forward_diagonal):
        h = torch.full((2, cfg.T, cfg.d), float("nan"), device="cuda")
        m = torch.full((2, cfg.L, cfg.m, cfg.d), float("nan"), device="cuda")
        fn(toks, mem0, h, m)
        torch.cuda.synchronize()
        outs.append((h.cpu().numpy(), m.cpu().numpy()))
    assert np.isfinite(outs[0][0]).all()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    model.set_batch(1)
    T = 2 * cfg.n + 37
    model.set_tokens(T)
    hs, ms = _call(run, model.forward_diagonal_static, T)
    hb, mb = _call(run, model.forward_diagonal, T)
    assert np.isfinite(hs).all() and np.array_equal(hs, hb) and np.array_equal(ms, mb)
    run.close()


def test_static_workspace_refuses_large_models():
    """A 1B-width model needs far more than the 64 MiB array: a clear error,
    before any device work."""
    import long_context_anti_amd as rmt
    from long_context_anti_amd import _lib
    cfg = ri.NORM_SWIGLU_1B
    gu.say(f"[no-alloc] {cfg.name}: refused")
    run = gu.GpuRun(cfg, S=1)
    with pytest.raises(rmt.RmtError) as e:
        run.model.forward_diagonal_static(run.tokens, run.mem0_dev, run.hidden, run.mem)
    assert e.value.code == _lib.RMT_EWORKSPACE and "static scratch" in str(e.value)
    run.close()
