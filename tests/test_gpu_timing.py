"""Per-stage launch timing through the C ABI: the split into full and ramp
diagonals (rmt_model_stage_times_groups) partitions the launches, flops and
bytes that rmt_model_stage_times reports, with one launch per stage per
diagonal."""
import ctypes as C

import pytest

import rmt_inputs as ri

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]

PER_DIAGONAL = ("norm1", "qkv", "attn", "oproj", "norm2", "gateup", "down")


def test_stage_times_split_by_groups():
    from long_context_anti_amd import _lib
    cfg = ri.TINY_LLAMA
    gu.say(f"[timing] {cfg.name} L={cfg.L} S={cfg.S}")
    run = gu.GpuRun(cfg)
    run.model.enable_timing(True)
    run.run("diagonal")
    g_full = min(cfg.L, cfg.S)
    full = run.model.stage_times(groups=(g_full, g_full))
    ramp = run.model.stage_times(groups=(1, g_full - 1))
    zero = run.model.stage_times(groups=(0, 0))
    h = _lib.lib()
    assert h.rmt_model_stage_times_groups(run.model._handle, 3, 2, None, None, None, None) == _lib.RMT_EINVAL
    total = run.model.stage_times()
    again = run.model.stage_times()
    run.model.enable_timing(False)
    n_diag = cfg.L + cfg.S - 1
    n_full = n_diag - 2 * (g_full - 1)
    for name in PER_DIAGONAL:
        assert total[name]["launches"] == n_diag, name
        assert full[name]["launches"] == n_full, name
        assert ramp[name]["launches"] == n_diag - n_full, name
        assert total[name]["ms"] > 0
    for name in total:
        for f in ("launches", "flops", "bytes"):
            assert full[name][f] + ramp[name][f] + zero[name][f] == pytest.approx(total[name][f]), (name, f)
        assert again[name]["launches"] == 0      # the unfiltered call cleared the totals
    run.close()
