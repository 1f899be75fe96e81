"""The LLaMA-8B-shaped workload (32 layers, d = 4096, 32 query / 8 KV heads
of 128, FFN 14336; cells of 2048 + 128 rows; 64 segments = 131,072 tokens)
on the GPU against the oracle.

At this depth bf16 operands miss the 2e-2 gate on the first segment already
(measured 1.79e-2 hidden / 2.14e-2 memory) and on the two-segment trajectory
(2.65e-2 / 3.17e-2).  The CPU emulation of the same six rounding points
(tests/precision_study.py) reproduces such figures, and shows that the error
is bf16's rounding step itself: with every 16-bit operand in fp16 instead --
same kernels, same MFMA rate, RMT_F16 -- the GPU measures 2.2e-3 / 2.7e-3 on
the first segment and 3.3e-3 / 4.0e-3 over two.  Keeping bf16 operands but
carrying some of them in two bf16 terms (hi + lo; the same module, --split)
clears the two-segment gate with margin only when the gate/up product, the
largest stage, runs twice.  So: bf16 against the gate as strict xfails with
the measured figures, fp16 against the gate as tests that must pass, and for
both diagonal == sequential bit for bit."""
import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]

TOL = 2e-2
BF16, F16 = 1, 2
CFG = ri.LLAMA_8B


@pytest.fixture(scope="module")
def inputs8b():
    gu.say(f"[8b] generating {CFG.name} inputs")
    return gu.inputs(CFG)          # weights, all 64 segments of token ids, M(., -1), embedding


@pytest.fixture(scope="module")
def oracle8b(inputs8b):
    """The oracle's first two segments: hidden rows and memory after each."""
    layers, tok, mem0, embed = inputs8b
    n = CFG.n
    gu.say("[8b] oracle: segments 0 and 1")
    h0, m0 = orc.forward_sequential(CFG, layers, tok[:n], mem0, embed)
    h1, m1 = orc.forward_sequential(CFG, layers, tok[n:2 * n], m0, embed)
    return h0, m0, h1, m1


def _prefix(run, S):
    """GPU diagonal and sequential runs of the first S segments (bitwise
    equal), as (hidden, memory)."""
    import torch
    cfg = run.cfg
    run.model.set_segments(S)
    outs = []
    for fn in (run.model.forward_diagonal, run.model.forward_sequential):
        h = torch.full((S * cfg.n, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((cfg.L, cfg.m, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
        fn(run.tokens[:S * cfg.n], run.mem0_dev, h, m)
        torch.cuda.synchronize()
        outs.append((h.cpu().numpy(), m.cpu().numpy()))
    run.model.set_segments(run.S)
    (hd, md), (hs, ms) = outs
    assert np.array_equal(hd, hs) and np.array_equal(md, ms), "diagonal != sequential"
    return hd, md


@pytest.fixture(scope="module")
def runs8b(inputs8b):
    layers, tok, mem0, embed = inputs8b
    out = {}
    for dt in (BF16, F16):
        gu.say(f"[8b] model with dtype {dt}")
        out[dt] = gu.GpuRun(CFG, S=CFG.S, layers=layers, x=tok, mem0=mem0, embed=embed, dtype=dt)
    yield out
    for r in out.values():
        r.close()


def _errors(run, oracle, S):
    h0, m0, h1, m1 = oracle
    hd, md = _prefix(run, S)
    ho = h0 if S == 1 else np.concatenate([h0, h1])
    mo = m0 if S == 1 else m1
    e = gu.rel_l2(hd, ho), gu.rel_l2(md, mo)
    gu.say(f"  S'={S}: rel L2 hidden {e[0]:.3e} mem {e[1]:.3e}")
    return e


@pytest.mark.timeout(900)
@pytest.mark.parametrize("S", [1, 2])
def test_f16_gate(runs8b, oracle8b, S):
    """fp16 operands: the first segment and the two-segment trajectory."""
    gu.say(f"[8b] fp16 operands, first {S} segment(s) against the gate")
    e_h, e_m = _errors(runs8b[F16], oracle8b, S)
    assert e_h <= TOL and e_m <= TOL


@pytest.mark.xfail(strict=True, reason=(
    "bf16 operand rounding at depth 32: first segment 1.79e-2 (hidden) / 2.14e-2 (memory), "
    "two-segment trajectory 2.65e-2 / 3.17e-2, above the 2e-2 gate; fp16 operands meet it"))
@pytest.mark.timeout(900)
@pytest.mark.parametrize("S", [1, 2])
def test_bf16_gate(runs8b, oracle8b, S):
    gu.say(f"[8b] bf16 operands, first {S} segment(s) against the gate")
    e_h, e_m = _errors(runs8b[BF16], oracle8b, S)
    assert e_h <= TOL and e_m <= TOL


@pytest.mark.timeout(900)
def test_bf16_teacher_forced_segment_1(runs8b, inputs8b):
    """bf16: segment 1 computed by the oracle from the GPU's own M(., 0) is
    within the gate (the per-segment error; the first segment's own error is
    what the trajectory carries)."""
    layers, tok, _, embed = inputs8b
    run = runs8b[BF16]
    n = CFG.n
    _, m_after0 = _prefix(run, 1)
    hd, md = _prefix(run, 2)
    h_o, m_o = orc.forward_sequential(CFG, layers, tok[n:2 * n], m_after0, embed)
    e_h, e_m = gu.rel_l2(hd[n:], h_o), gu.rel_l2(md, m_o)
    gu.say(f"  segment 1 (teacher-forced): rel L2 hidden {e_h:.3e} mem {e_m:.3e}")
    assert e_h <= TOL and e_m <= TOL


def _full_length_teacher_forced(run, inputs8b, label):
    """The full 131,072-token sequence (64 segments, ramps of 31 diagonals at
    each end): diagonal == sequential bitwise, and the last segment checked
    one step at a time from the GPU's own state, within 2e-2."""
    import torch
    layers, tok, _, embed = inputs8b
    gu.say(f"[8b] {label} full length S={CFG.S}")
    hd, md = run.run("diagonal")
    hs, ms = run.run("sequential")
    assert np.array_equal(hd, hs) and np.array_equal(md, ms)
    del hs, ms
    n, s = CFG.n, CFG.S - 1
    run.model.set_segments(s)
    m_in = torch.empty_like(run.mem)
    h_tmp = torch.empty((s * n, CFG.d), dtype=torch.float32, device="cuda")
    run.model.forward_diagonal(run.tokens[:s * n], run.mem0_dev, h_tmp, m_in)
    torch.cuda.synchronize()
    run.model.set_segments(CFG.S)
    del h_tmp
    h_o, m_o = orc.forward_sequential(CFG, layers, tok[s * n:(s + 1) * n], m_in.cpu().numpy(), embed)
    e_h, e_m = gu.rel_l2(hd[s * n:], h_o), gu.rel_l2(md, m_o)
    gu.say(f"  segment {s} (teacher-forced): rel L2 hidden {e_h:.3e} mem {e_m:.3e}")
    assert e_h <= TOL and e_m <= TOL


@pytest.mark.timeout(1200)
def test_bf16_full_length_teacher_forced(runs8b, inputs8b):
    _full_length_teacher_forced(runs8b[BF16], inputs8b, "bf16")


@pytest.mark.timeout(1200)
def test_f16_full_length_teacher_forced(runs8b, inputs8b):
    """fp16 operands, the configuration that meets the gate at this depth,
    over the whole sweep as well."""
    _full_length_teacher_forced(runs8b[F16], inputs8b, "fp16")


@pytest.mark.timeout(900)
def test_f16_batch_of_two_full_length(runs8b):
    """Two 131,072-token sequences through the same diagonals at this shape:
    every full diagonal holds 2 x 32 = 64 cells of 2,176 rows, so it takes two
    launches of 32, the largest the group tables carry.  Each sequence equals
    its own single-sequence run bit for bit (compared on the device: the
    batched hidden states are 4.3 GB)."""
    import torch
    from rmt_inputs import device as rdev
    run = runs8b[F16]
    gu.say("[8b] fp16, batch of two at full length")
    toks = [run.tokens, rdev.segment_inputs(CFG, ri.tokens(CFG, 1))]
    mems = [run.mem0_dev, rdev.f32_tensor(ri.initial_memory(CFG, 1))]
    T = CFG.S * CFG.n
    singles = []
    for b in range(2):
        h = torch.full((T, CFG.d), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((CFG.L, CFG.m, CFG.d), float("nan"), dtype=torch.float32, device="cuda")
        run.model.forward_diagonal(toks[b], mems[b], h, m)
        singles.append((h, m))
    torch.cuda.synchronize()
    try:
        run.model.set_batch(2)
        hb = torch.full((2, T, CFG.d), float("nan"), dtype=torch.float32, device="cuda")
        mb = torch.full((2, CFG.L, CFG.m, CFG.d), float("nan"), dtype=torch.float32, device="cuda")
        run.model.forward_diagonal(torch.stack(toks).contiguous(), torch.stack(mems).contiguous(), hb, mb)
        torch.cuda.synchronize()
        for b, (h, m) in enumerate(singles):
            assert torch.equal(hb[b], h), f"hidden of sequence {b}"
            assert torch.equal(mb[b], m), f"memory of sequence {b}"
        assert bool(torch.isfinite(hb).all())
    finally:
        run.model.set_batch(1)
