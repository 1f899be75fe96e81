"""fp16 operands (RMT_F16) through the C ABI: the grouped GEMM on its own,
and the LLaMA-shaped cell, whose every 16-bit operand (weights, normalised
rows, Q/K/V, probabilities, attention output, SwiGLU output) is then IEEE
half instead of bf16.  Same kernels, same MFMA rate; fp16 rounds with an
eighth of bf16's step, so against the same fp32 oracle the error must fall
well below the bf16 path's on the same inputs (which also shows the operands
really are fp16).  Diagonal == sequential bit for bit, as for bf16."""
import dataclasses

import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc
from rmt_inputs import device as rdev

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]

BF16, F16 = 1, 2


def _f16_np(t):
    import torch
    return t.float().cpu().numpy()


def _check(c, ref):
    """fp16 result: half an fp16 ulp (2^-11 relative) of rounding plus fp32
    accumulation error."""
    ref = np.asarray(ref, np.float64)
    err = np.abs(np.asarray(c, np.float64) - ref)
    bound = 2.0 ** -10 * np.abs(ref) + 1e-4 * np.sqrt(np.mean(ref * ref))
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), float(err.max()))


@pytest.mark.parametrize("G,M,N,K", [(1, 128, 256, 64), (3, 240, 320, 200), (2, 1152, 512, 2048),
                                     (4, 300, 768, 136)])
def test_grouped_gemm_f16(G, M, N, K):
    import torch
    import long_context_anti_amd as rmt
    gu.say(f"[f16 gemm] G={G} M={M} N={N} K={K}")
    rng = np.random.default_rng(G * 7 + M)
    Lw = G + 1
    A = rng.standard_normal((G, M, K)).astype(np.float16)
    W = (rng.standard_normal((Lw, K, N)) / np.sqrt(K)).astype(np.float16)
    layers = rng.permutation(Lw)[:G]
    A_d = torch.from_numpy(A).cuda()
    B_d = torch.from_numpy(np.ascontiguousarray(W.transpose(0, 2, 1))).cuda()   # [Lw][N][K]
    C_d = torch.empty((G, M, N), dtype=torch.float16, device="cuda")
    rmt.grouped_gemm(A_d, B_d, layers, C_d)
    torch.cuda.synchronize()
    C = _f16_np(C_d)
    for g in range(G):
        _check(C[g], A[g].astype(np.float64) @ W[layers[g]].astype(np.float64))


def test_grouped_gemm_f16_full_size_sampled():
    """1152 x 2048 x 8192 at G = 16 with the workload's operands in fp16."""
    import torch
    import long_context_anti_amd as rmt
    gc = ri.GROUPED_GEMM_1B
    G = gc.G_max
    gu.say(f"[f16 gemm] {gc.name} G={G}")
    A, Bm = ri.gemm_operands(gc, G=G)
    A16, B16 = A.astype(np.float16), Bm.astype(np.float16)
    A_d = torch.from_numpy(A16).cuda()
    B_d = torch.from_numpy(np.ascontiguousarray(B16.transpose(0, 2, 1))).cuda()
    C_d = torch.empty((G, gc.M, gc.N), dtype=torch.float16, device="cuda")
    rmt.grouped_gemm(A_d, B_d, list(range(G)), C_d)
    torch.cuda.synchronize()
    C = _f16_np(C_d)
    rng = np.random.default_rng(5)
    for g in range(G):
        rows = np.sort(rng.choice(gc.M, 24, replace=False))
        _check(C[g, rows], A16[g, rows].astype(np.float64) @ B16[g].astype(np.float64))


TINY_GQA2 = dataclasses.replace(ri.TINY_LLAMA, name="tiny_llama_gqa2", wid=32, Hq=4, Hkv=2)


def _both(cfg, S=None):
    """GPU runs of the same inputs with bf16 and with fp16 operands, the
    oracle, and the per-dtype errors (hidden, mem)."""
    out = {}
    oracle = None
    for dt in (BF16, F16):
        run = gu.GpuRun(cfg, S=S, dtype=dt)
        hd, md = run.run("diagonal")
        hs, ms = run.run("sequential")
        assert np.array_equal(hd, hs) and np.array_equal(md, ms), f"dtype {dt}: diagonal != sequential"
        if oracle is None:
            oracle = orc.forward_sequential(cfg, run.layers, run.x, run.mem0, run.embed)
        out[dt] = (gu.rel_l2(hd, oracle[0]), gu.rel_l2(md, oracle[1]))
        run.close()
    gu.say(f"  bf16 hidden {out[BF16][0]:.3e} mem {out[BF16][1]:.3e} | "
           f"fp16 hidden {out[F16][0]:.3e} mem {out[F16][1]:.3e}")
    return out


TINY_MHA_HD128 = dataclasses.replace(ri.TINY_LLAMA_HD128, name="tiny_llama_mha_hd128", wid=33, Hkv=4)


@pytest.mark.parametrize("cfg", [ri.TINY_LLAMA, ri.TINY_LLAMA_HD128, TINY_GQA2, TINY_MHA_HD128],
                         ids=lambda c: c.name)
def test_tiny_llama_f16(cfg):
    gu.say(f"[f16] {cfg.name}")
    e = _both(cfg)
    for i in range(2):
        assert e[F16][i] <= 2e-2
        assert e[F16][i] < e[BF16][i] / 3


@pytest.mark.timeout(600)
def test_llama1b_prefix_f16():
    cfg = ri.LLAMA_1B
    gu.say(f"[f16] {cfg.name} prefix S=2")
    e = _both(cfg, S=2)
    for i in range(2):
        assert e[F16][i] <= 2e-2
        assert e[F16][i] < e[BF16][i] / 3


def test_f16_sharp_attention():
    """Weights three times the tiny grid's spread: scaled scores of tens of
    log2 units, rows that raise their reference maximum after the first
    block, and probabilities up to 2^8 in fp16."""
    cfg = dataclasses.replace(ri.TINY_LLAMA, name="tiny_llama_sharp_f16", L=1, S=1, w_std=0.15)
    gu.say(f"[f16] {cfg.name}")
    run = gu.GpuRun(cfg, dtype=F16)
    hd, md = run.run("diagonal")
    ho, mo = orc.forward_sequential(cfg, run.layers, run.x, run.mem0, run.embed)
    assert np.isfinite(hd).all() and np.isfinite(md).all()
    assert gu.rel_l2(hd, ho) <= 5e-3 and gu.rel_l2(md, mo) <= 5e-3
    run.close()


def test_f16_poisoned_workspace():
    cfg = ri.TINY_LLAMA
    gu.say(f"[f16] {cfg.name} poisoned workspace")
    run = gu.GpuRun(cfg, dtype=F16)
    run.model.workspace.fill_(0)
    h0, m0 = run.run("diagonal")
    run.model.workspace.fill_(255)
    h1, m1 = run.run("diagonal")
    assert np.array_equal(h0, h1) and np.array_equal(m0, m1)
    run.close()
