"""The grouped GEMM entry point (rmt_grouped_gemm) against CPU products of
the same bf16 operands.  The result is rounded once to bf16, so an element
may differ from the exact product by half a bf16 ulp (2^-9 relative) plus
fp32 accumulation error."""
import numpy as np
import pytest

import rmt_inputs as ri
from rmt_inputs import device as rdev

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]


def _check(c, ref):
    ref = np.asarray(ref, np.float64)
    err = np.abs(np.asarray(c, np.float64) - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref * ref))
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), float(err.max()))


def _bf16_to_np(t):
    import torch
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (bits << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("G,M,N,K", [(1, 128, 256, 64), (3, 240, 320, 200), (5, 20, 64, 32),
                                     (2, 1152, 512, 2048), (4, 300, 768, 136)])
def test_grouped_gemm_small(G, M, N, K):
    import torch
    import long_context_anti_amd as rmt
    gu.say(f"[gemm] G={G} M={M} N={N} K={K}")
    rng = np.random.default_rng(G * 1000 + M)
    Lw = G + 2
    A = ri.round_bf16(rng.standard_normal((G, M, K)).astype(np.float32))
    W = ri.round_bf16((rng.standard_normal((Lw, K, N)) / np.sqrt(K)).astype(np.float32))
    layers = rng.permutation(Lw)[:G]
    A_d = rdev.bf16_tensor(A)
    W_d = rdev.bf16_tensor(W)
    B_d = torch.empty((Lw, N, K), dtype=torch.bfloat16, device="cuda")
    rmt.pack_weight(W_d, B_d)
    C_d = torch.empty((G, M, N), dtype=torch.bfloat16, device="cuda")
    rmt.grouped_gemm(A_d, B_d, layers, C_d)
    torch.cuda.synchronize()
    # packing is a pure relayout
    assert np.array_equal(_bf16_to_np(B_d), np.ascontiguousarray(W.transpose(0, 2, 1)))
    C = _bf16_to_np(C_d)
    for g in range(G):
        _check(C[g], A[g].astype(np.float64) @ W[layers[g]].astype(np.float64))


@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_grouped_gemm_full_size_sampled(G):
    """The isolated 1152 x 2048 x 8192 grouped GEMM at full size; every
    output column of 48 sampled rows per group is checked."""
    import torch
    import long_context_anti_amd as rmt
    gc = ri.GROUPED_GEMM_1B
    gu.say(f"[gemm] {gc.name} G={G}")
    A, Bm = ri.gemm_operands(gc, G=G)
    A_d = rdev.bf16_tensor(A)
    W_d = rdev.bf16_tensor(Bm)
    B_d = torch.empty((G, gc.N, gc.K), dtype=torch.bfloat16, device="cuda")
    rmt.pack_weight(W_d, B_d)
    del W_d
    C_d = torch.empty((G, gc.M, gc.N), dtype=torch.bfloat16, device="cuda")
    rmt.grouped_gemm(A_d, B_d, list(range(G)), C_d)
    torch.cuda.synchronize()
    C = _bf16_to_np(C_d)
    rng = np.random.default_rng(G)
    for g in range(G):
        rows = np.sort(rng.choice(gc.M, 48, replace=False))
        rows[0], rows[-1] = 0, gc.M - 1
        _check(C[g, rows], A[g, rows].astype(np.float64) @ Bm[g].astype(np.float64))
