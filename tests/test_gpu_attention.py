"""rmt_causal_attention against the oracle's causal grouped-query attention on
the same bf16 inputs.  The kernel rounds probabilities and the output to
bf16, so agreement is to bf16 resolution: relative L2 <= 1e-2 and max
abs error <= 2e-2 of the largest output."""
import math

import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc
from rmt_inputs import device as rdev

import gpu_util as gu

pytestmark = [pytest.mark.gpu, gu.needs_gpu]


def _bf16_to_np(t):
    import torch
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (bits << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("G,R,Hq,Hkv,hd", [(1, 1, 4, 1, 64), (3, 100, 8, 2, 64), (2, 240, 4, 1, 128),
                                           (2, 1152, 8, 2, 64), (1, 129, 8, 1, 128), (2, 200, 16, 2, 64),
                                           # one and two query heads per KV head: a workgroup
                                           # then spans 4 or 2 query blocks
                                           (2, 240, 4, 4, 64), (1, 300, 4, 2, 128), (1, 33, 2, 2, 64),
                                           (1, 1, 2, 1, 64)])
def test_attention_matches_oracle(G, R, Hq, Hkv, hd):
    import torch
    import long_context_anti_amd as rmt
    gu.say(f"[attention] G={G} R={R} Hq={Hq} Hkv={Hkv} hd={hd}")
    rng = np.random.default_rng(R * 7 + hd)
    W = (Hq + 2 * Hkv) * hd
    qkv = ri.round_bf16((rng.standard_normal((G, R, W)) * 1.5).astype(np.float32))
    qkv_d = rdev.bf16_tensor(qkv)
    out_d = torch.empty((G, R, Hq * hd), dtype=torch.bfloat16, device="cuda")
    rmt.causal_attention(qkv_d, out_d, Hq, Hkv, hd)
    torch.cuda.synchronize()
    out = _bf16_to_np(out_d)
    for g in range(G):
        q = qkv[g, :, :Hq * hd].reshape(R, Hq, hd)
        k = qkv[g, :, Hq * hd:(Hq + Hkv) * hd].reshape(R, Hkv, hd)
        v = qkv[g, :, (Hq + Hkv) * hd:].reshape(R, Hkv, hd)
        ref = orc.causal_gqa_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
        err = np.linalg.norm(out[g] - ref) / np.linalg.norm(ref)
        assert err <= 1e-2, err
        assert np.max(np.abs(out[g] - ref)) <= 2e-2 * np.max(np.abs(ref))


def test_attention_rejects_bad_arguments():
    import ctypes as C
    from long_context_anti_amd import _lib
    h = _lib.lib()
    p = C.c_void_p(256)
    assert h.rmt_causal_attention(1, 10, 8, 2, 96, p, p, None) == _lib.RMT_EUNSUPPORTED
    assert h.rmt_causal_attention(1, 10, 6, 2, 64, p, p, None) == _lib.RMT_EUNSUPPORTED   # ratio 3
    assert h.rmt_causal_attention(0, 10, 8, 2, 64, p, p, None) == _lib.RMT_EINVAL
    assert h.rmt_causal_attention(1, 10, 8, 2, 64, None, p, None) == _lib.RMT_EINVAL


def _unmasked_reference(q, k, v):
    """The oracle's unmasked multi-head attention, K/V heads repeated for
    grouped queries (query head h reads KV head h // (Hq / Hkv))."""
    rep = q.shape[1] // k.shape[1]
    return orc.full_mha(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1))


@pytest.mark.parametrize("G,R,Hq,Hkv,hd", [(1, 1, 4, 4, 64), (2, 240, 4, 4, 64), (2, 1152, 32, 32, 64),
                                           (2, 160, 4, 4, 128), (1, 100, 8, 2, 64), (3, 97, 8, 8, 128),
                                           (1, 70, 4, 1, 64)])
def test_unmasked_attention_matches_oracle(G, R, Hq, Hkv, hd):
    """Every row attends to all R rows of its cell (the encoder-layer cell)."""
    import torch
    import long_context_anti_amd as rmt
    gu.say(f"[attention unmasked] G={G} R={R} Hq={Hq} Hkv={Hkv} hd={hd}")
    rng = np.random.default_rng(R * 11 + hd + Hkv)
    W = (Hq + 2 * Hkv) * hd
    qkv = ri.round_bf16((rng.standard_normal((G, R, W)) * 1.5).astype(np.float32))
    qkv_d = rdev.bf16_tensor(qkv)
    out_d = torch.empty((G, R, Hq * hd), dtype=torch.bfloat16, device="cuda")
    rmt.attention(qkv_d, out_d, Hq, Hkv, hd, causal=False)
    torch.cuda.synchronize()
    out = _bf16_to_np(out_d)
    for g in range(G):
        q = qkv[g, :, :Hq * hd].reshape(R, Hq, hd).astype(np.float64)
        k = qkv[g, :, Hq * hd:(Hq + Hkv) * hd].reshape(R, Hkv, hd).astype(np.float64)
        v = qkv[g, :, (Hq + Hkv) * hd:].reshape(R, Hkv, hd).astype(np.float64)
        ref = _unmasked_reference(q, k, v)
        err = np.linalg.norm(out[g] - ref) / np.linalg.norm(ref)
        assert err <= 1e-2, err
        assert np.max(np.abs(out[g] - ref)) <= 2e-2 * np.max(np.abs(ref))


def test_causal_flag_of_rmt_attention_matches_causal_entry():
    """rmt_attention(causal=1) and rmt_causal_attention are the same kernel:
    bitwise equal outputs."""
    import torch
    import long_context_anti_amd as rmt
    rng = np.random.default_rng(3)
    G, R, Hq, Hkv, hd = 2, 150, 8, 2, 64
    qkv_d = rdev.bf16_tensor(ri.round_bf16(rng.standard_normal((G, R, (Hq + 2 * Hkv) * hd)).astype(np.float32)))
    a = torch.empty((G, R, Hq * hd), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    rmt.attention(qkv_d, a, Hq, Hkv, hd, causal=True)
    rmt.causal_attention(qkv_d, b, Hq, Hkv, hd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))



@pytest.mark.parametrize("causal", [True, False])
def test_sharp_attention_rescales(causal):
    """Q and K with std 6: scaled scores spread over ~50 units of log2, so the
    running reference maximum is raised (and O, l rescaled) many times per
    row; the result still matches the fp64 oracle on the same bf16 inputs."""
    import torch
    import long_context_anti_amd as rmt
    G, R, Hq, Hkv, hd = 2, 700, 8, 2, 64
    gu.say(f"[attention] sharp scores, causal={causal}")
    rng = np.random.default_rng(77)
    W = (Hq + 2 * Hkv) * hd
    x = rng.standard_normal((G, R, W))
    x[:, :, :(Hq + Hkv) * hd] *= 6.0          # Q and K
    qkv = ri.round_bf16(x.astype(np.float32))
    out_d = torch.empty((G, R, Hq * hd), dtype=torch.bfloat16, device="cuda")
    rmt.attention(rdev.bf16_tensor(qkv), out_d, Hq, Hkv, hd, causal=causal)
    torch.cuda.synchronize()
    out = _bf16_to_np(out_d)
    for g in range(G):
        q = qkv[g, :, :Hq * hd].reshape(R, Hq, hd).astype(np.float64)
        k = qkv[g, :, Hq * hd:(Hq + Hkv) * hd].reshape(R, Hkv, hd).astype(np.float64)
        v = qkv[g, :, (Hq + Hkv) * hd:].reshape(R, Hkv, hd).astype(np.float64)
        if causal:
            ref = orc.causal_gqa_attention(q, k, v)
        else:
            ref = orc.full_mha(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1))
        err = np.linalg.norm(out[g] - ref) / np.linalg.norm(ref)
        gu.say(f"  cell {g}: rel L2 {err:.3e}")
        assert np.isfinite(out[g]).all()
        assert err <= 1e-2, err
