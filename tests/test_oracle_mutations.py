"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  A pin set that passes a mutated oracle would not be pinning
that part of it."""
import dataclasses

import numpy as np
import pytest

import rmt_inputs as ri
from oracle import rmt_oracle as orc

import pins


def _fails(fn, *a, **k):
    try:
        fn(*a, **k)
    except AssertionError:
        return True
    return False


def _forward_with_split(split_first_m_to_memory=False, memory_after_x=False):
    """A sequential sweep with the write-back split or the input order changed."""
    def fwd(cfg, weights, inputs, mem0, embed=None, dtype=np.float32):
        S = inputs.shape[0] // cfg.n
        L, n, m = cfg.L, cfg.n, cfg.m
        ws = [{k: np.asarray(v, dtype) for k, v in w.items()} for w in weights]
        M = [np.array(mem0[l], dtype) for l in range(L)]
        hidden = []
        for s in range(S):
            x = orc.segment_input(cfg, inputs, s, embed, dtype)
            for l in range(L):
                A = np.concatenate([x, M[l]] if memory_after_x else [M[l], x])
                Y = orc.cell(cfg, ws[l], A)
                if split_first_m_to_memory:
                    M[l], x = Y[:m], Y[m:]
                else:
                    x, M[l] = Y[:n], Y[n:]
            hidden.append(x)
        return np.concatenate(hidden), np.stack(M)
    return fwd


def test_mutation_schedule_descending_layers():
    bad = lambda L, S: [list(reversed(dg)) for dg in orc.schedule(L, S)]  # noqa: E731
    assert _fails(pins.pin_schedule_golden, schedule=bad)
    assert _fails(pins.pin_schedule_invariants, 4, 6, schedule=bad)


def test_mutation_schedule_missing_last_diagonal():
    bad = lambda L, S: orc.schedule(L, S)[:-1]  # noqa: E731
    assert _fails(pins.pin_schedule_invariants, 4, 6, schedule=bad)


def test_mutation_writeback_split():
    bad = _forward_with_split(split_first_m_to_memory=True)
    assert _fails(pins.pin_linear_gelu_bruteforce, forward=bad)
    assert _fails(pins.pin_shift_register, ri.TINY_SWIGLU, forward=bad)


def test_mutation_memory_after_segment():
    bad = _forward_with_split(memory_after_x=True)
    assert _fails(pins.pin_linear_gelu_bruteforce, forward=bad)
    assert _fails(pins.pin_shift_register, ri.TINY_LLAMA, forward=bad)


def test_mutation_no_bias(monkeypatch):
    monkeypatch.setattr(orc, "cell_linear_gelu", lambda A, w: orc.gelu_erf(A @ w["w"]))
    assert _fails(pins.pin_linear_gelu_bruteforce)


def test_mutation_transposed_weight(monkeypatch):
    monkeypatch.setattr(orc, "cell_linear_gelu", lambda A, w: orc.gelu_erf(A @ w["w"].T + w["b"]))
    assert _fails(pins.pin_linear_gelu_bruteforce)


def test_mutation_gelu_tanh(monkeypatch):
    def gelu_tanh(z):
        return 0.5 * z * (1 + np.tanh(np.sqrt(2 / np.pi) * (z + 0.044715 * z ** 3)))
    assert _fails(pins.pin_gelu, gelu=gelu_tanh)


def test_mutation_rope_sign():
    def rope_bad(x, pos, theta):
        return orc.rope_rotate_half(x, -pos, theta)
    assert _fails(pins.pin_rope, rope=rope_bad)


def test_mutation_rope_interleaved_pairs():
    def rope_bad(x, pos, theta):
        hd = x.shape[-1]
        perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
        inv = np.argsort(perm)
        return orc.rope_rotate_half(x[..., perm], pos, theta)[..., inv]
    assert _fails(pins.pin_rope, rope=rope_bad)


def test_rope_position_origin_is_invisible(monkeypatch):
    """Not a mistake: attention sees only relative positions, so shifting every
    position by the same amount leaves the block's output unchanged."""
    real = orc.rope_rotate_half
    monkeypatch.setattr(orc, "rope_rotate_half", lambda x, pos, theta: real(x, pos + 7, theta))
    pins.pin_single_segment_against_torch(ri.TINY_LLAMA, tol=1e-10)


def test_mutation_rope_on_queries_only(monkeypatch):
    real = orc.rope_rotate_half
    calls = []

    def rope_q_only(x, pos, theta):
        calls.append(1)
        return real(x, pos, theta) if len(calls) % 2 == 1 else x
    monkeypatch.setattr(orc, "rope_rotate_half", rope_q_only)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_LLAMA)


def test_mutation_attention_not_causal(monkeypatch):
    def attn(q, k, v):
        R, Hq, hd = q.shape
        rep = Hq // k.shape[1]
        out = np.empty_like(q)
        for h in range(Hq):
            s = q[:, h] @ k[:, h // rep].T / np.sqrt(hd)
            p = np.exp(s - s.max(1, keepdims=True))
            out[:, h] = (p / p.sum(1, keepdims=True)) @ v[:, h // rep]
        return out.reshape(R, -1)
    assert _fails(pins.pin_attention, attn=attn)
    monkeypatch.setattr(orc, "causal_gqa_attention", attn)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_LLAMA)


def test_mutation_gqa_head_map(monkeypatch):
    real = orc.causal_gqa_attention

    def attn(q, k, v):
        # head h reads KV head h % Hkv instead of h // (Hq / Hkv)
        R, Hq, hd = q.shape
        Hkv = k.shape[1]
        idx = np.array([h % Hkv for h in range(Hq)])
        rep = Hq // Hkv
        order = np.argsort([i * rep + h // Hkv for h, i in enumerate(idx)], kind="stable")
        out = real(q[:, order], k, v).reshape(R, Hq, hd)
        return out[:, np.argsort(order)].reshape(R, -1)
    assert _fails(pins.pin_attention, attn=attn)
    cfg = dataclasses.replace(ri.TINY_LLAMA, Hq=4, Hkv=2)
    monkeypatch.setattr(orc, "causal_gqa_attention", attn)
    assert _fails(pins.pin_single_segment_against_torch, cfg)


def test_mutation_rmsnorm_no_eps():
    assert _fails(pins.pin_rms_norm, rms_norm=lambda x, g, eps: orc.rms_norm(x, g, 0.0) * 1.0
                  if eps == 0 else orc.rms_norm(x, g, 1e-2))


def test_mutation_swapped_gate_up(monkeypatch):
    monkeypatch.setattr(orc, "swiglu", lambda z, wg, wu, wd: (orc.silu(z @ wu) * (z @ wg)) @ wd)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_SWIGLU)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_LLAMA)


def _swap_gains(w):
    w = dict(w)
    w["g1"], w["g2"] = w["g2"], w["g1"]
    return w


def test_mutation_llama_norm_gains_exchanged(monkeypatch):
    """The two RMSNorms of a LLaMA cell read each other's gain (the tiny grids
    draw the gains around 1, so the two differ)."""
    real = orc.cell_llama
    monkeypatch.setattr(orc, "cell_llama", lambda A, w, *a: real(A, _swap_gains(w), *a))
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_LLAMA)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_LLAMA_HD128)


@pytest.mark.parametrize("cfg", [ri.TINY_LLAMA, ri.TINY_SWIGLU], ids=lambda c: c.name)
def test_mutation_rmsnorm_gain_dropped(monkeypatch, cfg):
    real = orc.rms_norm
    monkeypatch.setattr(orc, "rms_norm", lambda x, g, eps: real(x, np.ones_like(g), eps))
    assert _fails(pins.pin_single_segment_against_torch, cfg)


def test_mutation_dropped_residual(monkeypatch):
    monkeypatch.setattr(orc, "cell_norm_swiglu",
                        lambda A, w, eps: orc.swiglu(orc.rms_norm(A, w["g2"], eps), w["wg"], w["wu"], w["wd"]))
    assert _fails(pins.pin_shift_register, ri.TINY_SWIGLU)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_SWIGLU)


def test_mutation_attention_scale(monkeypatch):
    real = orc.causal_gqa_attention
    monkeypatch.setattr(orc, "causal_gqa_attention", lambda q, k, v: real(q * 2.0, k, v))
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_LLAMA)


def _forward_short_tail_mistake(keep_memory_on_tail=False, pad_tail=False):
    """A sweep that mishandles a short last segment: either the short cells
    leave the memory as it was, or the short segment is padded with zero rows
    up to n before the cells run."""
    def fwd(cfg, weights, inputs, mem0, embed=None, dtype=np.float32):
        T = inputs.shape[0]
        S = -(-T // cfg.n)
        L, n = cfg.L, cfg.n
        ws = [{k: np.asarray(v, dtype) for k, v in w.items()} for w in weights]
        M = [np.array(mem0[l], dtype) for l in range(L)]
        hidden = []
        for s in range(S):
            x = orc.segment_input(cfg, inputs, s, embed, dtype)
            ns = x.shape[0]
            if pad_tail and ns < n:
                x = np.concatenate([x, np.zeros((n - ns, x.shape[1]), dtype)])
            for l in range(L):
                Y = orc.cell(cfg, ws[l], np.concatenate([M[l], x]))
                rows = x.shape[0]
                x = Y[:rows]
                if not (keep_memory_on_tail and ns < n):
                    M[l] = Y[rows:]
            hidden.append(x[:ns])
        return np.concatenate(hidden), np.stack(M)
    return fwd


@pytest.mark.parametrize("T", [5 * 16 + 2, 5 * 16 + 7])
def test_mutation_short_tail_keeps_memory(T):
    bad = _forward_short_tail_mistake(keep_memory_on_tail=True)
    assert _fails(pins.pin_linear_gelu_bruteforce_ragged, T,
                  forward=lambda *a, **k: bad(*a, **{**k, "dtype": np.float64}))


@pytest.mark.parametrize("T", [5 * 16 + 2, 5 * 16 + 7])
def test_mutation_short_tail_zero_padded(T):
    bad = _forward_short_tail_mistake(pad_tail=True)
    assert _fails(pins.pin_linear_gelu_bruteforce_ragged, T,
                  forward=lambda *a, **k: bad(*a, **{**k, "dtype": np.float64}))


# ---------------------------------------------------------------------------
# The encoder-layer cell
# ---------------------------------------------------------------------------

def _post_norm_encoder(A, w, H, hd, eps, post_norm=False):
    """The layer with norm_first=False (whatever the workload asks): the norms
    follow the residual adds."""
    R = A.shape[0]
    qkv = A @ w["wqkv"] + w["bqkv"]
    nq = H * hd
    q, k, v = (qkv[:, i * nq:(i + 1) * nq].reshape(R, H, hd) for i in range(3))
    Hs = orc.layer_norm(A + (orc.full_mha(q, k, v) @ w["wo"] + w["bo"]), w["ln1_g"], w["ln1_b"], eps)
    return orc.layer_norm(Hs + (orc.relu(Hs @ w["w1"] + w["b1"]) @ w["w2"] + w["b2"]),
                          w["ln2_g"], w["ln2_b"], eps)


def test_mutation_encoder_post_norm(monkeypatch):
    monkeypatch.setattr(orc, "cell_encoder", _post_norm_encoder)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


def test_mutation_layer_norm_without_shift(monkeypatch):
    plain = orc.layer_norm
    monkeypatch.setattr(orc, "layer_norm", lambda x, g, b, eps: plain(x, g, np.zeros_like(b), eps))
    assert _fails(pins.pin_layer_norm, layer_norm=orc.layer_norm)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


def test_mutation_layer_norm_not_centred(monkeypatch):
    def rms_like(x, g, b, eps):
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g + b
    assert _fails(pins.pin_layer_norm, layer_norm=rms_like)
    monkeypatch.setattr(orc, "layer_norm", rms_like)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


def test_mutation_layer_norm_unbiased_variance():
    def unbiased(x, g, b, eps):
        xc = x - np.mean(x, axis=-1, keepdims=True)
        return xc / np.sqrt(np.var(x, axis=-1, ddof=1, keepdims=True) + eps) * g + b
    assert _fails(pins.pin_layer_norm, layer_norm=unbiased)


def test_mutation_encoder_attention_causal(monkeypatch):
    causal = lambda q, k, v: orc.causal_gqa_attention(q, k, v)  # noqa: E731
    assert _fails(pins.pin_full_attention, attn=causal)
    monkeypatch.setattr(orc, "full_mha", causal)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


@pytest.mark.parametrize("bias", ["bqkv", "bo", "b1", "b2"])
def test_mutation_encoder_dropped_bias(monkeypatch, bias):
    plain = orc.cell_encoder

    def dropped(A, w, H, hd, eps, post_norm=False):
        w = dict(w)
        w[bias] = np.zeros_like(w[bias])
        return plain(A, w, H, hd, eps, post_norm)
    monkeypatch.setattr(orc, "cell_encoder", dropped)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


def test_mutation_encoder_gelu_for_relu(monkeypatch):
    monkeypatch.setattr(orc, "relu", orc.gelu_erf)
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


def test_mutation_encoder_swapped_k_v(monkeypatch):
    plain = orc.full_mha
    monkeypatch.setattr(orc, "full_mha", lambda q, k, v: plain(q, v, k))
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER)


def test_mutation_encoder_pre_norm_for_post_norm(monkeypatch):
    """The post-norm workload computed in the pre-norm order fails its torch pin."""
    plain = orc.cell_encoder
    monkeypatch.setattr(orc, "cell_encoder",
                        lambda A, w, H, hd, eps, post_norm=False: plain(A, w, H, hd, eps, False))
    assert _fails(pins.pin_single_segment_against_torch, ri.TINY_ENCODER_POSTNORM)
