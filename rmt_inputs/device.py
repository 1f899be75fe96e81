"""Move seeded inputs onto the GPU as torch tensors in the layout the C ABI
takes (stacked over layers, mathematical orientation).  Byte marshalling
only: bf16 values are handed over as their exact bit patterns."""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import BF16, CELL_LINEAR_GELU, CELL_LLAMA, RMTConfig, bf16_bits


def bf16_tensor(arr: np.ndarray, device="cuda"):
    """bf16-representable float32 array -> torch.bfloat16 tensor, bit-exact."""
    import torch
    bits = bf16_bits(arr)
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def f32_tensor(arr: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


# generator key -> rmt_weights field (the encoder's LayerNorm parameters)
_ABI_NAME = {"ln1_g": "g1", "ln1_b": "beta1", "ln2_g": "g2", "ln2_b": "beta2"}
# fields the C ABI takes in fp32 whatever the model's dtype: gains, shifts, biases
_FP32_FIELDS = {"g1", "g2", "b", "beta1", "beta2", "bqkv", "bo", "b1", "b2"}


def device_weights(cfg: RMTConfig, layers: List[Dict[str, np.ndarray]],
                   embed: Optional[np.ndarray] = None, device="cuda") -> Dict[str, object]:
    """Stack per-layer weights and upload them.  Matrices go up as bf16 for
    bf16 workloads and fp32 otherwise; gains and biases are fp32."""
    out: Dict[str, object] = {}
    bf = cfg.dtype == BF16
    for key in layers[0]:
        stacked = np.stack([w[key] for w in layers])
        name = _ABI_NAME.get(key, key)
        if name in _FP32_FIELDS or not bf:
            out[name] = f32_tensor(stacked, device)
        else:
            out[name] = bf16_tensor(stacked, device)
        del stacked
    if cfg.cell == CELL_LLAMA:
        assert embed is not None
        out["embed"] = bf16_tensor(embed, device)
    return out


def model_kwargs(cfg: RMTConfig, S: Optional[int] = None) -> Dict[str, object]:
    """Keyword arguments of long_context_anti_amd.RMTModel for a workload."""
    return dict(cell=cfg.cell, dtype=0 if cfg.dtype != BF16 else 1, L=cfg.L,
                S=cfg.S if S is None else S, n=cfg.n, m=cfg.m, d=cfg.d, n_heads=cfg.Hq,
                n_kv_heads=cfg.Hkv, head_dim=cfg.hd, ffn=cfg.F, vocab=cfg.V, eps=cfg.eps,
                rope_theta=cfg.theta, post_norm=cfg.post_norm)


def segment_inputs(cfg: RMTConfig, inputs: np.ndarray, device="cuda"):
    """Token ids (int32) or input rows (fp32 / bf16) as a device tensor."""
    import torch
    if cfg.cell == CELL_LLAMA:
        return torch.from_numpy(np.ascontiguousarray(inputs, np.int32)).to(device)
    if cfg.cell == CELL_LINEAR_GELU or cfg.dtype != BF16:
        return f32_tensor(inputs, device)
    return bf16_tensor(inputs, device)
