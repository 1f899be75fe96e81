"""ctypes declarations for librmt.so (the C ABI in include/rmt.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation on the product path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librmt.so")

RMT_OK = 0
RMT_EINVAL = -1
RMT_EUNSUPPORTED = -2
RMT_EHIP = -3
RMT_ENOMEM = -4
RMT_EWORKSPACE = -5

# bytes of the static workspace behind rmt_forward_diagonal_static
STATIC_SCRATCH_BYTES = 64 << 20

RMT_BUF_WEIGHTS = 0
RMT_BUF_WORKSPACE = 1

RMT_CELL_LINEAR_GELU = 0
RMT_CELL_NORM_SWIGLU = 1
RMT_CELL_LLAMA = 2
RMT_CELL_ENCODER = 3
RMT_F32 = 0
RMT_BF16 = 1
RMT_F16 = 2

STAGES = ["gather", "norm1", "qkv", "attn", "oproj", "norm2", "gateup", "down", "linear"]
RMT_NUM_STAGES = len(STAGES)


class RmtConfig(C.Structure):
    _fields_ = [
        ("cell", C.c_int32), ("dtype", C.c_int32), ("L", C.c_int32), ("S", C.c_int32),
        ("n", C.c_int32), ("m", C.c_int32), ("d", C.c_int32), ("n_heads", C.c_int32),
        ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
        ("vocab", C.c_int32), ("eps", C.c_float), ("rope_theta", C.c_float),
        ("post_norm", C.c_int32),
    ]


class RmtWeights(C.Structure):
    _fields_ = [
        ("weight_dtype", C.c_int32), ("w", C.c_void_p), ("b", C.c_void_p), ("g1", C.c_void_p),
        ("wqkv", C.c_void_p), ("wo", C.c_void_p), ("g2", C.c_void_p), ("wg", C.c_void_p),
        ("wu", C.c_void_p), ("wd", C.c_void_p), ("embed", C.c_void_p),
        ("beta1", C.c_void_p), ("bqkv", C.c_void_p), ("bo", C.c_void_p), ("beta2", C.c_void_p),
        ("w1", C.c_void_p), ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p),
    ]


class RmtOutput(C.Structure):
    _fields_ = [("hidden", C.c_void_p), ("mem", C.c_void_p)]


# name -> (restype, argtypes); every symbol include/rmt.h declares
SIGNATURES = {
    "rmt_diag_schedule": (C.c_int32, [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "rmt_model_create": (C.c_int32, [C.POINTER(RmtConfig), C.POINTER(RmtWeights), C.c_void_p,
                                     C.POINTER(C.c_void_p)]),
    "rmt_workspace_bytes": (C.c_int32, [C.c_void_p, C.c_int32, C.POINTER(C.c_size_t)]),
    "rmt_model_bind": (C.c_int32, [C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t]),
    "rmt_model_set_segments": (C.c_int32, [C.c_void_p, C.c_int32]),
    "rmt_model_set_stream": (C.c_int32, [C.c_void_p, C.c_void_p]),
    "rmt_model_set_batch": (C.c_int32, [C.c_void_p, C.c_int32]),
    "rmt_model_set_tokens": (C.c_int32, [C.c_void_p, C.c_int64]),
    "rmt_model_device_bytes": (C.c_int32, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "rmt_forward_diagonal": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(RmtOutput)]),
    "rmt_forward_sequential": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(RmtOutput)]),
    "rmt_forward_diagonal_static": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p,
                                                C.POINTER(RmtOutput)]),
    "rmt_model_check": (C.c_int32, [C.c_void_p, C.POINTER(C.c_int32)]),
    "rmt_model_enable_timing": (C.c_int32, [C.c_void_p, C.c_int32]),
    "rmt_model_stage_times": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "rmt_model_stage_times_groups": (C.c_int32, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                                 C.c_void_p, C.c_void_p]),
    "rmt_model_destroy": (C.c_int32, [C.c_void_p]),
    "rmt_pack_weight": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_int32,
                                    C.c_void_p, C.c_void_p]),
    "rmt_grouped_gemm": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                     C.c_void_p]),
    "rmt_causal_attention": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_void_p, C.c_void_p, C.c_void_p]),
    "rmt_attention": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.c_void_p]),
    "rmt_last_error": (C.c_char_p, []),
}


class RmtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"rmt error {code}: {msg}")
        self.code = code


_LIB = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = h
    return _LIB


def check(rc: int) -> int:
    if rc < 0:
        raise RmtError(rc, lib().rmt_last_error().decode())
    return rc
