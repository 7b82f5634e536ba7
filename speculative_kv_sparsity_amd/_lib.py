"""ctypes declarations of libspc.so (mirrors include/spc.h).

The library is loaded on first use and the load fails loudly when it has not
been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspc.so")

SPC_OK = 0
SPC_ERR_INVALID_ARG = 1
SPC_ERR_UNSUPPORTED = 2
SPC_ERR_WORKSPACE = 3
SPC_ERR_NOT_MAPPED = 4
SPC_ERR_HIP = 5

SPC_F32 = 0
SPC_BF16 = 1

SPC_CALL_SCORES = 1
SPC_CALL_TOPK = 2
SPC_CALL_ELASTIC = 3
SPC_CALL_ATTN = 4
SPC_CALL_FRONT = 5

SPC_PLAN = 1
SPC_COPY = 2

SPC_ROWS_SLOTS = 0
SPC_ROWS_GATHER = 1


class SpcShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("budget", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class SpcKvLayout(ctypes.Structure):
    _fields_ = [("s_b", ctypes.c_int64), ("s_layer", ctypes.c_int64), ("s_head", ctypes.c_int64),
                ("s_row", ctypes.c_int64), ("s_kv", ctypes.c_int64)]


class SpcRope(ctypes.Structure):
    _fields_ = [("base", ctypes.c_float), ("factor", ctypes.c_float), ("orig_max_pos", ctypes.c_int32),
                ("beta_fast", ctypes.c_float), ("beta_slow", ctypes.c_float)]


class SpcMemModel(ctypes.Structure):
    _fields_ = [("gpu_bytes", ctypes.c_int64), ("fixed_bytes", ctypes.c_int64), ("token_bytes", ctypes.c_int64),
                ("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32)]


class SpcQLayout(ctypes.Structure):
    _fields_ = [("s_b", ctypes.c_int64), ("s_layer", ctypes.c_int64), ("s_head", ctypes.c_int64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

SIGNATURES = {
    "spc_abi_version": (_I, []),
    "spc_status_string": (ctypes.c_char_p, [_I]),
    "spc_last_error": (ctypes.c_char_p, []),
    "spc_workspace_size": (_SZ, [_I, ctypes.POINTER(SpcShape)]),
    "spc_retrieval_scores": (_I, [ctypes.POINTER(SpcShape), _P, _P, _P, _P, _P, _SZ, _P]),
    "spc_group_max_topk": (_I, [ctypes.POINTER(SpcShape), _P, _P, _P, _P, _P, _SZ, _P]),
    "spc_retrieval_logits": (_I, [ctypes.POINTER(SpcShape), _P, _P, _P, _P, _P, _SZ, _P]),
    "spc_score_tile": (_I, [ctypes.POINTER(SpcShape)]),
    "spc_tile_stats_size": (_SZ, [ctypes.POINTER(SpcShape)]),
    "spc_group_max_topk_logits": (_I, [ctypes.POINTER(SpcShape), _P, _P, _SZ, _P, _P, _P, _P, _SZ, _P]),
    "spc_group_max_topk_plan_logits": (_I, [ctypes.POINTER(SpcShape), _P, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _SZ, _P]),
    "spc_elastic_update": (_I, [ctypes.POINTER(SpcShape), _P, _P, _P, _P, _P, _P, _P, _P,
                                ctypes.POINTER(SpcKvLayout), _P, ctypes.POINTER(SpcKvLayout), _I32, _I32,
                                ctypes.c_uint, _P, _P]),
    "spc_elastic_reset": (_I, [ctypes.POINTER(SpcShape), _I32, _P, _P, _P]),
    "spc_sparse_decode_attn": (_I, [ctypes.POINTER(SpcShape), _P, ctypes.POINTER(SpcQLayout), _P,
                                    ctypes.POINTER(SpcKvLayout), _P, _P, _I, _I32, _I32, _P, _P, _SZ, _P]),
    "spc_sparse_decode_attn_noalloc": (_I, [ctypes.POINTER(SpcShape), _P, ctypes.POINTER(SpcQLayout), _P,
                                            ctypes.POINTER(SpcKvLayout), _P, _P, _I, _I32, _I32, _P, _P]),
    "spc_attn_partial": (_I, [ctypes.POINTER(SpcShape), _P, ctypes.POINTER(SpcQLayout), _P,
                              ctypes.POINTER(SpcKvLayout), _P, _P, _I, _I32, _I32, _P, _SZ, _P]),
    "spc_attn_merge": (_I, [ctypes.POINTER(SpcShape), _I32, _I32, _P, _SZ, _P, _P]),
    "spc_mla_expand": (_I, [ctypes.POINTER(SpcShape), _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "spc_mla_absorb_q": (_I, [ctypes.POINTER(SpcShape), _I32, _P, _P, _P, _P, _P]),
    "spc_mla_out_proj": (_I, [ctypes.POINTER(SpcShape), _I32, _P, _P, _I32, _P, _P]),
    "spc_mla_attn_out_proj": (_I, [ctypes.POINTER(SpcShape), _P, ctypes.POINTER(SpcQLayout), _P,
                                   ctypes.POINTER(SpcKvLayout), _P, _P, _I, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "spc_elastic_plan_lag1": (_I, [ctypes.POINTER(SpcShape), _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "spc_offload_thresholds": (_I, [ctypes.POINTER(SpcMemModel), ctypes.POINTER(ctypes.c_int32)]),
    "spc_retrieval_head_qk": (_I, [ctypes.POINTER(SpcShape), _I32, ctypes.c_int64, ctypes.POINTER(SpcRope),
                                   ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m speculative_kv_sparsity_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib
