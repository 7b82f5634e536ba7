"""Thin Python binding of libspc with the C-ABI's names (argument marshalling only).

Tensors are torch tensors; their ``data_ptr()`` is handed to the library.  Every
stage runs in the library's HIP kernels; nothing here computes.  A non-OK
status raises ``SpcError`` carrying the library's message.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib as L
from ._lib import (SPC_BF16, SPC_CALL_ATTN, SPC_CALL_FRONT, SPC_CALL_SCORES, SPC_CALL_TOPK, SPC_COPY, SPC_F32,
                   SPC_PLAN, SPC_ROWS_GATHER, SPC_ROWS_SLOTS, SpcKvLayout, SpcMemModel, SpcQLayout, SpcRope,
                   SpcShape)

__all__ = ["SpcError", "make_shape", "kv_layout", "q_layout", "spc_abi_version", "spc_workspace_size",
           "spc_retrieval_scores", "spc_group_max_topk", "spc_elastic_update", "spc_elastic_reset",
           "spc_sparse_decode_attn", "SPC_PLAN", "SPC_COPY", "SPC_ROWS_SLOTS", "SPC_ROWS_GATHER",
           "SPC_CALL_SCORES", "SPC_CALL_TOPK", "SPC_CALL_ATTN", "SPC_CALL_FRONT", "spc_mla_absorb_q",
           "spc_mla_out_proj", "rope_params", "spc_retrieval_head_qk", "spc_offload_thresholds",
           "spc_elastic_plan_lag1", "spc_retrieval_logits", "spc_group_max_topk_logits", "spc_score_tile",
           "spc_tile_stats_size", "tile_stats_shape", "spc_attn_partial", "spc_attn_merge",
           "spc_mla_expand", "spc_sparse_decode_attn_noalloc", "spc_group_max_topk_plan_logits"]


class SpcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        lib = L.lib()
        msg = lib.spc_last_error().decode() or lib.spc_status_string(status).decode()
        raise SpcError(status, msg)


def make_shape(batch, n_q_heads, n_kv_heads, n_groups, head_dim, v_dim, max_len, budget, n_layers, dtype,
               scale) -> SpcShape:
    dt = {"f32": SPC_F32, "bf16": SPC_BF16, torch.float32: SPC_F32, torch.bfloat16: SPC_BF16}[dtype]
    return SpcShape(batch, n_q_heads, n_kv_heads, n_groups, head_dim, v_dim, max_len, budget, n_layers, dt,
                    float(scale))


def kv_layout(t: torch.Tensor) -> SpcKvLayout:
    """Layout of a K/V store shaped [B][layers][H][rows][2][d] (any strides)."""
    assert t.dim() == 6, "expected [B][layers][H][rows][2][d]"
    s = t.stride()
    assert s[5] == 1, "d must be contiguous"
    return SpcKvLayout(s[0], s[1], s[2], s[3], s[4])


def q_layout(s_b: int, s_layer: int, s_head: int) -> SpcQLayout:
    return SpcQLayout(int(s_b), int(s_layer), int(s_head))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def spc_abi_version() -> int:
    return L.lib().spc_abi_version()


def spc_workspace_size(call: int, shape: SpcShape) -> int:
    return int(L.lib().spc_workspace_size(call, ctypes.byref(shape)))


_ws_cache = {}


def _workspace(call: int, shape: SpcShape, device) -> torch.Tensor:
    n = spc_workspace_size(call, shape)
    key = (call, n, str(device))
    ws = _ws_cache.get(key)
    if ws is None:
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def spc_retrieval_scores(shape: SpcShape, q, k, lengths, probs, ws=None, stream=None) -> None:
    for t, n in ((q, "q"), (k, "k"), (lengths, "lengths"), (probs, "probs")):
        _dev(t, n)
    ws = _workspace(SPC_CALL_SCORES, shape, q.device) if ws is None else ws
    _check(L.lib().spc_retrieval_scores(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(lengths), _ptr(probs),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spc_group_max_topk(shape: SpcShape, probs, lengths, sel_idx, sel_count, ws=None, stream=None) -> None:
    for t, n in ((probs, "probs"), (lengths, "lengths"), (sel_idx, "sel_idx"), (sel_count, "sel_count")):
        _dev(t, n)
    ws = _workspace(SPC_CALL_TOPK, shape, probs.device) if ws is None else ws
    _check(L.lib().spc_group_max_topk(ctypes.byref(shape), _ptr(probs), _ptr(lengths), _ptr(sel_idx),
                                      _ptr(sel_count), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spc_score_tile(shape: SpcShape) -> int:
    return int(L.lib().spc_score_tile(ctypes.byref(shape)))


def spc_tile_stats_size(shape: SpcShape) -> int:
    return int(L.lib().spc_tile_stats_size(ctypes.byref(shape)))


def tile_stats_shape(shape: SpcShape) -> tuple:
    """[B][H_q][n_tiles][2] float32 of spc_retrieval_logits' tile statistics."""
    T = spc_score_tile(shape)
    return (shape.batch, shape.n_q_heads, (shape.max_len + T - 1) // T, 2)


def spc_retrieval_logits(shape: SpcShape, q, k, lengths, logits, tile_stats, stream=None) -> None:
    """tile_stats may be None when every query head is its own group (no stats are then computed)."""
    for t, n in ((q, "q"), (k, "k"), (lengths, "lengths"), (logits, "logits")):
        _dev(t, n)
    if tile_stats is not None:
        _dev(tile_stats, "tile_stats")
    _check(L.lib().spc_retrieval_logits(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(lengths), _ptr(logits),
                                        _ptr(tile_stats), _nbytes(tile_stats), _stream(stream)))


def spc_group_max_topk_logits(shape: SpcShape, logits, tile_stats, lengths, sel_idx, sel_count, ws=None,
                              stream=None) -> None:
    for t, n in ((logits, "logits"), (lengths, "lengths"), (sel_idx, "sel_idx"), (sel_count, "sel_count")):
        _dev(t, n)
    if tile_stats is not None:
        _dev(tile_stats, "tile_stats")
    ws = _workspace(SPC_CALL_TOPK, shape, logits.device) if ws is None else ws
    _check(L.lib().spc_group_max_topk_logits(ctypes.byref(shape), _ptr(logits), _ptr(tile_stats),
                                             _nbytes(tile_stats), _ptr(lengths), _ptr(sel_idx), _ptr(sel_count),
                                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spc_group_max_topk_plan_logits(shape: SpcShape, logits, tile_stats, lengths, sel_idx, sel_count, slot_pos,
                                   resident_bm, load_pos, load_slot, load_count, ws=None, stream=None) -> None:
    """spc_group_max_topk_logits followed by the SPC_PLAN half of spc_elastic_update, in one call."""
    for t, n in ((logits, "logits"), (lengths, "lengths"), (sel_idx, "sel_idx"), (sel_count, "sel_count"),
                 (slot_pos, "slot_pos"), (resident_bm, "resident_bm"), (load_pos, "load_pos"),
                 (load_slot, "load_slot"), (load_count, "load_count")):
        _dev(t, n)
    if tile_stats is not None:
        _dev(tile_stats, "tile_stats")
    ws = _workspace(SPC_CALL_TOPK, shape, logits.device) if ws is None else ws
    _check(L.lib().spc_group_max_topk_plan_logits(
        ctypes.byref(shape), _ptr(logits), _ptr(tile_stats), _nbytes(tile_stats), _ptr(lengths), _ptr(sel_idx),
        _ptr(sel_count), _ptr(slot_pos), _ptr(resident_bm), _ptr(load_pos), _ptr(load_slot), _ptr(load_count),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spc_elastic_update(shape: SpcShape, sel_idx, sel_count, slot_pos, resident_bm, load_pos, load_slot,
                       load_count, host_kv=None, host_l: Optional[SpcKvLayout] = None, dev_kv=None,
                       dev_l: Optional[SpcKvLayout] = None, layer_begin: int = 0, layer_end: int = 0,
                       flags: int = SPC_PLAN, plan_stream=None, copy_stream=None) -> None:
    _check(L.lib().spc_elastic_update(
        ctypes.byref(shape), _ptr(sel_idx), _ptr(sel_count), _ptr(slot_pos), _ptr(resident_bm), _ptr(load_pos),
        _ptr(load_slot), _ptr(load_count), _ptr(host_kv), ctypes.byref(host_l) if host_l is not None else None,
        _ptr(dev_kv), ctypes.byref(dev_l) if dev_l is not None else None, int(layer_begin), int(layer_end),
        int(flags), _stream(plan_stream), _stream(copy_stream if copy_stream is not None else plan_stream)))


def spc_elastic_reset(shape: SpcShape, batch_index: int, slot_pos, resident_bm, stream=None) -> None:
    _check(L.lib().spc_elastic_reset(ctypes.byref(shape), int(batch_index), _ptr(slot_pos), _ptr(resident_bm),
                                     _stream(stream)))


def spc_sparse_decode_attn(shape: SpcShape, q, q_l: SpcQLayout, kv, kv_l: SpcKvLayout, rows, row_count,
                           rows_mode: int, layer_begin: int, layer_end: int, out, ws=None, stream=None) -> None:
    _dev(out, "out")
    for t, n in ((q, "q"), (kv, "kv"), (rows, "rows")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
    ws = _workspace(SPC_CALL_ATTN, shape, out.device) if ws is None else ws
    _check(L.lib().spc_sparse_decode_attn(
        ctypes.byref(shape), _ptr(q), ctypes.byref(q_l), _ptr(kv), ctypes.byref(kv_l), _ptr(rows), _ptr(row_count),
        int(rows_mode), int(layer_begin), int(layer_end), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spc_sparse_decode_attn_noalloc(shape: SpcShape, q, q_l: SpcQLayout, kv, kv_l: SpcKvLayout, rows, row_count,
                                   rows_mode: int, layer_begin: int, layer_end: int, out, stream=None) -> None:
    """spc_sparse_decode_attn with its partials in the library's scratch array (no workspace)."""
    _dev(out, "out")
    for t, n in ((q, "q"), (kv, "kv"), (rows, "rows")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
    _check(L.lib().spc_sparse_decode_attn_noalloc(
        ctypes.byref(shape), _ptr(q), ctypes.byref(q_l), _ptr(kv), ctypes.byref(kv_l), _ptr(rows), _ptr(row_count),
        int(rows_mode), int(layer_begin), int(layer_end), _ptr(out), _stream(stream)))


def spc_attn_partial(shape: SpcShape, q, q_l: SpcQLayout, kv, kv_l: SpcKvLayout, rows, row_count, rows_mode: int,
                     layer_begin: int, layer_end: int, ws, stream=None) -> None:
    """The split half of spc_sparse_decode_attn: per-split partials into ws (kept for spc_attn_merge)."""
    for t, n in ((q, "q"), (kv, "kv"), (rows, "rows"), (ws, "ws")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
    _check(L.lib().spc_attn_partial(
        ctypes.byref(shape), _ptr(q), ctypes.byref(q_l), _ptr(kv), ctypes.byref(kv_l), _ptr(rows), _ptr(row_count),
        int(rows_mode), int(layer_begin), int(layer_end), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spc_attn_merge(shape: SpcShape, layer_begin: int, layer_end: int, ws, out, stream=None) -> None:
    """The merge half of spc_sparse_decode_attn: the partials in ws -> out."""
    _dev(out, "out")
    _dev(ws, "ws")
    _check(L.lib().spc_attn_merge(ctypes.byref(shape), int(layer_begin), int(layer_end), _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(out), _stream(stream)))


def spc_mla_expand(shape: SpcShape, nope_dim: int, v_head_dim: int, latent, w_uk, w_uv, load_pos, load_slot,
                   load_count, kv_exp, q_nope=None, q_rope=None, q_exp=None, stream=None) -> None:
    """Literal MLA: the newly loaded rows of every head expanded into its K/V slots (and the joined query)."""
    for t, n in ((latent, "latent"), (w_uk, "w_uk"), (w_uv, "w_uv"), (load_pos, "load_pos"), (load_slot, "load_slot"),
                 (load_count, "load_count"), (kv_exp, "kv_exp")):
        _dev(t, n)
    for t, n in ((q_nope, "q_nope"), (q_rope, "q_rope"), (q_exp, "q_exp")):
        if t is not None:
            _dev(t, n)
    _check(L.lib().spc_mla_expand(ctypes.byref(shape), int(nope_dim), int(v_head_dim), _ptr(latent), _ptr(w_uk),
                                  _ptr(w_uv), _ptr(q_nope), _ptr(q_rope), _ptr(load_pos), _ptr(load_slot),
                                  _ptr(load_count), _ptr(kv_exp), _ptr(q_exp), _stream(stream)))


def spc_mla_absorb_q(shape: SpcShape, nope_dim: int, w_uk, q_nope, q_rope, q_abs, stream=None) -> None:
    for t, n in ((w_uk, "w_uk"), (q_nope, "q_nope"), (q_rope, "q_rope"), (q_abs, "q_abs")):
        _dev(t, n)
    _check(L.lib().spc_mla_absorb_q(ctypes.byref(shape), int(nope_dim), _ptr(w_uk), _ptr(q_nope), _ptr(q_rope),
                                    _ptr(q_abs), _stream(stream)))


def spc_mla_out_proj(shape: SpcShape, dv: int, w_uv, o_lat, layer: int, out, stream=None) -> None:
    for t, n in ((w_uv, "w_uv"), (o_lat, "o_lat"), (out, "out")):
        _dev(t, n)
    _check(L.lib().spc_mla_out_proj(ctypes.byref(shape), int(dv), _ptr(w_uv), _ptr(o_lat), int(layer), _ptr(out),
                                    _stream(stream)))


def spc_mla_attn_out_proj(shape: SpcShape, q, q_l: SpcQLayout, kv, kv_l: SpcKvLayout, rows, row_count,
                          rows_mode: int, layer: int, dv: int, w_uv, o_lat, out, ws=None, stream=None) -> None:
    for t, n in ((q, "q"), (kv, "kv"), (rows, "rows")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
    for t, n in ((w_uv, "w_uv"), (o_lat, "o_lat"), (out, "out")):
        _dev(t, n)
    ws = _workspace(SPC_CALL_ATTN, shape, out.device) if ws is None else ws
    _check(L.lib().spc_mla_attn_out_proj(
        ctypes.byref(shape), _ptr(q), ctypes.byref(q_l), _ptr(kv), ctypes.byref(kv_l), _ptr(rows), _ptr(row_count),
        int(rows_mode), int(layer), int(dv), _ptr(w_uv), _ptr(o_lat), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def rope_params(base: float, factor: float = 1.0, orig_max_pos: int = 2048, beta_fast: float = 32.0,
                beta_slow: float = 1.0) -> SpcRope:
    return SpcRope(float(base), float(factor), int(orig_max_pos), float(beta_fast), float(beta_slow))


def spc_retrieval_head_qk(shape: SpcShape, hidden: int, rope: SpcRope, eps: float, tokens, positions, emb, gamma,
                          wq, wk, q_out, dlm_k, ws=None, stream=None) -> None:
    for t, n in ((tokens, "tokens"), (positions, "positions"), (emb, "emb"), (gamma, "gamma"), (wq, "wq"),
                 (wk, "wk"), (q_out, "q_out"), (dlm_k, "dlm_k")):
        _dev(t, n)
    ws = _workspace(SPC_CALL_FRONT, shape, q_out.device) if ws is None else ws
    _check(L.lib().spc_retrieval_head_qk(ctypes.byref(shape), int(hidden), int(emb.shape[0]), ctypes.byref(rope),
                                         float(eps), _ptr(tokens), _ptr(positions), _ptr(emb), _ptr(gamma), _ptr(wq),
                                         _ptr(wk), _ptr(q_out), _ptr(dlm_k), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)))


def spc_offload_thresholds(gpu_bytes: int, fixed_bytes: int, token_bytes: int, n_layers: int, batch: int,
                           n_kv_heads: int, head_dim: int, v_dim: int, budget: int, elem_bytes: int) -> list:
    """threshold[c], c = 0..n_layers (host arithmetic in the library; see include/spc.h)."""
    m = SpcMemModel(int(gpu_bytes), int(fixed_bytes), int(token_bytes), int(n_layers), int(batch), int(n_kv_heads),
                    int(head_dim), int(v_dim), int(budget), int(elem_bytes))
    out = (ctypes.c_int32 * (int(n_layers) + 1))()
    _check(L.lib().spc_offload_thresholds(ctypes.byref(m), out))
    return list(out)


def spc_elastic_plan_lag1(pool_shape: SpcShape, sel_budget: int, sel_cur, cur_count, sel_next, next_count, slot_pos,
                          resident_bm, load_pos, load_slot, load_count, attend_rows, attend_count, stream=None) -> None:
    for t, n in ((sel_cur, "sel_cur"), (cur_count, "cur_count"), (sel_next, "sel_next"), (next_count, "next_count"),
                 (slot_pos, "slot_pos"), (resident_bm, "resident_bm"), (load_pos, "load_pos"),
                 (load_slot, "load_slot"), (load_count, "load_count"), (attend_rows, "attend_rows"),
                 (attend_count, "attend_count")):
        _dev(t, n)
    _check(L.lib().spc_elastic_plan_lag1(ctypes.byref(pool_shape), int(sel_budget), _ptr(sel_cur), _ptr(cur_count),
                                         _ptr(sel_next), _ptr(next_count), _ptr(slot_pos), _ptr(resident_bm),
                                         _ptr(load_pos), _ptr(load_slot), _ptr(load_count), _ptr(attend_rows),
                                         _ptr(attend_count), _stream(stream)))
