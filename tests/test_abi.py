"""The C-ABI library loads and exports every symbol include/spc.h declares;
host-side validation rejects bad arguments before anything is launched (no GPU)."""
import ctypes
import os
import re

import pytest

from speculative_kv_sparsity_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "spc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spc_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_stage_calls():
    names = _declared()
    for n in ("spc_retrieval_scores", "spc_group_max_topk", "spc_elastic_update", "spc_sparse_decode_attn"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(L.SIGNATURES), "binding and header disagree"


def test_abi_version_and_strings():
    lib = L.lib()
    assert lib.spc_abi_version() == 3
    assert lib.spc_status_string(0) == b"ok"
    assert b"workspace" in lib.spc_status_string(L.SPC_ERR_WORKSPACE)


def _shape(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, n_groups=8, head_dim=128, v_dim=128, max_len=4096,
                budget=256, n_layers=1, dtype=L.SPC_BF16, scale=128 ** -0.5)
    base.update(kw)
    return L.SpcShape(**base)


@pytest.mark.parametrize("bad", [dict(n_q_heads=30), dict(n_groups=3), dict(budget=0), dict(budget=5000),
                                 dict(batch=0), dict(scale=0.0), dict(dtype=7),
                                 dict(n_q_heads=48, n_kv_heads=16, n_groups=12)])
def test_invalid_shapes_are_rejected_before_launch(bad):
    lib = L.lib()
    s = _shape(**bad)
    dummy = ctypes.c_void_p(16)
    st = lib.spc_retrieval_scores(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, 1 << 30, None)
    assert st in (L.SPC_ERR_INVALID_ARG, L.SPC_ERR_UNSUPPORTED)
    assert lib.spc_last_error()


def test_null_pointers_and_small_workspace_rejected():
    lib = L.lib()
    s = _shape()
    p = ctypes.c_void_p(256)
    assert lib.spc_retrieval_scores(ctypes.byref(s), None, p, p, p, p, 1 << 30, None) == L.SPC_ERR_INVALID_ARG
    need = lib.spc_workspace_size(L.SPC_CALL_SCORES, ctypes.byref(s))
    assert need > 0
    assert lib.spc_retrieval_scores(ctypes.byref(s), p, p, p, p, p, need - 1, None) == L.SPC_ERR_WORKSPACE
    assert b"workspace" in lib.spc_last_error()
    unaligned = ctypes.c_void_p(258)
    assert lib.spc_retrieval_scores(ctypes.byref(s), unaligned, p, p, p, p, need, None) == L.SPC_ERR_INVALID_ARG
    assert lib.spc_group_max_topk(ctypes.byref(s), None, p, p, p, None, 0, None) == L.SPC_ERR_INVALID_ARG
    assert lib.spc_elastic_update(ctypes.byref(s), p, p, p, p, p, p, p, None, None, None, None, 0, 1, 0,
                                  None, None) == L.SPC_ERR_INVALID_ARG            # no flags
    assert lib.spc_elastic_reset(ctypes.byref(s), 3, p, p, None) == L.SPC_ERR_INVALID_ARG   # batch index
    ql = L.SpcQLayout(32 * 128, 0, 128)
    kl = L.SpcKvLayout(0, 0, 0, 256, 128)
    assert lib.spc_sparse_decode_attn(ctypes.byref(s), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                      L.SPC_ROWS_GATHER, 0, 1, p, p, 1 << 30, None) == L.SPC_ERR_INVALID_ARG
    assert lib.spc_sparse_decode_attn(ctypes.byref(s), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                      L.SPC_ROWS_SLOTS, 0, 2, p, p, 1 << 30, None) == L.SPC_ERR_INVALID_ARG
    s2 = _shape(head_dim=96, v_dim=96)
    assert lib.spc_sparse_decode_attn(ctypes.byref(s2), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                      L.SPC_ROWS_SLOTS, 0, 1, p, p, 1 << 30, None) == L.SPC_ERR_UNSUPPORTED


def test_workspace_sizes():
    lib = L.lib()
    s = _shape(batch=2, max_len=32768, budget=2048, n_layers=32)
    # one (max, sum) pair per head and tile of 128 positions (MLA scoring: tiles of 256 or 512)
    assert lib.spc_workspace_size(L.SPC_CALL_SCORES, ctypes.byref(s)) == 2 * 32 * 256 * 8
    # one (max, sum) pair and one v_dim vector per head, layer and split of 128 rows
    assert lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(s)) == 2 * 32 * 32 * 16 * (128 * 4 + 8)
    # keys (one uint32 per position) + 256-bin histograms per 1024-position chunk
    assert lib.spc_workspace_size(L.SPC_CALL_TOPK, ctypes.byref(s)) == 2 * 8 * (32768 * 4 + 32 * 256 * 4)
    assert lib.spc_workspace_size(L.SPC_CALL_ELASTIC, ctypes.byref(s)) == 0
    # MLA: 4 sequences, 128 heads over one shared latent head (576 scored dims, 512 value dims)
    m = _shape(batch=4, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
               budget=2048, scale=192 ** -0.5)
    assert lib.spc_workspace_size(L.SPC_CALL_SCORES, ctypes.byref(m)) == 4 * 128 * 64 * 8   # tiles of 512
    # one 2048-row split per head for budgets of up to 2048 rows with >= 512 heads (4 x 128 here; the
    # whole call then writes the output from the split kernel, but spc_attn_partial still fills these)
    assert lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(m)) == 4 * 128 * 1 * (512 * 4 + 8)
    # a larger budget: 1024-row splits once the launch has >= 1024 workgroups (4 x 128 x 3 here)
    m3 = _shape(batch=4, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                budget=3000, scale=192 ** -0.5)
    assert lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(m3)) == 4 * 128 * 3 * (512 * 4 + 8)
    small = _shape(batch=1, n_q_heads=16, n_kv_heads=1, n_groups=16, head_dim=576, v_dim=512, max_len=4096,
                   budget=512, scale=192 ** -0.5)
    assert lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(small)) == 16 * 2 * (512 * 4 + 8)   # 256-row splits


def test_front_end_host_validation():
    """spc_retrieval_head_qk rejects bad sizes before launching (pointers are never dereferenced)."""
    lib = L.lib()
    s = _shape()
    rope = L.SpcRope(500000.0, 16.0, 2048, 32.0, 1.0)
    p = ctypes.c_void_p(256)
    ws_ok = lib.spc_workspace_size(L.SPC_CALL_FRONT, ctypes.byref(s))
    # one (max) float32 partial per slice, sequence and output row, plus the per-slice sums of squares
    assert ws_ok == 16 * 16 * ((32 + 8) * 128 + 1) * 4

    def call(shape=s, hidden=4096, vocab=1000, r=rope, eps=1e-5, ptr=p, ws_bytes=ws_ok):
        return lib.spc_retrieval_head_qk(ctypes.byref(shape), hidden, vocab, ctypes.byref(r), eps, ptr, ptr, ptr, ptr,
                                         ptr, ptr, ptr, ptr, ptr, ws_bytes, None)

    assert call(hidden=4000) == L.SPC_ERR_INVALID_ARG          # not a multiple of 1024
    assert call(hidden=32768) == L.SPC_ERR_INVALID_ARG         # above 16384
    assert call(vocab=0) == L.SPC_ERR_INVALID_ARG
    assert call(eps=-1.0) == L.SPC_ERR_INVALID_ARG
    assert call(r=L.SpcRope(500000.0, 16.0, 2048, 1.0, 32.0)) == L.SPC_ERR_INVALID_ARG   # beta_fast <= beta_slow
    assert call(r=L.SpcRope(0.5, 1.0, 2048, 32.0, 1.0)) == L.SPC_ERR_INVALID_ARG         # base <= 1
    assert call(shape=_shape(batch=17)) == L.SPC_ERR_UNSUPPORTED
    assert call(shape=_shape(head_dim=96, v_dim=96)) == L.SPC_ERR_UNSUPPORTED
    assert call(ptr=None) == L.SPC_ERR_INVALID_ARG
    assert call(ptr=ctypes.c_void_p(258)) == L.SPC_ERR_INVALID_ARG                      # misaligned
    assert call(ws_bytes=ws_ok - 1) == L.SPC_ERR_WORKSPACE
    assert b"workspace" in lib.spc_last_error()


def test_offload_thresholds_match_the_oracle():
    """Host arithmetic in the library (no GPU): bit-exact against the oracle's bisection."""
    import json
    import numpy as np

    from oracle import spc_oracle as O
    from speculative_kv_sparsity_amd import api
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "offload_thresholds.json")))
    assert api.spc_offload_thresholds(g["gpu_bytes"], **g["model"]) == g["thresholds"]
    rng = np.random.default_rng(11)
    for _ in range(200):
        model = dict(fixed_bytes=int(rng.integers(0, 10 ** 11)), token_bytes=int(rng.integers(0, 10 ** 6)),
                     n_layers=int(rng.integers(1, 81)), batch=int(rng.integers(1, 65)),
                     n_kv_heads=int(rng.integers(1, 33)), head_dim=int(rng.choice([64, 128, 576])),
                     v_dim=int(rng.choice([0, 64, 128, 512])), budget=int(rng.integers(0, 8193)),
                     elem_bytes=int(rng.choice([1, 2, 4])))
        gpu = int(rng.integers(0, 3 * 10 ** 11))
        assert api.spc_offload_thresholds(gpu, **model) == O.offload_thresholds(gpu, **model), (gpu, model)
    lib = L.lib()
    bad = L.SpcMemModel(-1, 0, 0, 1, 1, 1, 1, 1, 1, 1)
    out = (ctypes.c_int32 * 2)()
    assert lib.spc_offload_thresholds(ctypes.byref(bad), out) == L.SPC_ERR_INVALID_ARG


def test_thresholds_from_the_memory_model():
    """The library's thresholds for the 32K step's shapes on a GPU budget that holds about 20 of the 32
    layers' full K/V at 32K: the count of offloaded layers follows the pages' loop."""
    from oracle import spc_oracle as O
    from speculative_kv_sparsity_amd import api
    from speculative_kv_sparsity_amd import workload as W
    p = W.PRESETS["b1_32k"]
    per_layer_32k = p.batch * p.n_kv_heads * (p.head_dim + p.v_dim) * 2 * p.max_len
    model = dict(fixed_bytes=16 * 10 ** 9, token_bytes=p.n_kv_heads * p.head_dim * 2 + p.n_q_heads * 4,
                 n_layers=p.n_layers, batch=p.batch, n_kv_heads=p.n_kv_heads, head_dim=p.head_dim, v_dim=p.v_dim,
                 budget=p.budget, elem_bytes=2)
    gpu = 16 * 10 ** 9 + 20 * per_layer_32k
    th = api.spc_offload_thresholds(gpu, **model)
    assert th == O.offload_thresholds(gpu, **model)
    c = O.offloaded_layers(p.max_len, th)
    assert 12 <= c <= 16
    assert O.memory_bytes(p.max_len, c, **model) <= gpu < O.memory_bytes(p.max_len, c - 1, **model)


def test_lag1_plan_host_validation():
    """spc_elastic_plan_lag1 needs a pool of at least two selections and rejects NULLs before launching
    (every call here fails validation: the fake pointers are never dereferenced)."""
    lib = L.lib()
    p = ctypes.c_void_p(256)
    ptrs = [p] * 11                       # sel_cur ... attend_count
    pool = _shape(budget=512)

    def call(shape, sel_budget, pointers=ptrs):
        assert len(pointers) == 11
        return lib.spc_elastic_plan_lag1(ctypes.byref(shape), sel_budget, *pointers, None)

    assert call(pool, 300) == L.SPC_ERR_INVALID_ARG            # 512 < 2 * 300
    assert call(pool, 0) == L.SPC_ERR_INVALID_ARG
    assert call(_shape(max_len=65536, budget=9000), 4000) == L.SPC_ERR_UNSUPPORTED
    assert call(_shape(max_len=65536, budget=8000), 4000) == L.SPC_ERR_UNSUPPORTED   # LDS words
    for i in range(11):
        bad = list(ptrs)
        bad[i] = None
        assert call(pool, 256, bad) == L.SPC_ERR_INVALID_ARG


def test_log_domain_scoring_sizes_and_validation():
    """spc_retrieval_logits / spc_group_max_topk_logits: tile sizes, the stats buffer size, and
    rejection before launch (every call here fails validation: the fake pointers are never used)."""
    lib = L.lib()
    s = _shape(batch=2, max_len=1000)
    assert lib.spc_score_tile(ctypes.byref(s)) == 128
    assert lib.spc_tile_stats_size(ctypes.byref(s)) == 2 * 32 * 8 * 8          # ceil(1000 / 128) = 8 tiles
    mla = _shape(batch=4, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                 budget=2048, scale=192 ** -0.5)
    # 4 sequences x 64 tiles of 512 = 256 scoring workgroups (all 128 heads each): the large tile
    assert lib.spc_score_tile(ctypes.byref(mla)) == 512
    assert lib.spc_tile_stats_size(ctypes.byref(mla)) == 4 * 128 * 64 * 8
    mla1 = _shape(batch=1, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                  budget=2048, scale=192 ** -0.5)
    assert lib.spc_score_tile(ctypes.byref(mla1)) == 256                      # 64 workgroups of 512: too few
    assert lib.spc_tile_stats_size(ctypes.byref(mla1)) == 128 * 128 * 8
    assert lib.spc_score_tile(ctypes.byref(_shape(budget=0))) == 0
    p = ctypes.c_void_p(256)
    ts = lib.spc_tile_stats_size(ctypes.byref(s))
    assert lib.spc_retrieval_logits(ctypes.byref(s), p, p, p, p, None, ts, None) == L.SPC_ERR_INVALID_ARG
    assert lib.spc_retrieval_logits(ctypes.byref(s), p, p, p, p, ctypes.c_void_p(260), ts,
                                    None) == L.SPC_ERR_INVALID_ARG
    # a tile_stats buffer smaller than the shape needs is rejected by the library itself
    assert lib.spc_retrieval_logits(ctypes.byref(s), p, p, p, p, p, ts - 8, None) == L.SPC_ERR_INVALID_ARG
    assert b"tile_stats" in lib.spc_last_error()
    assert lib.spc_retrieval_logits(ctypes.byref(_shape(head_dim=96)), p, p, p, p, p, 1 << 40,
                                    None) == L.SPC_ERR_UNSUPPORTED
    # one KV head's keys are read through a 32-bit range: 2^23 bf16 rows of 128 reach 2 GiB
    assert lib.spc_retrieval_logits(ctypes.byref(_shape(max_len=1 << 23)), p, p, p, p, p, 1 << 40,
                                    None) == L.SPC_ERR_UNSUPPORTED
    assert lib.spc_retrieval_logits(ctypes.byref(_shape(max_len=1 << 22)), p, p, p, p, None, 1 << 40,
                                    None) == L.SPC_ERR_INVALID_ARG
    # with one query head per group the stats may be NULL: validation goes on past them (here to the
    # unsupported head_dim) instead of rejecting the NULL
    one = _shape(n_q_heads=8, n_groups=8, head_dim=96)
    assert lib.spc_retrieval_logits(ctypes.byref(one), p, p, p, p, None, 0, None) == L.SPC_ERR_UNSUPPORTED
    assert b"tile_stats" not in lib.spc_last_error()
    need = lib.spc_workspace_size(L.SPC_CALL_TOPK, ctypes.byref(s))
    # four heads per group: the tile stats are required, and their size is checked
    assert lib.spc_group_max_topk_logits(ctypes.byref(s), p, None, 0, p, p, p, p, need, None) == L.SPC_ERR_INVALID_ARG
    assert b"tile_stats" in lib.spc_last_error()
    assert lib.spc_group_max_topk_logits(ctypes.byref(s), p, p, ts - 8, p, p, p, p, need,
                                         None) == L.SPC_ERR_INVALID_ARG
    assert b"tile_stats" in lib.spc_last_error()
    assert lib.spc_group_max_topk_logits(ctypes.byref(s), p, p, ts, p, p, p, p, need - 1, None) == L.SPC_ERR_WORKSPACE
    assert lib.spc_group_max_topk_logits(ctypes.byref(s), p, ctypes.c_void_p(260), ts, p, p, p, p, need,
                                         None) == L.SPC_ERR_INVALID_ARG
    wide = _shape(n_q_heads=128, n_kv_heads=1, n_groups=1)                      # 128 heads in one group
    assert lib.spc_group_max_topk_logits(ctypes.byref(wide), p, p, 1 << 40, p, p, p, p, 1 << 40,
                                         None) == L.SPC_ERR_UNSUPPORTED
    # one head per group: NULL stats of size 0 are accepted (checked here with a workspace too small)
    mha = _shape(n_q_heads=8, n_kv_heads=8, n_groups=8)
    need_mha = lib.spc_workspace_size(L.SPC_CALL_TOPK, ctypes.byref(mha))
    assert lib.spc_group_max_topk_logits(ctypes.byref(mha), p, None, 0, p, p, p, p, need_mha - 1,
                                         None) == L.SPC_ERR_WORKSPACE


def test_noalloc_attention_rejects_partials_beyond_its_scratch():
    """The allocation-free attention holds the partials of one call in a 64 MiB array: a layer range
    needing more is rejected before anything launches; a bad layer range too (fake pointers unused)."""
    lib = L.lib()
    p = ctypes.c_void_p(256)
    ql, kl = L.SpcQLayout(4096, 0, 128), L.SpcKvLayout(0, 0, 0, 256, 128)
    big = _shape(batch=16, n_layers=32, max_len=32768, budget=2048)    # 16 x 32 x 32 x 16 x 520 B = 136 MB
    st = lib.spc_sparse_decode_attn_noalloc(ctypes.byref(big), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                            L.SPC_ROWS_SLOTS, 0, 32, p, None)
    assert st == L.SPC_ERR_WORKSPACE and b"split the layer range" in lib.spc_last_error()
    st = lib.spc_sparse_decode_attn_noalloc(ctypes.byref(big), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                            L.SPC_ROWS_SLOTS, 3, 2, p, None)
    assert st == L.SPC_ERR_INVALID_ARG


def test_attention_halves_validation():
    """spc_attn_partial / spc_attn_merge reject bad arguments before launching (fake pointers unused)."""
    lib = L.lib()
    s = _shape(n_layers=4)
    p = ctypes.c_void_p(256)
    need = lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(s))
    assert need > 0
    ql = L.SpcQLayout(32 * 128, 0, 128)
    kl = L.SpcKvLayout(0, 0, 0, 256, 128)
    assert lib.spc_attn_partial(ctypes.byref(s), p, ctypes.byref(ql), p, ctypes.byref(kl), None, None,
                                L.SPC_ROWS_SLOTS, 0, 4, p, need, None) == L.SPC_ERR_INVALID_ARG      # rows
    assert lib.spc_attn_partial(ctypes.byref(s), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                L.SPC_ROWS_SLOTS, 0, 4, p, need - 1, None) == L.SPC_ERR_WORKSPACE
    assert lib.spc_attn_merge(ctypes.byref(s), 0, 4, None, need, p, None) == L.SPC_ERR_INVALID_ARG
    assert lib.spc_attn_merge(ctypes.byref(s), 0, 4, p, need - 1, p, None) == L.SPC_ERR_WORKSPACE
    assert lib.spc_attn_merge(ctypes.byref(s), 2, 5, p, need, p, None) == L.SPC_ERR_INVALID_ARG    # layers
    assert lib.spc_attn_merge(ctypes.byref(s), 0, 4, p, need, ctypes.c_void_p(264), None) == L.SPC_ERR_INVALID_ARG
    big = _shape(max_len=1 << 20, budget=200000)                                  # > 1024 splits
    assert lib.spc_attn_merge(ctypes.byref(big), 0, 1, p, 1 << 40, p, None) == L.SPC_ERR_UNSUPPORTED
    # rows are read through 32-bit ranges: one head's rows must stay under 2 GiB, and a row stride
    # below the key or value width is refused (MLA latent rows here; the GQA case below)
    for max_len, row, ok in ((1 << 20, 576, True), (1 << 21, 576, False), (4096, 512, False)):
        mla = _shape(batch=1, n_q_heads=16, n_kv_heads=1, n_groups=16, head_dim=576, v_dim=512, max_len=max_len,
                     budget=2048, scale=192 ** -0.5)
        need_m = lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(mla))
        mql = L.SpcQLayout(16 * 576, 0, 576)
        mkl = L.SpcKvLayout(max_len * row, 0, 0, row, 0)
        rc = lib.spc_attn_partial(ctypes.byref(mla), p, ctypes.byref(mql), p, ctypes.byref(mkl), p, p,
                                  L.SPC_ROWS_GATHER, 0, 1, p, need_m - 1, None)
        assert rc == (L.SPC_ERR_WORKSPACE if ok else L.SPC_ERR_UNSUPPORTED), (max_len, row, rc)
    for max_len, row, ok in ((1 << 21, 256, True), (1 << 22, 128, True), (1 << 23, 128, False), (1 << 22, 256, False),
                             (4096, 96, False)):
        g = _shape(max_len=max_len, budget=2048)
        need_g = lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(g))
        gkl = L.SpcKvLayout(0, 0, 0, row, row // 2 if row == 256 else 0)
        rc = lib.spc_attn_partial(ctypes.byref(g), p, ctypes.byref(ql), p, ctypes.byref(gkl), p, p,
                                  L.SPC_ROWS_GATHER, 0, 1, p, need_g - 1, None)
        assert rc == (L.SPC_ERR_WORKSPACE if ok else L.SPC_ERR_UNSUPPORTED), (max_len, row, rc)


def test_mla_expand_validation():
    """spc_mla_expand rejects what it does not support before launching (fake pointers unused)."""
    lib = L.lib()
    mla = _shape(batch=4, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                 budget=2048, scale=192 ** -0.5)
    p = ctypes.c_void_p(256)
    args = [p] * 7                                   # latent, w_uk, w_uv, q_nope, q_rope, load_pos, load_slot
    assert lib.spc_mla_expand(ctypes.byref(mla), 96, 128, *args, p, p, p, None) == L.SPC_ERR_UNSUPPORTED  # nope 96
    assert lib.spc_mla_expand(ctypes.byref(mla), 128, 128, None, *args[1:], p, p, p, None) == L.SPC_ERR_INVALID_ARG
    # the query triple is all or nothing
    assert lib.spc_mla_expand(ctypes.byref(mla), 128, 128, p, p, p, None, p, p, p, p, p, p, None) \
        == L.SPC_ERR_INVALID_ARG
    assert lib.spc_mla_expand(ctypes.byref(mla), 128, 128, ctypes.c_void_p(264), *args[1:], p, p, p, None) \
        == L.SPC_ERR_INVALID_ARG                                                               # latent alignment
    gqa = _shape()
    assert lib.spc_mla_expand(ctypes.byref(gqa), 128, 128, *args, p, p, p, None) == L.SPC_ERR_UNSUPPORTED
    big = _shape(batch=17, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                 budget=2048)
    assert lib.spc_mla_expand(ctypes.byref(big), 128, 128, *args, p, p, p, None) == L.SPC_ERR_UNSUPPORTED
    one_group = _shape(batch=4, n_q_heads=128, n_kv_heads=1, n_groups=1, head_dim=576, v_dim=512,
                       max_len=32768, budget=2048)
    assert lib.spc_mla_expand(ctypes.byref(one_group), 128, 128, *args, p, p, p, None) == L.SPC_ERR_INVALID_ARG


def test_grid_limits_are_checked_before_launch():
    """Instance counts that would not fit the second grid dimension are rejected, not launched."""
    lib = L.lib()
    p = ctypes.c_void_p(256)
    wide = _shape(batch=1024, n_q_heads=128, n_kv_heads=8, n_groups=8)           # 131072 (sequence, head) pairs
    assert lib.spc_retrieval_scores(ctypes.byref(wide), p, p, p, p, p, 1 << 40, None) == L.SPC_ERR_UNSUPPORTED
    assert b"n_q_heads" in lib.spc_last_error()
    s = _shape(batch=64, n_q_heads=32, n_kv_heads=32, n_groups=32, n_layers=64)   # 64 * 64 * 32 instances
    ql = L.SpcQLayout(32 * 128, 0, 128)
    kl = L.SpcKvLayout(0, 0, 0, 256, 128)
    ws = lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(s))
    assert lib.spc_sparse_decode_attn(ctypes.byref(s), p, ctypes.byref(ql), p, ctypes.byref(kl), p, None,
                                      L.SPC_ROWS_SLOTS, 0, 64, p, p, ws, None) == L.SPC_ERR_UNSUPPORTED
    assert b"layer range" in lib.spc_last_error()


def test_group_and_kv_head_counts():
    """One of n_groups and n_kv_heads must divide the other: a group inside one KV head (GQA, MHA,
    MLA) or KV heads inside one group (one selection shared by all heads, or by pairs of KV heads).
    The copy needs every KV head inside one group.  Only validation runs (fake pointers)."""
    lib = L.lib()
    p = ctypes.c_void_p(256)
    for g in (1, 2, 4, 8, 16, 32):
        s = _shape(n_groups=g)
        assert lib.spc_workspace_size(L.SPC_CALL_TOPK, ctypes.byref(s)) > 0, g
        assert lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(s)) > 0, g
    assert lib.spc_workspace_size(L.SPC_CALL_TOPK, ctypes.byref(_shape(n_q_heads=48, n_kv_heads=16,
                                                                       n_groups=12))) == 0
    lay = L.SpcKvLayout(0, 0, 0, 256, 128)
    for g, want in ((16, L.SPC_ERR_UNSUPPORTED), (32, L.SPC_ERR_UNSUPPORTED)):
        st = lib.spc_elastic_update(ctypes.byref(_shape(n_groups=g)), None, None, None, None, p, p, p, p,
                                    ctypes.byref(lay), p, ctypes.byref(lay), 0, 1, L.SPC_COPY, None, None)
        assert st == want and b"KV head" in lib.spc_last_error()
    # one selection for every KV head passes the group check (and fails later, on the unpinned host pointer)
    st = lib.spc_elastic_update(ctypes.byref(_shape(n_groups=1)), None, None, None, None, p, p, p, p,
                                ctypes.byref(lay), p, ctypes.byref(lay), 0, 1, L.SPC_COPY, None, None)
    assert st == L.SPC_ERR_NOT_MAPPED


def test_mla_attention_with_projection_validation():
    """spc_mla_attn_out_proj rejects what it does not support before launching (fake pointers unused)."""
    lib = L.lib()
    mla = _shape(batch=4, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                 budget=2048, scale=192 ** -0.5)
    p = ctypes.c_void_p(256)
    ql = L.SpcQLayout(128 * 576, 0, 576)
    kl = L.SpcKvLayout(32768 * 576, 0, 0, 576, 0)
    ws_ok = lib.spc_workspace_size(L.SPC_CALL_ATTN, ctypes.byref(mla))

    def call(shape=mla, q=p, rows=p, layer=0, dv=128, w_uv=p, o_lat=p, out=p, ws_bytes=ws_ok, kvl=kl):
        return lib.spc_mla_attn_out_proj(ctypes.byref(shape), q, ctypes.byref(ql), p, ctypes.byref(kvl), rows, p,
                                         L.SPC_ROWS_GATHER, layer, dv, w_uv, o_lat, out, p, ws_bytes, None)

    assert call(q=None) == L.SPC_ERR_INVALID_ARG
    assert call(w_uv=None) == L.SPC_ERR_INVALID_ARG and call(o_lat=None) == L.SPC_ERR_INVALID_ARG
    assert call(out=None) == L.SPC_ERR_INVALID_ARG
    assert call(layer=1) == L.SPC_ERR_INVALID_ARG and call(layer=-1) == L.SPC_ERR_INVALID_ARG
    assert call(dv=0) == L.SPC_ERR_INVALID_ARG and call(dv=4097) == L.SPC_ERR_INVALID_ARG
    assert call(w_uv=ctypes.c_void_p(264)) == L.SPC_ERR_INVALID_ARG                   # alignment
    assert call(ws_bytes=ws_ok - 1) == L.SPC_ERR_WORKSPACE
    assert call(kvl=L.SpcKvLayout(32768 * 576, 0, 0, 576, 512)) == L.SPC_ERR_UNSUPPORTED   # V inside the row
    assert call(shape=_shape()) == L.SPC_ERR_UNSUPPORTED                              # a GQA shape
    big = _shape(batch=17, n_q_heads=128, n_kv_heads=1, n_groups=128, head_dim=576, v_dim=512, max_len=32768,
                 budget=2048)
    assert call(shape=big) == L.SPC_ERR_UNSUPPORTED
