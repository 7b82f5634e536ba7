"""The allocation-free attention entry point (spc_sparse_decode_attn_noalloc) against the entry point
with a caller's workspace, through the C-ABI: two calls in a row on one GPU, the second smaller, each
bit-identical to the workspace call on the same inputs (the same kernels run on the same partial
layout; only where the partials live differs)."""
import numpy as np
import pytest
import torch

from speculative_kv_sparsity_amd import api
from speculative_kv_sparsity_amd import workload as W
from tests.gpu_util import dev_lengths, shape_of

pytestmark = pytest.mark.gpu


def _resident_rows(p, seed):
    """A step's inputs: selections from the GPU's scores and Top-K, K/V placed by plan + copy."""
    w = W.generate(p, device="cuda", seed=seed, steps=1, pin_host=True)
    shape = shape_of(p)
    B, G, K, NL = p.batch, p.n_groups, p.budget, p.n_layers
    lengths = dev_lengths(w.lengths[0])
    logits = torch.empty((B, p.n_q_heads, p.max_len), device="cuda")
    stats = torch.empty(api.tile_stats_shape(shape), device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    sel, cnt = torch.empty((B, G, K), **i32), torch.empty((B, G), **i32)
    slot_pos, bm = torch.empty((B, G, K), **i32), torch.empty((B, G, (p.max_len + 31) // 32), **i32)
    lp, ls, lc = torch.empty((B, G, K), **i32), torch.empty((B, G, K), **i32), torch.empty((B, G), **i32)
    dev = torch.zeros((B, NL, p.n_kv_heads, K, 2, p.head_dim), dtype=p.torch_dtype, device="cuda")
    q = w.q[0].contiguous()
    api.spc_retrieval_logits(shape, q, w.dlm_k, lengths, logits, stats)
    api.spc_group_max_topk_logits(shape, logits, stats, lengths, sel, cnt)
    api.spc_elastic_reset(shape, -1, slot_pos, bm)
    api.spc_elastic_update(shape, sel, cnt, slot_pos, bm, lp, ls, lc, w.host_kv, api.kv_layout(w.host_kv), dev,
                           api.kv_layout(dev), 0, NL, flags=api.SPC_PLAN | api.SPC_COPY)
    return shape, q, dev, slot_pos, sel, cnt


def _compare(p, shape, q, kv, rows, counts, mode, a, z):
    ql = api.q_layout(p.n_q_heads * p.head_dim, 0, p.head_dim)
    shp = (p.batch, p.n_layers, p.n_q_heads, p.v_dim)
    with_ws = torch.full(shp, float("nan"), device="cuda")
    no_alloc = torch.full(shp, float("nan"), device="cuda")
    api.spc_sparse_decode_attn(shape, q, ql, kv, api.kv_layout(kv), rows, counts, mode, a, z, with_ws)
    api.spc_sparse_decode_attn_noalloc(shape, q, ql, kv, api.kv_layout(kv), rows, counts, mode, a, z, no_alloc)
    torch.cuda.synchronize()
    x, y = with_ws.cpu().numpy(), no_alloc.cpu().numpy()
    assert not np.isnan(x[:, a:z]).any()
    np.testing.assert_array_equal(y[:, a:z], x[:, a:z])
    assert np.isnan(y[:, :a]).all() and np.isnan(y[:, z:]).all()      # layers outside the range untouched


def test_noalloc_attention_matches_the_workspace_call_twice_in_a_row():
    # first call: the 32K step's first layer chunk shape (28 of 32 layers, budget 2048; 7.5 MB of partials)
    big = W.PRESETS["b1_32k"].with_(max_len=8192)
    shape, q, dev, slot_pos, _, _ = _resident_rows(big, seed=41)
    _compare(big, shape, q, dev, slot_pos, None, api.SPC_ROWS_SLOTS, 0, 28)
    # second call, smaller: two sequences, 3 layers, budget 96, rows gathered by position from a full cache
    small = W.PRESETS["b16_grow"].with_(batch=2, n_layers=3, max_len=1000, budget=96, start_len=700,
                                        offset_max=200)
    w = W.generate(small, device="cuda", seed=42, steps=1, pin_host=True)
    shape_s, q_s, _, _, sel, cnt = _resident_rows(small, seed=42)
    full = w.host_kv.cuda()
    _compare(small, shape_s, q_s, full, sel, cnt, api.SPC_ROWS_GATHER, 1, 3)


def test_noalloc_attention_rejects_a_range_beyond_its_scratch():
    p = W.PRESETS["b16_grow"].with_(n_layers=32, budget=2048, max_len=4096)
    shape = shape_of(p)
    t = torch.zeros(16, device="cuda")
    ql, kl = api.q_layout(4096, 0, 128), api.SpcKvLayout(0, 0, 0, 256, 128)
    with pytest.raises(api.SpcError) as e:
        api.spc_sparse_decode_attn_noalloc(shape, t, ql, t, kl, t, None, api.SPC_ROWS_SLOTS, 0, 32, t)
    assert e.value.status == 3
