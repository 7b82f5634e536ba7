"""Adaptive offloading (mixed residency) on the GPU against the oracle: layers still on the GPU attend
over the selection gathered from their full cache, offloaded layers over the elastic slots, and a
layer offloaded mid-run gets its slots filled from the host store."""
import numpy as np
import pytest
import torch

from oracle import OracleDecoder
from oracle import spc_oracle as O
from speculative_kv_sparsity_amd import workload as W
from speculative_kv_sparsity_amd.driver import SparseDecoder
from tests.gpu_util import ATTN_DERIVED, ATTN_MAX_ABS, check_topk_tolerance, dev_lengths, raw, sel_lists

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1


def _check_slots(dec, p, kv_raw):
    """Every offloaded layer's slot x holds the host row of position slot_pos[x] (bit-exact)."""
    sp = dec.slot_pos.cpu().numpy()
    dev = raw(dec.dev_kv)
    for layer in range(dec.n_res, p.n_layers):
        for b in range(p.batch):
            for g in range(p.n_groups):
                xs = np.nonzero(sp[b, g] >= 0)[0]
                np.testing.assert_array_equal(dev[b, layer, g, xs], kv_raw[b, layer, g, sp[b, g, xs]])


def test_layers_offloaded_one_at_a_time_while_growing():
    p = W.PRESETS["b16_grow"].with_(batch=3, n_layers=5, max_len=3000, budget=128, start_len=1000,
                                    offset_max=1500)
    steps = 6
    w = W.generate(p, device="cuda", seed=8, steps=steps, pin_host=True)
    L0 = int(w.lengths[0].max())
    th = [L0 + 1, L0 + 2, L0 + 2, L0 + 4, L0 + 5, INT32_MAX]
    expect = [0, 1, 3, 3, 4, 5]
    dec = SparseDecoder(p, w.dlm_k, w.host_kv, layer_chunks=2, thresholds=th)
    ora = OracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale, p.dtype)
    k_raw, kv_raw = raw(w.dlm_k), raw(w.host_kv)
    lens_dev = dev_lengths(w.lengths)
    for t in range(steps):
        seq_len = int(w.lengths[t].max())
        assert dec.offload_for(seq_len) == expect[t] == O.offloaded_layers(seq_len, th)
        q = w.q[t].contiguous()
        dec.step(q, lens_dev[t])
        torch.cuda.synchronize()
        probs, ref_sel = ora.select(raw(q), k_raw, w.lengths[t])
        gsel = sel_lists(dec.sel_idx, dec.sel_count)
        check_topk_tolerance(gsel, ref_sel, O.group_scores(probs, p.n_groups), p.budget)
        plans = ora.plan(gsel)
        lc = dec.load_count.cpu().numpy()
        sp = dec.slot_pos.cpu().numpy()
        for b in range(p.batch):
            for g in range(p.n_groups):
                assert lc[b, g] == len(plans[b][g][0])
                np.testing.assert_array_equal(sp[b, g], ora.slot_pos[b][g])
        # all layers, resident or offloaded, against attention read from the host store by position
        ref = ora.attend(raw(q), kv_raw, gsel, list(range(p.n_layers)))
        err = float(np.max(np.abs(dec.out.cpu().numpy().astype(np.float64) - ref)))
        assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, (t, dec.n_off, err)
        _check_slots(dec, p, kv_raw)


def test_all_resident_matches_all_offloaded():
    """With every layer on the GPU the step is the gather path only; its outputs equal those of the
    all-offloaded step on the same inputs (both read the same K/V rows)."""
    p = W.PRESETS["b1_32k"].with_(max_len=4096, budget=512, n_layers=6)
    w = W.generate(p, device="cuda", seed=9, steps=3, pin_host=True)
    a = SparseDecoder(p, w.dlm_k, w.host_kv, layer_chunks=2)
    r = SparseDecoder(p, w.dlm_k, w.host_kv, layer_chunks=2, thresholds=[INT32_MAX] * (p.n_layers + 1))
    lens = dev_lengths(w.lengths)
    for t in range(3):
        q = w.q[t].contiguous()
        assert r.offload_for(int(w.lengths[t].max())) == 0
        a.step(q, lens[t])
        r.step(q, lens[t])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(a.sel_idx.cpu().numpy(), r.sel_idx.cpu().numpy())
        np.testing.assert_allclose(a.out.cpu().numpy(), r.out.cpu().numpy(), rtol=0, atol=1e-6)
