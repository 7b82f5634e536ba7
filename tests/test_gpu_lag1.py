"""The pipelined loop (lag 1) on the GPU against its oracle: each step's selection (of the next step's
positions), the pool's plan and attended slots bit-exact, the copy of the rows, and the attention over
the previous step's selection read from the host store by position."""
import numpy as np
import pytest
import torch

from oracle import spc_oracle as O
from oracle.decoder import LagOneOracleDecoder
from speculative_kv_sparsity_amd import workload as W
from speculative_kv_sparsity_amd.driver import LagOneDecoder
from tests.gpu_util import ATTN_DERIVED, ATTN_MAX_ABS, check_topk_tolerance, dev_lengths, raw, sel_lists

pytestmark = pytest.mark.gpu


def _run(p, steps, seed, check_layers=None, delay_cycles=0):
    w = W.generate(p, device="cuda", seed=seed, steps=steps, pin_host=True)
    dec = LagOneDecoder(p, w.dlm_k, w.host_kv)
    if delay_cycles:
        # hold the copy stream back each step: the events must still order attention after the copy
        side, step = dec.side, dec.step

        def slow_step(q, lengths):
            with torch.cuda.stream(side):
                torch.cuda._sleep(delay_cycles)
            step(q, lengths)

        dec.step = slow_step
    ora = LagOneOracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale,
                              p.dtype, pool=dec.P)
    k_raw, kv_raw = raw(w.dlm_k), raw(w.host_kv)
    layers = list(range(p.n_layers)) if check_layers is None else check_layers
    lens = dev_lengths(w.lengths)
    outs = []
    for t in range(steps):
        q = w.q[t].contiguous()
        nx = dec.t % 2
        dec.step(q, lens[t])
        torch.cuda.synchronize()
        probs, ref_sel = ora.select(raw(q), k_raw, w.lengths[t])
        gsel = sel_lists(dec.sel[nx], dec.cnt[nx])
        check_topk_tolerance(gsel, ref_sel, O.group_scores(probs, p.n_groups), p.budget)
        plans, cur = ora.plan_lag1(gsel)
        lp, ls = dec.load_pos[nx].cpu().numpy(), dec.load_slot[nx].cpu().numpy()
        lc = dec.load_count[nx].cpu().numpy()
        sp = dec.slot_pos.cpu().numpy()
        ar, ac = dec.attend_rows.cpu().numpy(), dec.attend_count.cpu().numpy()
        dev = raw(dec.dev_kv)
        for b in range(p.batch):
            for g in range(p.n_groups):
                to_load, load_slot, attend = plans[b][g]
                assert lc[b, g] == len(to_load)
                np.testing.assert_array_equal(lp[b, g, :lc[b, g]], to_load)
                np.testing.assert_array_equal(ls[b, g, :lc[b, g]], load_slot)
                np.testing.assert_array_equal(sp[b, g], ora.slot_pos[b][g])
                assert ac[b, g] == len(attend)
                np.testing.assert_array_equal(ar[b, g, :ac[b, g]], attend)
                # every pool row holds the host row of its position, in every layer
                xs = np.nonzero(sp[b, g] >= 0)[0]
                for layer in layers:
                    np.testing.assert_array_equal(dev[b, layer, g, xs], kv_raw[b, layer, g, sp[b, g, xs]])
        ref = ora.attend(raw(q), kv_raw, cur, layers)
        got = dec.out.cpu().numpy().astype(np.float64)[:, layers]
        err = float(np.max(np.abs(got - ref)))
        assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, (t, err)
        outs.append(got)
    return outs


def test_lag1_tiny():
    _run(W.PRESETS["tiny"], steps=8, seed=0)


def test_lag1_ragged_growing_batch():
    p = W.PRESETS["b16_grow"].with_(batch=3, n_layers=4, max_len=3000, budget=256, start_len=1000,
                                    offset_max=1500)
    _run(p, steps=6, seed=1)


def test_lag1_delayed_copies_do_not_change_results():
    p = W.PRESETS["b1_32k"].with_(max_len=4096, budget=512, n_layers=6)
    a = _run(p, steps=4, seed=2)
    b = _run(p, steps=4, seed=2, delay_cycles=2_000_000)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_lag1_llama8b_32k_full_size():
    _run(W.PRESETS["b1_32k"], steps=3, seed=3, check_layers=[0, 31])
