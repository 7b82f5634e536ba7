"""End-to-end decode steps through the stream driver, checked step by step against the oracle."""
import os
import time

import numpy as np
import pytest
import torch

from oracle import OracleDecoder
from oracle import spc_oracle as O
from speculative_kv_sparsity_amd import workload as W
from speculative_kv_sparsity_amd.driver import SparseDecoder
from tests.gpu_util import ATTN_DERIVED, ATTN_MAX_ABS, check_topk_tolerance, dev_lengths, raw, sel_lists

pytestmark = pytest.mark.gpu

PROGRESS_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")


def _progress(name, msg):
    """A line in gpurun_out/progress_<name>.log, so that a long run shows it is alive."""
    os.makedirs(PROGRESS_DIR, exist_ok=True)
    with open(os.path.join(PROGRESS_DIR, f"progress_{name}.log"), "a") as f:
        f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")


def _oracle_selection(p, q, k64, lengths):
    """The oracle's stages 1-3 (scores, group score, Top-K per sequence and group) on keys widened once."""
    probs = O.retrieval_scores(O.to_f64(raw(q), p.dtype), k64, lengths, p.scale)
    grp = O.group_scores(probs, p.n_groups)
    return O.select_all(grp, lengths, p.budget), grp


def _run_and_check(p, steps, layer_chunks=4, seed=0, delay_cycles=0, check_layers=None, attend_every=1,
                   name=None):
    w = W.generate(p, device="cuda", seed=seed, steps=steps, pin_host=True)
    dec = SparseDecoder(p, w.dlm_k, w.host_kv, layer_chunks=layer_chunks)
    if delay_cycles:
        # hold back every copy (main stream) and every side-stream attention by a spin, so a
        # missing wait between them shows up as a wrong output in this or the next step
        copy_chunk, attend_chunk = dec.copy_chunk, dec.attend_chunk

        def slow_copy(c):
            torch.cuda._sleep(delay_cycles)
            copy_chunk(c)

        def slow_attend(q, c, stream=None, mark=None):
            with torch.cuda.stream(stream if stream is not None else dec.main):
                torch.cuda._sleep(delay_cycles)
            attend_chunk(q, c, stream, mark)

        dec.copy_chunk, dec.attend_chunk = slow_copy, slow_attend
    ora = OracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale, p.dtype)
    lens_dev = dev_lengths(w.lengths)
    k64, kv_raw = O.to_f64(raw(w.dlm_k), p.dtype), raw(w.host_kv)
    layers = list(range(p.n_layers)) if check_layers is None else check_layers
    outs, overlaps = [], []
    prev = None
    for t in range(steps):
        q = w.q[t].contiguous()
        dec.step(q, lens_dev[t])
        torch.cuda.synchronize()
        lengths = w.lengths[t]
        # selection against the fp64 oracle chain (near-ties only)
        ref_sel, ref_grp = _oracle_selection(p, q, k64, lengths)
        gsel = sel_lists(dec.sel_idx, dec.sel_count)
        check_topk_tolerance(gsel, ref_sel, ref_grp, p.budget)
        # plan: bit-exact against the oracle plan fed the GPU's selection
        plans = ora.plan(gsel)
        lp, ls, lc = dec.load_pos.cpu().numpy(), dec.load_slot.cpu().numpy(), dec.load_count.cpu().numpy()
        sp = dec.slot_pos.cpu().numpy()
        for b in range(p.batch):
            for g in range(p.n_groups):
                to_load, lslot = plans[b][g]
                assert lc[b, g] == len(to_load)
                np.testing.assert_array_equal(lp[b, g, :lc[b, g]], to_load)
                np.testing.assert_array_equal(ls[b, g, :lc[b, g]], lslot)
                np.testing.assert_array_equal(sp[b, g], ora.slot_pos[b][g])
        # attention: the oracle reads the host store by position
        if t % attend_every == 0 or t == steps - 1:
            ref = ora.attend(raw(q), kv_raw, gsel, layers)
            got = dec.out.cpu().numpy().astype(np.float64)[:, layers]
            err = float(np.max(np.abs(got - ref)))
            assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, (t, err)
            outs.append(got)
        if name and t % 8 == 7:
            _progress(name, f"step {t + 1}/{steps} checked")
        if prev is not None:
            overlaps.append(np.mean([O.overlap(prev[b][g], gsel[b][g]) for b in range(p.batch)
                                     for g in range(p.n_groups)]))
        prev = gsel
    return outs, overlaps


def test_tiny_steps_match_oracle():
    _, ovl = _run_and_check(W.PRESETS["tiny"], steps=8, layer_chunks=1)
    assert 0.75 <= np.mean(ovl) <= 0.95


def test_gqa_multi_layer_chunks_and_ragged_batch():
    p = W.PRESETS["b16_grow"].with_(batch=3, n_layers=6, max_len=3000, budget=256, start_len=1000,
                                    offset_max=1500)
    _run_and_check(p, steps=6, layer_chunks=3)


def test_side_stream_delay_does_not_change_results():
    """Hazard test: every copy and every side-stream attention is held back by a spin each step;
    the events between the streams must keep the outputs identical."""
    p = W.PRESETS["b1_32k"].with_(max_len=4096, budget=512, n_layers=8)
    a, _ = _run_and_check(p, steps=4, layer_chunks=4, seed=3)
    b, _ = _run_and_check(p, steps=4, layer_chunks=4, seed=3, delay_cycles=2_000_000)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_batch_level_retrieval_steps():
    """One selection per sequence shared by all 32 query heads (8 KV heads): the comparison the pages
    draw against head-level retrieval.  Group max over every head, one slot map copied into every
    KV head's slots, attention of every head over it."""
    p = W.PRESETS["b1_32k"].with_(kind="mqa", max_len=4096, budget=512, n_layers=6, batch=2)
    _, ovl = _run_and_check(p, steps=4, layer_chunks=2, seed=5)
    assert np.mean(ovl) > 0.5


def test_llama8b_32k_full_size_all_64_steps():
    """The Llama3.1-8B-shaped 32K step at full size (4.29 GB pinned host K/V): all 64 correlated steps,
    every step's selection against the fp64 oracle chain and its plan bit-exact from the GPU's own
    slot maps carried step to step; attention of layers 0, 13 and 31 against the oracle every step."""
    p = W.PRESETS["b1_32k"]
    _, ovl = _run_and_check(p, steps=p.steps, layer_chunks=2, check_layers=[0, 13, 31], name="b1_32k")
    assert len(ovl) == p.steps - 1 and np.mean(ovl) > 0.7


def test_batch_level_retrieval_32k_full_shape():
    """Batch-level retrieval at the full 32K shape: one selection of 2048 positions per step shared by
    the 32 query heads of all 8 KV heads."""
    p = W.PRESETS["b1_32k"].with_(kind="mqa")
    _, ovl = _run_and_check(p, steps=4, layer_chunks=2, check_layers=[0, 31], name="b1_32k_batch")
    assert np.mean(ovl) > 0.5


def _growth_checked_steps(n_steps):
    """Steps 0..63, 16 steps spread over the rest of the schedule, and the last 8."""
    first = list(range(64))
    mid = [int(round(x)) for x in np.linspace(64, n_steps - 9, 16)]
    last = list(range(n_steps - 8, n_steps))
    return sorted(set(first + mid + last))


def test_batch16_growth_full_schedule():
    """Batch 16, 32 layers, ragged lengths growing by one token per step from 2048 + U{0..2047} to 16384,
    budget 1024, 34.4 GB pinned host K/V: the GPU runs all 14 336 steps of the schedule with its own
    state chained from step to step.  At steps 0-63, 16 sampled steps and the last 8: the selection
    against the fp64 oracle chain; the plan bit-exact against the oracle's plan fed the GPU's slot
    map of step t-1; attention of layers 0 and 31 against the oracle at every 8th of the first 64,
    at the sampled steps and at the last steps."""
    p = W.PRESETS["b16_grow"]
    w = W.generate(p, device="cuda", seed=0, pin_host=True)
    n_steps = p.steps
    assert w.lengths.shape[0] == n_steps == 14336
    assert len(set(w.lengths[0].tolist())) > 8 and np.all(w.lengths[-1] == 16384)
    dec = SparseDecoder(p, w.dlm_k, w.host_kv, layer_chunks=2)
    ora = OracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale, p.dtype)
    lens_dev = dev_lengths(w.lengths)
    k64, kv_raw = O.to_f64(raw(w.dlm_k), p.dtype), raw(w.host_kv)
    checked = set(_growth_checked_steps(n_steps))
    attend_at = {t for t in checked if t >= 64 or t % 8 == 0}
    loads = {}
    t_start = time.time()
    for t in range(n_steps):
        if t in checked:
            torch.cuda.synchronize()
            slot_before = dec.slot_pos.cpu().numpy().astype(np.int64)
        q = w.q[t].contiguous()
        dec.step(q, lens_dev[t])
        if t % 512 == 511:
            torch.cuda.synchronize()
            _progress("b16_grow", f"step {t + 1}/{n_steps}, {time.time() - t_start:.0f} s")
        if t not in checked:
            continue
        torch.cuda.synchronize()
        lengths = w.lengths[t]
        ref_sel, ref_grp = _oracle_selection(p, q, k64, lengths)
        gsel = sel_lists(dec.sel_idx, dec.sel_count)
        check_topk_tolerance(gsel, ref_sel, ref_grp, p.budget)
        lp, ls, lc = dec.load_pos.cpu().numpy(), dec.load_slot.cpu().numpy(), dec.load_count.cpu().numpy()
        sp = dec.slot_pos.cpu().numpy()
        for b in range(p.batch):
            for g in range(p.n_groups):
                to_load, lslot, new = O.elastic_plan(gsel[b][g], slot_before[b, g])
                assert lc[b, g] == len(to_load), (t, b, g)
                np.testing.assert_array_equal(lp[b, g, :lc[b, g]], to_load)
                np.testing.assert_array_equal(ls[b, g, :lc[b, g]], lslot)
                np.testing.assert_array_equal(sp[b, g], new)
        loads[t] = int(lc.sum())
        if t in attend_at:
            ref = ora.attend(raw(q), kv_raw, gsel, [0, 31])
            got = dec.out.cpu().numpy().astype(np.float64)[:, [0, 31]]
            err = float(np.max(np.abs(got - ref)))
            assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, (t, err)
    _progress("b16_grow", f"done in {time.time() - t_start:.0f} s")
    # the cold first step loads the whole budget; steady steps load part of it
    assert loads[0] == p.batch * p.n_groups * p.budget
    assert max(v for t, v in loads.items() if t > 0) < loads[0]


def test_mha_64k_full_shape_16_steps():
    """MHA: 32 q-heads = 32 KV heads, 65536 positions, budget 4096 per head (Top-K streamed from
    global memory), 2 sequences, 16 correlated steps with the GPU's state chained."""
    p = W.PRESETS["mha_64k"]
    _, ovl = _run_and_check(p, steps=16, layer_chunks=1, check_layers=[0], name="mha_64k")
    assert np.mean(ovl) > 0.6
