"""Pins of the oracle's chaining code: the functions that compose the pinned stage
definitions into decode steps (OracleDecoder, LagOneOracleDecoder, select_all) and the
per-head key expansion of MLA (mla_expand_keys).

Like tests/pins.py, each check takes what it pins as an argument, so the same check runs
against the real oracle (test_oracle_chain.py) and against copies with a planted mistake,
which must fail.  The sources of truth, none of them the chaining code retyped:
  * the library's dense attention (torch scaled_dot_product_attention, float64, CPU) with a
    boolean mask per query head and the library's GQA head map (enable_gqa);
  * the pages' worked example of elastic loading (tests/golden/elastic_worked_example.json)
    and its run through the pipelined loop (tests/golden/elastic_lag1_example.json), driven
    through the decoders from keys and queries built so that the retrieval head selects
    exactly those positions;
  * brute force on tiny ragged inputs (the unique set whose members all beat every
    non-member under (score desc, index asc), within each sequence's own length);
  * brute-force integer sums for the MLA key expansion;
  * the stage functions pinned in tests/pins.py, composed by hand step after step.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _masked_sdpa(q, K, V, mask):
    """Library attention, float64 CPU: q [B][Hq][d], K/V [B][Hkv][L][*], mask [B][Hq][L] bool.
    Query head i reads KV head i // (Hq / Hkv) (enable_gqa).  Returns [B][Hq][dv]."""
    qt = torch.from_numpy(np.ascontiguousarray(q[:, :, None, :])).to(torch.float64)
    kt = torch.from_numpy(np.ascontiguousarray(K)).to(torch.float64)
    vt = torch.from_numpy(np.ascontiguousarray(V)).to(torch.float64)
    mt = torch.from_numpy(np.ascontiguousarray(mask[:, :, None, :]))
    scale = 1.0 / math.sqrt(q.shape[-1])
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, enable_gqa=True, scale=scale).numpy()[:, :, 0]


# ----------------------------------------------------------------------------- decoder attention

def check_decoder_attend_vs_library(make_decoder):
    """OracleDecoder.attend against masked library attention on a host store whose K and V rows
    differ, for groups of 1 (one selection for every head), H_kv (GQA) and H_q (per head), over
    a layer list that is neither complete nor in order.  Empty selections give zeros."""
    rng = np.random.default_rng(31)
    B, n_layers, Hq, Hkv, L, d = 2, 3, 4, 2, 12, 8
    host_kv = rng.standard_normal((B, n_layers, Hkv, L, 2, d))
    q = rng.standard_normal((B, Hq, d)) * 1.5
    layers = [2, 0]
    for G in (1, Hkv, Hq):
        dec = make_decoder(B, Hq, Hkv, G, d, 5, 1.0 / math.sqrt(d), "f64")
        sel = [[np.sort(rng.choice(L, size=int(rng.integers(1, 6)), replace=False)) for _ in range(G)]
               for _ in range(B)]
        sel[1][G - 1] = np.zeros(0, dtype=np.int64)                      # one empty selection
        out = dec.attend(q, host_kv, sel, layers)
        assert out.shape == (B, len(layers), Hq, d)
        mask = np.zeros((B, Hq, L), dtype=bool)
        for b in range(B):
            for i in range(Hq):
                mask[b, i, sel[b][i // (Hq // G)]] = True
        for li, layer in enumerate(layers):
            ref = _masked_sdpa(q, host_kv[:, layer, :, :, 0, :], host_kv[:, layer, :, :, 1, :], mask)
            for b in range(B):
                for i in range(Hq):
                    if mask[b, i].any():
                        np.testing.assert_allclose(out[b, li, i], ref[b, i], rtol=1e-12, atol=1e-13)
                    else:
                        assert np.all(out[b, li, i] == 0.0)


# ----------------------------------------------------------------------------- the pages' example through a decoder

def _worked_example_inputs():
    """One head over 64 positions (d = 4): positions 1, 8, 21 score 10 at every step; 35 scores 10
    under q0 and 0 under q1; 50 the reverse; every other position scores -1.  With K = 4 the
    retrieval head selects S_last = {1, 8, 21, 35} from q0 and S_now = {1, 8, 21, 50} from q1."""
    ex = json.load(open(os.path.join(GOLDEN, "elastic_worked_example.json")))
    L, d = 64, 4
    e0, e1 = np.eye(d)[0], np.eye(d)[1]
    k = np.tile(-e0, (L, 1))
    common = set(ex["S_last"]) & set(ex["S_now"])
    (left,) = set(ex["S_last"]) - common
    (came,) = set(ex["S_now"]) - common
    for j in common:
        k[j] = 10 * e0
    k[left] = 5 * e0 + 5 * e1
    k[came] = 5 * e0 - 5 * e1
    q0, q1 = e0 + e1, e0 - e1
    return ex, k[None, None], [q0[None, None], q1[None, None], q1[None, None]]


def check_decoder_step_worked_example(make_decoder):
    """The pages' example through OracleDecoder.step: a cold step loads S_last into slots 0..3;
    the next step loads only the new position, into the slot of the one that left; repeating
    the selection loads nothing.  Attention of each step is over that step's selection."""
    ex, dlm_k, qs = _worked_example_inputs()
    L, d = dlm_k.shape[2], dlm_k.shape[3]
    rng = np.random.default_rng(32)
    host_kv = rng.standard_normal((1, 1, 1, L, 2, d))
    dec = make_decoder(1, 1, 1, 1, d, 4, 1.0 / math.sqrt(d), "f64")
    r0 = dec.step(qs[0], dlm_k, [L], host_kv, [0])
    assert list(r0["sel"][0][0]) == ex["S_last"]
    to_load, load_slot = r0["plans"][0][0]
    assert list(to_load) == ex["S_last"] and list(load_slot) == [0, 1, 2, 3]
    r1 = dec.step(qs[1], dlm_k, [L], host_kv, [0])
    assert list(r1["sel"][0][0]) == ex["S_now"]
    to_load, load_slot = r1["plans"][0][0]
    assert list(to_load) == ex["to_load"]
    for old, new in ex["replaced"]:
        assert list(load_slot) == [ex["S_last"].index(old)]
        assert dec.slot_pos[0][0][ex["S_last"].index(old)] == new
    assert r1["overlap"] == [[0.75]]
    r2 = dec.step(qs[2], dlm_k, [L], host_kv, [0])
    assert len(r2["plans"][0][0][0]) == 0 and r2["overlap"] == [[1.0]]
    for r, S, q in ((r0, ex["S_last"], qs[0]), (r1, ex["S_now"], qs[1])):
        mask = np.zeros((1, 1, L), dtype=bool)
        mask[0, 0, S] = True
        ref = _masked_sdpa(q, host_kv[:, 0, :, :, 0, :], host_kv[:, 0, :, :, 1, :], mask)
        np.testing.assert_allclose(r["out"][0, 0], ref[0], rtol=1e-12, atol=1e-13)


def check_lag1_decoder_worked_example(make_lag1_decoder):
    """The pages' example through LagOneOracleDecoder.plan_lag1 with a pool of 5: the warm-up step
    has no previous selection and serves its own (loaded cold into slots 0..3); then the two steps
    of tests/golden/elastic_lag1_example.json follow, each attending the previous step's selection."""
    g = json.load(open(os.path.join(GOLDEN, "elastic_lag1_example.json")))
    S0, S1 = g["steps"][0]["current"], g["steps"][0]["next"]
    dec = make_lag1_decoder(1, 1, 1, 1, 4, 4, 0.5, "f64", 5)
    plans, cur = dec.plan_lag1([[np.asarray(S0)]])
    to_load, load_slot, attend = plans[0][0]
    assert list(cur[0][0]) == S0
    assert list(to_load) == S0 and list(load_slot) == [0, 1, 2, 3] and list(attend) == [0, 1, 2, 3]
    assert list(dec.slot_pos[0][0]) == g["steps"][0]["slot_pos"]
    for st, nxt in zip(g["steps"], (S1, S1)):
        assert list(dec.slot_pos[0][0]) == st["slot_pos"]
        plans, cur = dec.plan_lag1([[np.asarray(nxt)]])
        to_load, load_slot, attend = plans[0][0]
        assert list(cur[0][0]) == st["current"]
        assert list(to_load) == st["to_load"] and list(load_slot) == st["load_slot"]
        assert list(attend) == st["attend_slots"]
        assert list(dec.slot_pos[0][0]) == st["new_slot_pos"]


# ----------------------------------------------------------------------------- ragged selection

def check_select_all_ragged(select_all):
    """Every (sequence, group) selects within its own length: the unique set of min(K, n_b)
    positions of [0, n_b) whose members all beat every non-member under (score desc, index asc),
    ascending.  Scores past a sequence's length are large, so reading them would show."""
    rng = np.random.default_rng(33)
    B, G, L = 5, 3, 9
    for trial in range(60):
        lengths = [9, 0, 5, 1, int(rng.integers(0, L + 1))]
        K = int(rng.integers(1, 7))
        if trial % 2:
            grp = rng.choice([0.0, 0.25, 0.5], size=(B, G, L))
        else:
            grp = rng.random((B, G, L))
        for b in range(B):
            grp[b, :, lengths[b]:] = 10.0 + rng.random((G, L - lengths[b]))
        sel = select_all(grp, lengths, K)
        assert len(sel) == B and all(len(row) == G for row in sel)
        for b in range(B):
            n = lengths[b]
            for r in range(G):
                s = grp[b, r]
                got = [int(x) for x in sel[b][r]]
                assert got == sorted(got) and len(got) == min(K, n)
                for j in got:
                    assert 0 <= j < n
                    for x in range(n):
                        if x not in got:
                            assert s[j] > s[x] or (s[j] == s[x] and j < x)


# ----------------------------------------------------------------------------- whole steps vs a hand composition

def check_decoder_matches_stage_composition(make_decoder, O):
    """Three steps of OracleDecoder.step on ragged, growing sequences (GQA, one group for all
    heads, and per-head groups) against the pinned stage functions composed by hand: scores ->
    group scores -> Top-K per (sequence, group) within its length -> plan with the slot maps
    carried from step to step -> attention of every listed layer over the selection, K and V
    taken from the host store's two halves."""
    rng = np.random.default_rng(34)
    B, n_layers, Hq, Hkv, L, d, K = 3, 2, 4, 2, 20, 8, 5
    dlm_k = rng.standard_normal((B, Hkv, L, d))
    host_kv = rng.standard_normal((B, n_layers, Hkv, L, 2, d))
    scale = 1.0 / math.sqrt(d)
    for G in (Hkv, 1, Hq):
        dec = make_decoder(B, Hq, Hkv, G, d, K, scale, "f64")
        slots = [[np.full(K, -1, dtype=np.int64) for _ in range(G)] for _ in range(B)]
        lengths = np.array([20, 3, 11])
        for t in range(3):
            q = rng.standard_normal((B, Hq, d)) * 2
            res = dec.step(q, dlm_k, list(lengths), host_kv, [1, 0])
            probs = O.retrieval_scores(q, dlm_k, lengths, scale)
            grp = O.group_scores(probs, G)
            for b in range(B):
                for r in range(G):
                    S = O.topk_select(grp[b, r], lengths[b], K)
                    np.testing.assert_array_equal(res["sel"][b][r], S)
                    to_load, load_slot, slots[b][r] = O.elastic_plan(S, slots[b][r])
                    np.testing.assert_array_equal(res["plans"][b][r][0], to_load)
                    np.testing.assert_array_equal(res["plans"][b][r][1], load_slot)
                    np.testing.assert_array_equal(dec.slot_pos[b][r], slots[b][r])
            for li, layer in enumerate([1, 0]):
                ref = O.sparse_decode_layer(q, host_kv[:, layer, :, :, 0, :], host_kv[:, layer, :, :, 1, :],
                                            res["sel"], G, scale)
                np.testing.assert_allclose(res["out"][:, li], ref, rtol=1e-12, atol=1e-13)
            lengths = np.minimum(lengths + np.array([0, 2, 1]), L)


# ----------------------------------------------------------------------------- MLA key expansion

def check_mla_expand_keys_exact(mla_expand_keys):
    """Integer latent rows and sparse integer weights: K_h[j] = (W_UK[h] c_j) || r_j equals a
    brute-force integer sum per head and dimension, the rotary dims copied, every head its own."""
    rng = np.random.default_rng(35)
    H, n, C, dn, R = 3, 6, 32, 5, 4
    lat = rng.integers(-3, 4, (n, C))
    rope = rng.integers(-9, 10, (n, R)) / 8.0
    W_UK = np.zeros((H, dn, C), dtype=np.int64)
    for h in range(H):
        for r in range(dn):
            cols = rng.choice(C, 4, replace=False)
            W_UK[h, r, cols] = rng.integers(-3, 4, 4)
    keys = mla_expand_keys(lat.astype(np.float64), rope, W_UK.astype(np.float64))
    assert keys.shape == (H, n, dn + R)
    for h in range(H):
        for j in range(n):
            for r in range(dn):
                assert keys[h, j, r] == sum(int(lat[j, c]) * int(W_UK[h, r, c]) for c in range(C))
            np.testing.assert_array_equal(keys[h, j, dn:], rope[j])


def check_mla_expand_keys_match_rows(mla_expand_keys, mla_expand_rows):
    """Per head, the keys equal the key half of the literal row expansion (itself pinned by
    brute-force integer sums) on random real data."""
    rng = np.random.default_rng(36)
    H, n, C, dn, dv, R = 4, 9, 16, 6, 5, 3
    lat, rope = rng.standard_normal((n, C)), rng.standard_normal((n, R))
    W_UK, W_UV = rng.standard_normal((H, dn, C)), rng.standard_normal((H, dv, C))
    keys = mla_expand_keys(lat, rope, W_UK)
    for h in range(H):
        Kh, _ = mla_expand_rows(lat, rope, W_UK[h], W_UV[h])
        np.testing.assert_allclose(keys[h], Kh, rtol=1e-13, atol=1e-13)

