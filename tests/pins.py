"""Checks that pin the CPU oracle to facts fixed outside of it.

Each check takes the oracle function it pins as an argument, so the same check
runs against the real oracle (test_oracle_pins.py) and against deliberately
broken copies of it (test_oracle_mutations.py), which must fail.

Sources of truth used here, none of them the oracle's own formula retyped:
  * closed forms (two- and three-position softmax with known dot products);
  * special cases that reduce to an independent library routine:
    torch.nn.functional.scaled_dot_product_attention in float64 on the CPU
    (with V = I it returns the attention weights themselves; with a boolean
    mask it is attention over a subset; enable_gqa gives the GQA head map);
  * brute force on tiny inputs (all subsets for Top-K);
  * the pages' worked example (tests/golden/elastic_worked_example.json);
  * invariants the pages state (set difference plus reused slots = new
    selection, in-place loads within a fixed budget, K = L gives full
    attention, GQA group max = max of per-head results).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _sdpa(q, k, v, mask=None, gqa=False, scale=None):
    """Library attention in float64 on the CPU: q [B][Hq][1][d], k/v [B][Hkv][n][*]."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, enable_gqa=gqa, scale=scale).numpy()


# ----------------------------------------------------------------------------- O1 scores

def check_scores_closed_form(retrieval_scores):
    d = 128
    a, b = 3.0, 5.0
    q = np.zeros((1, 1, d)); q[0, 0, 0] = a
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = b            # position 1 is the zero key
    p = retrieval_scores(q, k, [2], 1.0 / math.sqrt(d))
    x = a * b / math.sqrt(d)
    assert abs(p[0, 0, 0] - 1.0 / (1.0 + math.exp(-x))) < 1e-12
    assert abs(p[0, 0, 1] - 1.0 / (1.0 + math.exp(x))) < 1e-12
    # three positions with logits x, 0, -x
    k3 = np.zeros((1, 1, 3, d)); k3[0, 0, 0, 0] = b; k3[0, 0, 2, 0] = -b
    p3 = retrieval_scores(q, k3, [3], 1.0 / math.sqrt(d))
    z = math.exp(x) + 1.0 + math.exp(-x)
    np.testing.assert_allclose(p3[0, 0, :3], [math.exp(x) / z, 1.0 / z, math.exp(-x) / z], rtol=1e-12)


def check_scores_zero_query_uniform(retrieval_scores):
    rng = np.random.default_rng(1)
    k = rng.standard_normal((2, 2, 37, 16))
    q = np.zeros((2, 4, 16))
    p = retrieval_scores(q, k, [37, 10], 0.25)
    np.testing.assert_allclose(p[0, :, :37], 1.0 / 37, rtol=1e-12)
    np.testing.assert_allclose(p[1, :, :10], 1.0 / 10, rtol=1e-12)
    assert np.all(p[1, :, 10:] == 0)


def check_scores_length_masking(retrieval_scores):
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 16))
    k = rng.standard_normal((1, 2, 50, 16))
    p1 = retrieval_scores(q, k, [23], 0.25)
    k2 = k.copy(); k2[:, :, 23:] = 100.0 * rng.standard_normal(k2[:, :, 23:].shape)
    p2 = retrieval_scores(q, k2, [23], 0.25)
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_allclose(p1[0, :, :23].sum(axis=-1), 1.0, rtol=1e-12)
    assert np.all(p1[0, :, 23:] == 0)


def check_scores_vs_library(retrieval_scores):
    """softmax(q K^T/sqrt(d)) = SDPA(q, K, V=I); GQA head map = library's enable_gqa."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, n, d = 2, 8, 2, 19, 32
    q = rng.standard_normal((B, Hq, d)) * 2
    k = rng.standard_normal((B, Hkv, n, d))
    p = retrieval_scores(q, k, [n, n], 1.0 / math.sqrt(d))
    eye = np.broadcast_to(np.eye(n), (B, Hkv, n, n))
    ref = _sdpa(q[:, :, None, :], k, eye, gqa=True)[:, :, 0, :]
    np.testing.assert_allclose(p[:, :, :n], ref, rtol=1e-10, atol=1e-14)


# ----------------------------------------------------------------------------- O2 group max

def check_group_max_is_max_of_per_head(retrieval_scores, group_scores):
    """GQA group score = element-wise max of the per-head weights, each head scored alone."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, L, d = 2, 8, 2, 40, 16
    q = rng.standard_normal((B, Hq, d)) * 3
    k = rng.standard_normal((B, Hkv, L, d))
    lens = [40, 29]
    grp = group_scores(retrieval_scores(q, k, lens, 0.3), Hkv)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            per_head = [retrieval_scores(q[b:b + 1, i:i + 1], k[b:b + 1, g:g + 1], [lens[b]], 0.3)[0, 0]
                        for i in range(g * G, (g + 1) * G)]
            np.testing.assert_array_equal(grp[b, g], np.maximum.reduce(per_head))


def check_group_modes(group_scores):
    rng = np.random.default_rng(5)
    p = rng.random((1, 6, 11))
    # MHA: groups of one head are the heads themselves
    np.testing.assert_array_equal(group_scores(p, 6), p)
    # MQA: one group, the max over every head
    np.testing.assert_array_equal(group_scores(p, 1)[0, 0], p[0].max(axis=0))
    # identical heads in a group equal one head
    same = np.repeat(p[:, :1], 3, axis=1)
    np.testing.assert_array_equal(group_scores(same, 1)[0, 0], p[0, 0])


# ----------------------------------------------------------------------------- O3 Top-K

def _dominates(s, i, j):
    return s[i] > s[j] or (s[i] == s[j] and i < j)


def check_topk_bruteforce(topk_select):
    """Exhaustive over subsets: the selection is the unique set whose members all
    beat every non-member under (score desc, index asc)."""
    rng = np.random.default_rng(6)
    for trial in range(300):
        n = int(rng.integers(0, 9))
        k = int(rng.integers(1, 11))
        if trial % 2:
            s = rng.choice([0.0, 0.25, 0.5], size=max(n, 1))
        else:
            s = rng.random(max(n, 1))
        m = min(k, n)
        valid = [set(c) for c in itertools.combinations(range(n), m)
                 if all(_dominates(s, i, j) for i in c for j in range(n) if j not in c)]
        assert len(valid) == 1
        got = topk_select(s, n, k)
        assert list(got) == sorted(valid[0])


def check_topk_python_sorted(topk_select):
    rng = np.random.default_rng(7)
    for trial in range(50):
        n = int(rng.integers(1, 400))
        k = int(rng.integers(1, 64))
        s = rng.choice(np.linspace(0, 1, 7), size=n) if trial % 2 else rng.random(n)
        ref = sorted(sorted(range(n), key=lambda j: (-s[j], j))[:k])
        assert list(topk_select(s, n, k)) == ref


def check_topk_edge_cases(topk_select):
    assert list(topk_select(np.full(10, 0.5), 10, 4)) == [0, 1, 2, 3]          # all equal: lowest indices
    assert list(topk_select(np.arange(5.0), 5, 9)) == [0, 1, 2, 3, 4]         # K >= n: everything
    assert len(topk_select(np.arange(5.0), 0, 3)) == 0                         # n = 0: nothing
    assert list(topk_select(np.array([0.1, 0.9, 0.5, 0.9]), 3, 2)) == [1, 2]   # only j < n counts
    # -0.0 and +0.0 are one value: a tie, broken by the lower index (not +0 above -0)
    assert list(topk_select(np.array([0.0, -0.0, -0.0, 0.0]), 4, 2)) == [0, 1]
    assert list(topk_select(np.array([-1.0, -0.0, 0.0, -2.0]), 4, 1)) == [1]


# ----------------------------------------------------------------------------- O4 plan

def check_plan_worked_example(elastic_plan):
    ex = json.load(open(os.path.join(GOLDEN, "elastic_worked_example.json")))
    slot_pos = np.array(ex["S_last"])
    to_load, load_slot, new = elastic_plan(ex["S_now"], slot_pos)
    assert list(to_load) == ex["to_load"]
    for old, nw in ex["replaced"]:
        x = list(slot_pos).index(old)
        assert list(load_slot) == [x] and new[x] == nw
    assert sorted(p for p in new if p != -1) == sorted(ex["S_now"])
    for x, p in enumerate(slot_pos):                     # kept positions do not move
        if p in ex["S_now"]:
            assert new[x] == p


def _check_plan_invariants(S_now, slot_before, to_load, load_slot, new):
    S_now = set(int(x) for x in S_now)
    S_last = set(int(p) for p in slot_before if p != -1)
    kept = S_now & S_last
    assert set(int(x) for x in to_load).isdisjoint(kept)
    assert set(int(x) for x in to_load) | kept == S_now                       # difference + reused = new
    assert len(to_load) == len(S_now - S_last)
    assert set(int(p) for p in new if p != -1) == S_now                        # resident = selected
    assert len(new) == len(slot_before)                                        # fixed budget
    for x, p in enumerate(slot_before):                                        # in place: kept stay
        if p != -1 and p in S_now:
            assert new[x] == p
    for pos, x in zip(to_load, load_slot):                                     # loads go to freed slots
        assert slot_before[x] == -1 or slot_before[x] not in S_now
        assert new[x] == pos
    assert list(to_load) == sorted(to_load)
    assert list(load_slot) == sorted(load_slot)


def check_plan_invariants(elastic_plan):
    rng = np.random.default_rng(8)
    K, L = 16, 64
    for trial in range(40):
        slot_pos = np.full(K, -1)
        S_prev = set()
        for step in range(12):
            n = int(rng.integers(0, L + 1))
            keep = [p for p in S_prev if p < n and rng.random() < 0.8]
            pool = [p for p in range(n) if p not in keep]
            m = min(K, n) - len(keep)
            S_now = set(keep) | set(rng.choice(pool, size=max(m, 0), replace=False).tolist()) if n else set()
            to_load, load_slot, new = elastic_plan(sorted(S_now), slot_pos)
            _check_plan_invariants(sorted(S_now), slot_pos, to_load, load_slot, new)
            slot_pos, S_prev = np.asarray(new), S_now


def check_plan_cold_repeat_growth(elastic_plan):
    K = 8
    S = [3, 5, 9, 10, 20]
    to_load, load_slot, new = elastic_plan(S, np.full(K, -1))                 # cold start
    assert list(to_load) == S and list(load_slot) == [0, 1, 2, 3, 4]
    assert list(new) == S + [-1, -1, -1]
    t2, s2, new2 = elastic_plan(S, new)                                        # repeated plan is empty
    assert len(t2) == 0 and len(s2) == 0 and list(new2) == list(new)
    # growth with K >= n: each step exactly the new position loads
    slot_pos = np.full(K, -1)
    for n in range(1, K + 1):
        t, s, slot_pos = elastic_plan(list(range(n)), slot_pos)
        assert list(t) == [n - 1]
    assert list(slot_pos) == list(range(K))


# ----------------------------------------------------------------------------- O5 copy

def check_copy(elastic_copy, elastic_plan):
    rng = np.random.default_rng(9)
    host = rng.integers(0, 2 ** 16, size=(50, 2, 8), dtype=np.uint16)
    dev = np.zeros((6, 2, 8), dtype=np.uint16)
    slot_pos = np.full(6, -1)
    for S in ([1, 4, 7], [1, 7, 30, 31, 49], [0, 30, 31, 32, 33, 49]):
        to_load, load_slot, slot_pos = elastic_plan(S, slot_pos)
        elastic_copy(host, dev, to_load, load_slot)
        for x, p in enumerate(slot_pos):
            if p != -1:
                np.testing.assert_array_equal(dev[x], host[p])


# ----------------------------------------------------------------------------- O6 attention

def check_attention_full_budget(topk_select, sparse_decode_layer):
    """K >= n reproduces dense attention (library SDPA) over all n positions."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, n, d = 2, 8, 2, 33, 16
    q = rng.standard_normal((B, Hq, d)) * 2
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    sel = [[topk_select(rng.random(n), n, 64) for _ in range(Hkv)] for _ in range(B)]
    out = sparse_decode_layer(q, K, V, sel, Hkv, 1.0 / math.sqrt(d))
    ref = _sdpa(q[:, :, None, :], K, V, gqa=True)[:, :, 0, :]
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def check_attention_subset_vs_masked_library(sparse_attention):
    rng = np.random.default_rng(11)
    n, d = 40, 16
    for _ in range(10):
        q = rng.standard_normal(d) * 2
        K = rng.standard_normal((n, d)); V = rng.standard_normal((n, 24))
        S = np.sort(rng.choice(n, size=int(rng.integers(1, n)), replace=False))
        mask = np.zeros((1, 1, 1, n), dtype=bool); mask[..., S] = True
        ref = _sdpa(q[None, None, None], K[None, None], V[None, None], mask=mask, scale=0.3)[0, 0, 0]
        np.testing.assert_allclose(sparse_attention(q, K, V, S, 0.3), ref, rtol=1e-10, atol=1e-12)
        perm = rng.permutation(S)                           # order of the rows does not matter
        np.testing.assert_allclose(sparse_attention(q, K, V, perm, 0.3), ref, rtol=1e-10, atol=1e-12)


def check_attention_special_cases(sparse_attention):
    rng = np.random.default_rng(12)
    K = rng.standard_normal((30, 8)); V = rng.standard_normal((30, 8))
    q = rng.standard_normal(8)
    np.testing.assert_array_equal(sparse_attention(q, K, V, [17], 0.5), V[17])         # K = 1
    np.testing.assert_allclose(sparse_attention(np.zeros(8), K, V, [2, 5, 11], 0.5),
                               V[[2, 5, 11]].mean(axis=0), rtol=1e-12)                  # q = 0
    assert np.all(sparse_attention(q, K, V, [], 0.5) == 0)                               # empty


# ----------------------------------------------------------------------------- MLA

def check_mla_literal_vs_absorbed(mla_sparse_attention, mla_retrieval_scores):
    """Literal expansion of the selected rows equals the algebraically absorbed form."""
    rng = np.random.default_rng(13)
    H, dn, C, R, L = 3, 8, 12, 4, 30
    W_UK = rng.standard_normal((H, dn, C)) / math.sqrt(C)
    W_UV = rng.standard_normal((H, dn, C)) / math.sqrt(C)
    lat = rng.standard_normal((L, C)); rope = rng.standard_normal((L, R))
    qn = rng.standard_normal((H, dn)) * 2; qr = rng.standard_normal((H, R))
    scale = 1.0 / math.sqrt(dn + R)
    S = [1, 4, 9, 20, 29]
    for h in range(H):
        qt = W_UK[h].T @ qn[h]                                    # absorbed query (C)
        logit = (lat[S] @ qt + rope[S] @ qr[h]) * scale
        w = np.exp(logit - logit.max()); w /= w.sum()
        ref = W_UV[h] @ (w @ lat[S])
        np.testing.assert_allclose(mla_sparse_attention(qn[h], qr[h], lat, rope, W_UK, W_UV, S, h, scale),
                                   ref, rtol=1e-10, atol=1e-12)
    probs = mla_retrieval_scores(qn[None], qr[None], lat[None], rope[None], W_UK, [L], scale)
    for h in range(H):
        Kh = np.concatenate([lat @ W_UK[h].T, rope], axis=1)      # library: SDPA with V = I
        ref = _sdpa(np.concatenate([qn[h], qr[h]])[None, None, None], Kh[None, None],
                    np.eye(L)[None, None], scale=scale)[0, 0, 0]
        np.testing.assert_allclose(probs[(0, h)], ref, rtol=1e-10, atol=1e-14)


def check_round_bf16(round_bf16, to_bf16_bits):
    """Nearest bf16 with ties to even (8 significant bits): halfway cases by hand, and agreement
    with an independent bit-level rounding on float32 inputs (where rounding through float32 is
    exact, so the two must agree)."""
    u = 2.0 ** -7                                            # bf16 spacing on [1, 2)
    cases = [(1.0 + u / 2, 1.0),                             # halfway, even below
             (1.0 + 3 * u / 2, 1.0 + 2 * u),                 # halfway, even above
             (1.0 + u / 2 + 2.0 ** -20, 1.0 + u),            # just above halfway
             (-(1.0 + u / 2), -1.0), (3.0, 3.0), (0.0, 0.0),
             (255.0, 255.0), (257.0, 256.0), (259.0, 260.0),  # integers: 8 significant bits
             (2.0 ** -30 * (1 + 3 * u / 2), 2.0 ** -30 * (1 + 2 * u))]
    for x, want in cases:
        assert float(round_bf16(np.float64(x))) == want, (x, float(round_bf16(np.float64(x))), want)
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = (to_bf16_bits(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), ref)


def check_mla_expand_exact(mla_expand_rows):
    """Integer latent rows and sparse integer weights: every up-projected value is an integer of
    at most 8 significant bits, so the bf16-stored expansion is exact and equals a brute-force
    integer sum; K takes W_UK, V takes W_UV, the rotary dims are copied."""
    rng = np.random.default_rng(22)
    n, C, dn, dv, R = 7, 64, 6, 5, 4
    lat = rng.integers(-3, 4, (n, C))
    rope = rng.integers(-9, 10, (n, R)) / 8.0
    W_UK = np.zeros((dn, C), dtype=np.int64)
    W_UV = np.zeros((dv, C), dtype=np.int64)
    for W in (W_UK, W_UV):
        for r in range(W.shape[0]):
            cols = rng.choice(C, 5, replace=False)
            W[r, cols] = rng.integers(-3, 4, 5)
    K, V = mla_expand_rows(lat.astype(np.float64), rope, W_UK.astype(np.float64), W_UV.astype(np.float64), "bf16")
    for j in range(n):
        for r in range(dn):
            assert K[j, r] == sum(int(lat[j, c]) * int(W_UK[r, c]) for c in range(C))
        for r in range(dv):
            assert V[j, r] == sum(int(lat[j, c]) * int(W_UV[r, c]) for c in range(C))
        np.testing.assert_array_equal(K[j, dn:], rope[j])
    # rounding applies to the projections only: a value needing 9 bits rounds to 8
    K1, _ = mla_expand_rows(np.array([[257.0] + [0.0] * (C - 1)]), np.zeros((1, R)),
                            np.eye(dn, C), np.eye(dv, C), "bf16")
    assert K1[0, 0] == 256.0


# ----------------------------------------------------------------------------- sizes

def check_kv_cache_size(kv_cache_bytes):
    ex = json.load(open(os.path.join(GOLDEN, "kv_cache_size.json")))
    m = ex["model"]
    for pt in ex["points"]:
        gb = kv_cache_bytes(m["n_layers"], m["n_kv_heads"], m["head_dim"], m["elem_bytes"], pt["seq_len"]) / 2 ** 30
        assert abs(gb - pt["approx_gb"]) <= ex["rel_tolerance"] * pt["approx_gb"]


# ----------------------------------------------------------------------------- adaptive offloading (C3)

def check_offload_golden(offload_thresholds, offloaded_layers):
    g = json.load(open(os.path.join(GOLDEN, "offload_thresholds.json")))
    th = offload_thresholds(g["gpu_bytes"], **g["model"])
    assert list(th) == g["thresholds"]
    for L, c in g["offloaded_at"]:
        assert offloaded_layers(L, th) == c, (L, c)


def check_offload_invariants(offload_thresholds, memory_bytes):
    """Each finite threshold t is the first length that does not fit: L = t - 1 fits, t does not."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        model = dict(fixed_bytes=int(rng.integers(0, 10 ** 10)), token_bytes=int(rng.integers(0, 10 ** 5)),
                     n_layers=int(rng.integers(1, 40)), batch=int(rng.integers(1, 17)),
                     n_kv_heads=int(rng.integers(1, 9)), head_dim=128, v_dim=128,
                     budget=int(rng.integers(1, 4097)), elem_bytes=2)
        gpu = int(rng.integers(10 ** 9, 3 * 10 ** 11))
        th = offload_thresholds(gpu, **model)
        assert len(th) == model["n_layers"] + 1
        for c, t in enumerate(th):
            if t == 0:
                assert memory_bytes(0, c, **model) > gpu
            elif t < 2 ** 31 - 1:
                assert memory_bytes(t - 1, c, **model) <= gpu < memory_bytes(t, c, **model)


# ----------------------------------------------------------------------------- pipelined loop (lag 1)

def check_plan_lag1_worked_example(elastic_plan_lag1):
    g = json.load(open(os.path.join(GOLDEN, "elastic_lag1_example.json")))
    for st in g["steps"]:
        to_load, load_slot, new, attend = elastic_plan_lag1(st["current"], st["next"], st["slot_pos"])
        assert list(to_load) == st["to_load"] and list(load_slot) == st["load_slot"]
        assert list(new) == st["new_slot_pos"] and list(attend) == st["attend_slots"]


def check_plan_lag1_reduces_to_lag0(elastic_plan_lag1, elastic_plan):
    """With the same selection as current and next the pipelined plan is the plan of the blog's loop."""
    rng = np.random.default_rng(21)
    K, L = 16, 60
    slots = np.full(K, -1)
    for _ in range(20):
        S = np.sort(rng.choice(L, size=int(rng.integers(0, K + 1)), replace=False))
        a = elastic_plan(S, slots)
        b = elastic_plan_lag1(S, S, slots)
        for x, y in zip(a, b[:3]):
            np.testing.assert_array_equal(x, y)
        slots = a[2]
        np.testing.assert_array_equal(np.sort(slots[b[3]]), S)


def check_plan_lag1_invariants(elastic_plan_lag1):
    """Over random correlated sequences with a pool of twice the budget: the pool holds exactly the
    union of current and next; the current selection's slots never move while it is attended; loads
    go to slots that held neither selection; the attended slots hold exactly the current selection."""
    rng = np.random.default_rng(22)
    K, L = 12, 50
    slots = np.full(2 * K, -1)
    nxt = np.sort(rng.choice(L, size=K, replace=False))
    cur = nxt
    for _ in range(40):
        before = np.array(slots)
        to_load, load_slot, new, attend = elastic_plan_lag1(cur, nxt, before)
        U = set(cur.tolist()) | set(nxt.tolist())
        assert set(p for p in new.tolist() if p >= 0) == U
        for x, p in enumerate(before.tolist()):
            if p in set(cur.tolist()):
                assert new[x] == p
        assert not (set(to_load.tolist()) & set(p for p in before.tolist() if p >= 0))
        for x in load_slot.tolist():
            assert before[x] == -1 or before[x] not in U
        assert sorted(new[attend].tolist()) == sorted(cur.tolist())
        slots = new
        cur = nxt
        keep = rng.choice(cur, size=int(rng.integers(K // 2, K + 1)), replace=False)
        fresh = rng.choice(np.setdiff1d(np.arange(L), keep), size=K - len(keep), replace=False)
        nxt = np.sort(np.concatenate([keep, fresh]))
