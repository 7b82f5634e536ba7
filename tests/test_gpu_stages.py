"""Stage-by-stage parity of the HIP path against the CPU oracle (through the C-ABI)."""
import math

import numpy as np
import pytest
import torch

from oracle import spc_oracle as O
from speculative_kv_sparsity_amd import api
from speculative_kv_sparsity_amd import workload as W
from tests.gpu_util import (ATTN_DERIVED, ATTN_MAX_ABS, PROBS_RTOL, check_topk_tolerance, dev_lengths, f64, raw,
                            sel_lists, shape_of)

pytestmark = pytest.mark.gpu

GQA_SMALL = W.Preset("gqa_small", "gqa", batch=2, n_layers=4, n_q_heads=8, n_kv_heads=2, head_dim=128, v_dim=128,
                     dtype="bf16", max_len=1000, budget=96, steps=4)


def _scores(p, w, lengths):
    shape = shape_of(p)
    probs = torch.full((p.batch, p.n_q_heads, p.max_len), float("nan"), device="cuda")
    api.spc_retrieval_scores(shape, w.q[0].contiguous(), w.dlm_k, dev_lengths(lengths), probs)
    torch.cuda.synchronize()
    return shape, probs


SCORE_CASES = [
    ("tiny_f32", W.PRESETS["tiny"], None),
    ("gqa_ragged", GQA_SMALL, [1000, 517]),
    ("gqa_edge_lengths", GQA_SMALL.with_(batch=4), [0, 1, 255, 1000]),
    ("mha", GQA_SMALL.with_(kind="mha", n_q_heads=4, n_kv_heads=4, max_len=777), [777, 300]),
    ("mqa", GQA_SMALL.with_(kind="mqa", n_q_heads=8, n_kv_heads=1, max_len=600), [600, 599]),
    ("heads_per_kv_16", GQA_SMALL.with_(n_q_heads=32, n_kv_heads=2, max_len=513), [513, 257]),
    ("d64", GQA_SMALL.with_(head_dim=64, v_dim=64, max_len=300), [300, 3]),
    # batch-level retrieval: one selection per sequence over the heads of every KV head
    ("batch_level", GQA_SMALL.with_(kind="mqa"), [1000, 517]),
    ("batch_level_32_heads", GQA_SMALL.with_(kind="mqa", n_q_heads=32, n_kv_heads=8, max_len=1500), [1500, 1001]),
]


@pytest.mark.parametrize("name,p,lengths", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_scores_match_oracle(name, p, lengths):
    w = W.generate(p, device="cuda", seed=11, steps=1)
    lengths = list(w.lengths[0]) if lengths is None else lengths
    _, probs = _scores(p, w, lengths)
    ref = O.retrieval_scores(f64(w.q[0], p.dtype), f64(w.dlm_k, p.dtype), lengths, p.scale)
    got = probs.cpu().numpy().astype(np.float64)
    for b, n in enumerate(lengths):
        if n == 0:
            continue
        np.testing.assert_allclose(got[b, :, :n], ref[b, :, :n], rtol=PROBS_RTOL, atol=0)
        assert np.all(np.isnan(got[b, :, n:]))          # positions past the length are not written


def _topk_gpu(shape, probs, lengths):
    B, G, K = shape.batch, shape.n_groups, shape.budget
    sel_idx = torch.full((B, G, K), -7, dtype=torch.int32, device="cuda")
    sel_count = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    api.spc_group_max_topk(shape, probs, dev_lengths(lengths), sel_idx, sel_count)
    torch.cuda.synchronize()
    return sel_idx, sel_count


def _oracle_topk(probs_f64, lengths, n_groups, K):
    return O.select_all(O.group_scores(probs_f64, n_groups), lengths, K)


def _assert_sel_equal(sel_idx, sel_count, ref, K):
    si, sc = sel_idx.cpu().numpy(), sel_count.cpu().numpy()
    for b in range(len(ref)):
        for g in range(len(ref[b])):
            r = ref[b][g]
            assert sc[b, g] == len(r), (b, g)
            np.testing.assert_array_equal(si[b, g, :len(r)], r)
            assert np.all(si[b, g, len(r):] == -1)


@pytest.mark.parametrize("name,p,lengths", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_topk_exact_on_gpu_scores_and_tolerant_vs_oracle_chain(name, p, lengths):
    w = W.generate(p, device="cuda", seed=12, steps=1)
    lengths = list(w.lengths[0]) if lengths is None else lengths
    shape, probs = _scores(p, w, lengths)
    sel_idx, sel_count = _topk_gpu(shape, probs, lengths)
    # bit-exact against the oracle's Top-K run on the GPU's own float32 scores
    gp = np.nan_to_num(probs.cpu().numpy().astype(np.float64), nan=0.0)
    _assert_sel_equal(sel_idx, sel_count, _oracle_topk(gp, lengths, p.n_groups, p.budget), p.budget)
    # against the fp64 oracle chain: only near-ties may differ
    ref_probs = O.retrieval_scores(f64(w.q[0], p.dtype), f64(w.dlm_k, p.dtype), lengths, p.scale)
    ref_grp = O.group_scores(ref_probs, p.n_groups)
    ref_sel = O.select_all(ref_grp, lengths, p.budget)
    check_topk_tolerance(sel_lists(sel_idx, sel_count), ref_sel, ref_grp, p.budget)


# --------------------------------------------------------------- log-domain form of stages 1-2


def _logits(p, w, lengths, t=0):
    shape = shape_of(p)
    nan = float("nan")
    logits = torch.full((p.batch, p.n_q_heads, p.max_len), nan, device="cuda")
    stats = torch.full(api.tile_stats_shape(shape), nan, device="cuda")
    api.spc_retrieval_logits(shape, w.q[t].contiguous(), w.dlm_k, dev_lengths(lengths), logits, stats)
    torch.cuda.synchronize()
    return shape, logits, stats


def _lse(stats_bh, nt):
    """log-sum-exp of a head from its first nt tile pairs, in float64."""
    m, s = stats_bh[:nt, 0].astype(np.float64), stats_bh[:nt, 1].astype(np.float64)
    M = np.max(m)
    return M + np.log(np.sum(s * np.exp(m - M)))


@pytest.mark.parametrize("name,p,lengths", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_logits_and_tile_stats_give_the_oracle_probabilities(name, p, lengths):
    w = W.generate(p, device="cuda", seed=11, steps=1)
    lengths = list(w.lengths[0]) if lengths is None else lengths
    shape, logits, stats = _logits(p, w, lengths)
    T = api.spc_score_tile(shape)
    ref = O.retrieval_scores(f64(w.q[0], p.dtype), f64(w.dlm_k, p.dtype), lengths, p.scale)
    lg = logits.cpu().numpy()
    st = stats.cpu().numpy()
    for b, n in enumerate(lengths):
        assert np.all(np.isnan(lg[b, :, n:]))              # positions past the length are not written
        nt = (n + T - 1) // T
        assert np.all(np.isnan(st[b, :, nt:]))             # nor the tiles past it
        if n == 0:
            continue
        for i in range(p.n_q_heads):
            x = lg[b, i, :n].astype(np.float64)
            # each tile pair is the exact max and the sum of exp over the tile's own logits
            for t in range(nt):
                seg = x[t * T:min(n, (t + 1) * T)]
                assert st[b, i, t, 0] == np.max(seg)
                np.testing.assert_allclose(st[b, i, t, 1], np.sum(np.exp(seg - np.max(seg))), rtol=1e-5)
            # exp(logit - lse) are the oracle's probabilities
            pr = np.exp(x - _lse(st[b, i], nt))
            np.testing.assert_allclose(pr, ref[b, i, :n], rtol=PROBS_RTOL, atol=0)


def _topk_logits_gpu(shape, logits, stats, lengths):
    B, G, K = shape.batch, shape.n_groups, shape.budget
    sel_idx = torch.full((B, G, K), -7, dtype=torch.int32, device="cuda")
    sel_count = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    api.spc_group_max_topk_logits(shape, logits, stats, dev_lengths(lengths), sel_idx, sel_count)
    torch.cuda.synchronize()
    return sel_idx, sel_count


@pytest.mark.parametrize("name,p,lengths", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_topk_on_logits_matches_the_oracle_chain(name, p, lengths):
    w = W.generate(p, device="cuda", seed=12, steps=1)
    lengths = list(w.lengths[0]) if lengths is None else lengths
    shape, logits, stats = _logits(p, w, lengths)
    sel_idx, sel_count = _topk_logits_gpu(shape, logits, stats, lengths)
    if p.n_groups == p.n_q_heads:
        # one head per group: the GPU's float32 logits are ranked as they are (bit-exact)
        gl = np.nan_to_num(logits.cpu().numpy().astype(np.float64), nan=-np.inf)
        _assert_sel_equal(sel_idx, sel_count, _oracle_topk(gl, lengths, p.n_groups, p.budget), p.budget)
    ref_probs = O.retrieval_scores(f64(w.q[0], p.dtype), f64(w.dlm_k, p.dtype), lengths, p.scale)
    ref_grp = O.group_scores(ref_probs, p.n_groups)
    ref_sel = O.select_all(ref_grp, lengths, p.budget)
    check_topk_tolerance(sel_lists(sel_idx, sel_count), ref_sel, ref_grp, p.budget)
    # the probability path on the same inputs agrees with it up to the same near-ties
    _, probs = _scores(p, w, lengths)
    ps, pc = _topk_gpu(shape, probs, lengths)
    check_topk_tolerance(sel_lists(sel_idx, sel_count), sel_lists(ps, pc), ref_grp, p.budget)


def _host_stats(vals, T):
    """float32 tile pairs (max, sum exp) of given logits [B][H][L] (test input construction)."""
    B, H, L = vals.shape
    nt = (L + T - 1) // T
    st = np.zeros((B, H, nt, 2), dtype=np.float32)
    for t in range(nt):
        seg = vals[:, :, t * T:(t + 1) * T].astype(np.float64)
        m = seg.max(axis=2)
        st[:, :, t, 0] = m
        st[:, :, t, 1] = np.exp(seg - m[..., None]).sum(axis=2)
    return st


LOGIT_TIE_CASES = [
    # (B, Hq, G, L, K, lengths, value pool or None, same pool for every head)
    (1, 4, 1, 3000, 64, [3000], [0.125], True),                     # all equal: lowest indices win
    (2, 8, 2, 5000, 300, [5000, 4097], [-3.0, 0.0, 2.5], True),     # heavy ties inside each head
    (1, 2, 2, 40000, 2048, [40000], None, False),                   # keys streamed from global memory
    (1, 6, 2, 33000, 5000, [33000], None, False),                   # 3 heads per group, LDS limit crossed
    (3, 2, 1, 2000, 100, [100, 101, 0], None, False),               # n = K, n = K + 1, n = 0
    (2, 4, 4, 1500, 1, [1500, 7], [-1.0, 4.0], True),               # K = 1, one head per group
    # one head per group at the LDS size limit: 64 values one ulp apart (the top 24 bits of every
    # key agree, so the last radix digit decides), and the boundary inside a tie group
    (2, 4, 4, 32768, 2000, [32768, 20001], list(np.float32(1.0) + np.arange(64, dtype=np.float32)
                                                 * np.float32(2.0 ** -23)), False),
    # -0.0 and +0.0 are one value: ties broken by the lower index
    (1, 2, 2, 30000, 2048, [30000], [-0.0, 0.0, -1.0], False),
    # rows that do not start 16-byte aligned (a length no multiple of 4), one head per group
    (2, 3, 3, 4999, 100, [4999, 4998], None, False),
    # rows past the LDS stage (keys held in registers): unaligned rows, and every key equal, so the
    # threshold bin outgrows the candidate list
    (2, 3, 3, 40001, 1000, [40001, 39000], None, False),
    (1, 2, 2, 50000, 3000, [50000], [0.125], True),
    # more than 256 instances of one head each (the 512-thread register select, two workgroups per
    # CU): heavy ties; unaligned rows with n < K; every key equal in rows of 32768, so the threshold
    # bin outgrows its 4096-entry list; an empty sequence beside a full one
    (2, 136, 136, 3000, 300, [3000, 2999], [-3.0, 0.0, 2.5], False),
    (2, 130, 130, 4001, 400, [4001, 1], None, False),
    (1, 300, 300, 32768, 2048, [32768], [0.125], False),
    (2, 140, 140, 20000, 2048, [20000, 0], None, False),
]


@pytest.mark.parametrize("case", LOGIT_TIE_CASES, ids=[f"ltie{i}" for i in range(len(LOGIT_TIE_CASES))])
def test_topk_on_logits_with_ties_and_edges(case):
    B, Hq, G, L, K, lengths, pool, shared = case
    rng = np.random.default_rng(7)
    if pool is None:
        vals = (4.0 * rng.standard_normal((B, Hq, L))).astype(np.float32)
    else:
        vals = rng.choice(np.asarray(pool, dtype=np.float32), size=(B, Hq, L))
        if shared:                       # every head of a group sees the same values: equal lse
            vals[:] = vals[:, :1]
    for b, n in enumerate(lengths):
        vals[b, :, n:] = np.nan                                # never read
    shape = api.make_shape(B, Hq, G, G, 128, 128, L, K, 1, "bf16", 1.0)
    T = api.spc_score_tile(shape)
    stats = np.zeros((B, Hq, (L + T - 1) // T, 2), dtype=np.float32)
    for b, n in enumerate(lengths):
        if n:
            stats[b:b + 1, :, :(n + T - 1) // T] = _host_stats(vals[b:b + 1, :, :n], T)
    sel_idx, sel_count = _topk_logits_gpu(shape, torch.from_numpy(vals).cuda(),
                                          torch.from_numpy(stats).cuda() if Hq > G else None, lengths)
    # fp64 reference: the probabilities exp(l - lse) of the same logits, group max, Top-K
    probs = np.zeros((B, Hq, L))
    for b, n in enumerate(lengths):
        if n:
            x = vals[b, :, :n].astype(np.float64)
            m = x.max(axis=1, keepdims=True)
            probs[b, :, :n] = np.exp(x - m) / np.exp(x - m).sum(axis=1, keepdims=True)
    grp = O.group_scores(probs, G)
    ref = O.select_all(grp, lengths, K)
    if shared or Hq == G:
        _assert_sel_equal(sel_idx, sel_count, ref, K)          # ties are exact in both domains
    else:
        check_topk_tolerance(sel_lists(sel_idx, sel_count), ref, grp, K)


def test_topk_logits_rejects_missing_stats():
    shape = api.make_shape(1, 8, 2, 2, 128, 128, 1000, 64, 1, "bf16", 1.0)
    lg = torch.zeros((1, 8, 1000), device="cuda")
    sel = torch.zeros((1, 2, 64), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(api.SpcError):
        api.spc_group_max_topk_logits(shape, lg, None, dev_lengths([1000]), sel, cnt)


TIE_CASES = [
    # (B, Hq, G, L, K, lengths, value pool or None)
    (2, 8, 2, 5000, 300, [5000, 4097], [0.0, 0.25, 0.5]),          # heavy ties across radix passes
    (1, 4, 4, 3000, 64, [3000], [0.125]),                           # all equal: lowest indices
    (3, 2, 1, 2000, 100, [100, 101, 0], None),                      # n = K, n = K + 1, n = 0
    (1, 2, 2, 40000, 2048, [40000], None),                          # keys streamed from global memory
    (1, 2, 2, 70000, 4096, [65537], [0.0, 1e-30, 2.0 ** -126, 1.0]), # streaming + ties + subnormal-ish
    (2, 4, 4, 1500, 1, [1500, 7], None),                            # K = 1
    (1, 6, 2, 33000, 5000, [33000], [-1.0, -0.5, 0.0, 0.5]),        # negative scores, heads 3 per group
    # rows that do not start 16-byte aligned, and a threshold bin of some 2300 tied keys (the
    # select's candidate list) next to the 3-value case above, whose bin outgrows the list
    (2, 4, 2, 3001, 200, [3001, 2500], [0.0, 0.25]),
]


@pytest.mark.parametrize("case", TIE_CASES, ids=[f"tie{i}" for i in range(len(TIE_CASES))])
def test_topk_exact_with_ties_and_edges(case):
    B, Hq, G, L, K, lengths, pool = case
    rng = np.random.default_rng(99)
    if pool is None:
        vals = rng.random((B, Hq, L)).astype(np.float32)
    else:
        vals = rng.choice(np.asarray(pool, dtype=np.float32), size=(B, Hq, L))
    shape = api.make_shape(B, Hq, G, G, 128, 128, L, K, 1, "bf16", 1.0)
    probs = torch.from_numpy(vals).cuda()
    sel_idx, sel_count = _topk_gpu(shape, probs, lengths)
    ref = _oracle_topk(vals.astype(np.float64), lengths, G, K)
    _assert_sel_equal(sel_idx, sel_count, ref, K)


# ------------------------------------------------------------------------------ plan


def _random_selection_sequence(rng, B, G, L, K, steps):
    seqs = []
    prev = [[set() for _ in range(G)] for _ in range(B)]
    for t in range(steps):
        step = []
        for b in range(B):
            row = []
            n = int(rng.choice([0, 1, K - 1, K, L // 2, L])) if t % 5 == 4 else L
            for g in range(G):
                m = min(K, n)
                keep = [x for x in prev[b][g] if x < n and rng.random() < 0.8][:m]
                pool = np.setdiff1d(np.arange(n), np.asarray(keep, dtype=np.int64))
                extra = rng.choice(pool, size=m - len(keep), replace=False) if m > len(keep) else []
                s = np.sort(np.asarray(list(keep) + list(extra), dtype=np.int64))
                row.append(s)
                prev[b][g] = set(s.tolist())
            step.append(row)
        seqs.append(step)
    return seqs


# bitmap plan with 1, 2, 4 and 8 entries per thread; the binary-search plan where the lists and the
# bitmap of S outgrow 64 KB of LDS (budget 8192; a 2^20-position cache)
@pytest.mark.parametrize("B,G,L,K", [(2, 3, 5000, 300), (1, 8, 32768, 2048), (1, 2, 65536, 4096), (1, 1, 40000, 6000),
                                     (1, 1, 9000, 8192), (1, 2, 1 << 20, 1024), (3, 2, 50, 1)])
def test_plan_bit_exact_over_steps(B, G, L, K):
    rng = np.random.default_rng(B * 1000 + K)
    shape = api.make_shape(B, G, G, G, 128, 128, L, K, 1, "bf16", 1.0)
    i32 = dict(dtype=torch.int32, device="cuda")
    slot_pos = torch.empty((B, G, K), **i32)
    bm = torch.empty((B, G, (L + 31) // 32), **i32)
    load_pos, load_slot = torch.empty((B, G, K), **i32), torch.empty((B, G, K), **i32)
    load_count = torch.empty((B, G), **i32)
    api.spc_elastic_reset(shape, -1, slot_pos, bm)
    ref_slots = [[np.full(K, -1, dtype=np.int64) for _ in range(G)] for _ in range(B)]
    for step in _random_selection_sequence(rng, B, G, L, K, 12):
        si = np.full((B, G, K), -1, dtype=np.int32)
        sc = np.zeros((B, G), dtype=np.int32)
        for b in range(B):
            for g in range(G):
                si[b, g, :len(step[b][g])] = step[b][g]
                sc[b, g] = len(step[b][g])
        api.spc_elastic_update(shape, torch.from_numpy(si).cuda(), torch.from_numpy(sc).cuda(), slot_pos, bm,
                               load_pos, load_slot, load_count, flags=api.SPC_PLAN)
        torch.cuda.synchronize()
        sp, lp, ls, lc = (t.cpu().numpy() for t in (slot_pos, load_pos, load_slot, load_count))
        bmn = bm.cpu().numpy().view(np.uint32)
        for b in range(B):
            for g in range(G):
                to_load, lslot, new = O.elastic_plan(step[b][g], ref_slots[b][g])
                ref_slots[b][g] = new
                assert lc[b, g] == len(to_load)
                np.testing.assert_array_equal(lp[b, g, :len(to_load)], to_load)
                np.testing.assert_array_equal(ls[b, g, :len(to_load)], lslot)
                assert np.all(lp[b, g, len(to_load):] == -1) and np.all(ls[b, g, len(to_load):] == -1)
                np.testing.assert_array_equal(sp[b, g], new)
                bits = np.zeros(bmn.shape[-1] * 32, dtype=bool)
                bits[new[new >= 0]] = True
                np.testing.assert_array_equal(np.unpackbits(bmn[b, g].view(np.uint8), bitorder="little")
                                              .astype(bool), bits)


# ------------------------------------------------------------------------------ copy


def _pinned_kv(rng, B, NL, H, L, d, dtype):
    t = torch.empty((B, NL, H, L, 2, d), dtype=dtype, pin_memory=True)
    if dtype == torch.bfloat16:
        bits = rng.integers(-(2 ** 15), 2 ** 15, size=t.shape, dtype=np.int16)
        t.view(torch.int16).copy_(torch.from_numpy(bits))
    else:
        t.copy_(torch.from_numpy(rng.standard_normal(t.shape).astype(np.float32)))
    return t


@pytest.mark.parametrize("dtype,G,H", [(torch.bfloat16, 3, 3), (torch.float32, 3, 3), (torch.bfloat16, 1, 4),
                                       (torch.bfloat16, 2, 4)])
def test_copy_moves_exactly_the_loaded_rows(dtype, G, H):
    """G selection groups over H KV heads: every KV head takes the load lists of its group
    h // (H / G) (G = H: one group per KV head; G = 1: one selection for every head)."""
    rng = np.random.default_rng(5)
    B, NL, L, K, d = 2, 4, 700, 64, 128
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    shape = api.make_shape(B, H, H, G, d, d, L, K, NL, dt, 1.0)
    host = _pinned_kv(rng, B, NL, H, L, d, dtype)
    dev = torch.zeros((B, NL, H, K, 2, d), dtype=dtype, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    slot_pos, bm = torch.empty((B, G, K), **i32), torch.empty((B, G, (L + 31) // 32), **i32)
    lp, ls, lc = torch.empty((B, G, K), **i32), torch.empty((B, G, K), **i32), torch.empty((B, G), **i32)
    api.spc_elastic_reset(shape, -1, slot_pos, bm)
    for step in _random_selection_sequence(rng, B, G, L, K, 6):
        si = np.full((B, G, K), -1, dtype=np.int32); sc = np.zeros((B, G), dtype=np.int32)
        for b in range(B):
            for g in range(G):
                si[b, g, :len(step[b][g])] = step[b][g]; sc[b, g] = len(step[b][g])
        before = dev.clone()
        api.spc_elastic_update(shape, torch.from_numpy(si).cuda(), torch.from_numpy(sc).cuda(), slot_pos, bm,
                               lp, ls, lc, host, api.kv_layout(host), dev, api.kv_layout(dev), 1, 3,
                               flags=api.SPC_PLAN | api.SPC_COPY)
        torch.cuda.synchronize()
        sp = slot_pos.cpu().numpy(); lpn, lsn, lcn = lp.cpu().numpy(), ls.cpu().numpy(), lc.cpu().numpy()
        hraw, draw, braw = raw(host), raw(dev), raw(before)
        # layers outside [1, 3) untouched
        np.testing.assert_array_equal(draw[:, [0, 3]], braw[:, [0, 3]])
        for b in range(B):
            for h in range(H):
                g = h // (H // G)
                for layer in (1, 2):
                    ref = braw[b, layer, h].copy()
                    O.elastic_copy(hraw[b, layer, h], ref, lpn[b, g, :lcn[b, g]], lsn[b, g, :lcn[b, g]])
                    np.testing.assert_array_equal(draw[b, layer, h], ref)
        # copies of every step leave the slots of layers 1-2 holding exactly their positions
        for b in range(B):
            for h in range(H):
                g = h // (H // G)
                for x in np.nonzero(sp[b, g] >= 0)[0]:
                    np.testing.assert_array_equal(draw[b, 1:3, h, x], hraw[b, 1:3, h, sp[b, g, x]])


def test_copy_rejects_unpinned_host_memory():
    B, G, NL, L, K, d = 1, 1, 1, 64, 8, 128
    shape = api.make_shape(B, G, G, G, d, d, L, K, NL, "bf16", 1.0)
    host = torch.zeros((B, NL, G, L, 2, d), dtype=torch.bfloat16)          # pageable
    dev = torch.zeros((B, NL, G, K, 2, d), dtype=torch.bfloat16, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    lp, ls, lc = torch.full((B, G, K), -1, **i32), torch.full((B, G, K), -1, **i32), torch.zeros((B, G), **i32)
    with pytest.raises(api.SpcError) as e:
        api.spc_elastic_update(shape, None, None, None, None, lp, ls, lc, host, api.kv_layout(host), dev,
                               api.kv_layout(dev), 0, 1, flags=api.SPC_COPY)
    assert e.value.status == 4


# ------------------------------------------------------------------------------ attention


def _attend(shape, q, ql, kv, rows, counts, mode, NL, out, halves):
    if not halves:
        api.spc_sparse_decode_attn(shape, q, ql, kv, api.kv_layout(kv), rows, counts, mode, 0, NL, out)
        return
    ws = torch.empty(api.spc_workspace_size(api.SPC_CALL_ATTN, shape), dtype=torch.uint8, device="cuda")
    api.spc_attn_partial(shape, q, ql, kv, api.kv_layout(kv), rows, counts, mode, 0, NL, ws)
    api.spc_attn_merge(shape, 0, NL, ws, out)


def _attn_case(p, lengths, mode, seed=21, halves=False):
    """Selections from the GPU scores + Top-K, K/V placed by plan + copy (SLOTS) or a full cache (GATHER);
    halves: the attention as spc_attn_partial + spc_attn_merge."""
    w = W.generate(p, device="cuda", seed=seed, steps=1, pin_host=True)
    shape, probs = _scores(p, w, lengths)
    sel_idx, sel_count = _topk_gpu(shape, probs, lengths)
    B, G, K, NL = p.batch, p.n_groups, p.budget, p.n_layers
    out = torch.full((B, NL, p.n_q_heads, p.v_dim), float("nan"), device="cuda")
    q = w.q[0].contiguous()
    ql = api.q_layout(p.n_q_heads * p.head_dim, 0, p.head_dim)
    if mode == api.SPC_ROWS_SLOTS:
        i32 = dict(dtype=torch.int32, device="cuda")
        slot_pos, bm = torch.empty((B, G, K), **i32), torch.empty((B, G, (p.max_len + 31) // 32), **i32)
        lp, ls, lc = torch.empty((B, G, K), **i32), torch.empty((B, G, K), **i32), torch.empty((B, G), **i32)
        dev = torch.zeros((B, NL, p.n_kv_heads, K, 2, p.head_dim), dtype=p.torch_dtype, device="cuda")
        api.spc_elastic_reset(shape, -1, slot_pos, bm)
        api.spc_elastic_update(shape, sel_idx, sel_count, slot_pos, bm, lp, ls, lc, w.host_kv,
                               api.kv_layout(w.host_kv), dev, api.kv_layout(dev), 0, NL,
                               flags=api.SPC_PLAN | api.SPC_COPY)
        _attend(shape, q, ql, dev, slot_pos, None, mode, NL, out, halves)
    else:
        full = w.host_kv.cuda()
        _attend(shape, q, ql, full, sel_idx, sel_count, mode, NL, out, halves)
    torch.cuda.synchronize()
    return w, sel_lists(sel_idx, sel_count), out.cpu().numpy().astype(np.float64)


def _oracle_out(p, w, sel):
    from oracle import OracleDecoder
    dec = OracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale, p.dtype)
    return dec.attend(raw(w.q[0]), raw(w.host_kv), sel, list(range(p.n_layers)))


ATTN_CASES = [
    ("gqa_slots", GQA_SMALL, [1000, 517], api.SPC_ROWS_SLOTS),
    ("gqa_gather", GQA_SMALL, [1000, 517], api.SPC_ROWS_GATHER),
    ("gqa_short_and_empty", GQA_SMALL.with_(batch=3), [40, 0, 96], api.SPC_ROWS_SLOTS),
    ("tiny_f32_slots", W.PRESETS["tiny"].with_(n_layers=2), [4096], api.SPC_ROWS_SLOTS),
    ("mha_slots", GQA_SMALL.with_(kind="mha", n_q_heads=4, n_kv_heads=4, max_len=777, budget=200), [777, 500],
     api.SPC_ROWS_SLOTS),
    ("mqa_gather", GQA_SMALL.with_(kind="mqa", n_q_heads=8, n_kv_heads=1, max_len=600), [600, 33],
     api.SPC_ROWS_GATHER),
    ("d64_slots", GQA_SMALL.with_(head_dim=64, v_dim=64, max_len=300), [300, 299], api.SPC_ROWS_SLOTS),
    ("budget1", GQA_SMALL.with_(budget=1), [1000, 5], api.SPC_ROWS_SLOTS),
    ("split_tail", GQA_SMALL.with_(budget=333, max_len=2000), [2000, 1999], api.SPC_ROWS_SLOTS),
    # batch-level retrieval: the heads of every KV head attend over one shared selection
    ("batch_level_slots", GQA_SMALL.with_(kind="mqa"), [1000, 517], api.SPC_ROWS_SLOTS),
    ("batch_level_gather", GQA_SMALL.with_(kind="mqa"), [1000, 0], api.SPC_ROWS_GATHER),
    ("batch_level_32_heads_slots", GQA_SMALL.with_(kind="mqa", n_q_heads=32, n_kv_heads=8, max_len=1500),
     [1500, 1001], api.SPC_ROWS_SLOTS),
    # 400 workgroups per split index (4 sequences x 25 layers x 4 groups x 4 head chunks or the
    # like) and 300 rows: 3 splits of 128 rows need 2 rounds of 1024 workgroups, 2 of 160 rows
    # one, so the launch takes the 160-row kernels, the second split ragged (140 rows)
    ("wide_splits_slots", GQA_SMALL.with_(batch=4, n_layers=25, n_q_heads=16, n_kv_heads=4, max_len=600,
                                          budget=300), [600, 599, 301, 17], api.SPC_ROWS_SLOTS),
    ("wide_splits_2_heads_gather", GQA_SMALL.with_(batch=4, n_layers=25, n_q_heads=8, n_kv_heads=4, max_len=600,
                                                   budget=300), [600, 0, 450, 299], api.SPC_ROWS_GATHER),
    ("wide_splits_mha_slots", GQA_SMALL.with_(kind="mha", batch=4, n_layers=25, n_q_heads=4, n_kv_heads=4,
                                              max_len=600, budget=300), [600, 1, 160, 161], api.SPC_ROWS_SLOTS),
]


@pytest.mark.parametrize("name,p,lengths,mode", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_matches_oracle(name, p, lengths, mode):
    w, sel, got = _attn_case(p, lengths, mode)
    ref = _oracle_out(p, w, sel)
    err = np.max(np.abs(got - ref))
    assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, err
    for b, n in enumerate(lengths):
        if n == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("name,p,lengths,mode", [ATTN_CASES[i] for i in (0, 1, 2, 3, 12, 13)],
                         ids=[ATTN_CASES[i][0] for i in (0, 1, 2, 3, 12, 13)])
def test_partial_then_merge_equals_the_whole_call(name, p, lengths, mode):
    _, _, whole = _attn_case(p, lengths, mode)
    _, _, halves = _attn_case(p, lengths, mode, halves=True)
    np.testing.assert_array_equal(halves, whole)


def test_full_budget_reproduces_dense_attention():
    """K = L (>= n): sparse attention equals dense attention over every position."""
    p = GQA_SMALL.with_(max_len=512, budget=512, n_layers=2)
    lengths = [512, 300]
    w, sel, got = _attn_case(p, lengths, api.SPC_ROWS_SLOTS)
    for b, n in enumerate(lengths):
        assert all(len(s) == n for s in sel[b])
    q = f64(w.q[0], p.dtype)
    kv = f64(w.host_kv, p.dtype)
    import torch.nn.functional as F
    for b, n in enumerate(lengths):
        for layer in range(p.n_layers):
            K_ = torch.from_numpy(kv[b, layer, :, :n, 0]); V_ = torch.from_numpy(kv[b, layer, :, :n, 1])
            ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[:, None, :], K_, V_, enable_gqa=True,
                                                 scale=p.scale)[:, 0, :].numpy()
            assert np.max(np.abs(got[b, layer] - ref)) <= ATTN_DERIVED


def test_topk_exact_long_rows_and_large_budget():
    """Rows beyond 2^16 positions with a budget of 9000 (counts beyond 16 bits) and heavy ties."""
    B, Hq, G, L, K = 1, 2, 1, 70000, 9000
    rng = np.random.default_rng(7)
    vals = rng.choice(np.asarray([0.0, 0.5, 0.75, 1.0], dtype=np.float32), size=(B, Hq, L), p=[0.6, 0.3, 0.05, 0.05])
    shape = api.make_shape(B, Hq, G, G, 128, 128, L, K, 1, "bf16", 1.0)
    sel_idx, sel_count = _topk_gpu(shape, torch.from_numpy(vals).cuda(), [L])
    _assert_sel_equal(sel_idx, sel_count, _oracle_topk(vals.astype(np.float64), [L], G, K), K)


# ------------------------------------------------------------------------------ Top-K + plan in one call


FUSED_CASES = [
    # (name, preset, lengths per step): the plan inside the LDS select's workgroup (rows of at most
    # 32768 positions) with several heads per group and with one (raw logits, 2 KB per thread of plan
    # lists at budget 4096), a batch with a short and an empty sequence and a row length that is no
    # multiple of 32, budget 8192 (8 slots per thread) with sequences at, below and just above the
    # budget; the register-resident select for rows past 32768 with the plan in its tail (two bitmap
    # words per thread): MHA at 64K and two heads per group at 40000 positions with short rows; and
    # budget 8192 at 40000 positions, where the plan runs as its own launch after the select
    ("gqa_32k", W.PRESETS["b1_32k"].with_(n_layers=1), None),
    ("mha_32k_raw", W.PRESETS["mha_64k"].with_(max_len=32768, batch=1), None),
    ("ragged", GQA_SMALL.with_(batch=3, max_len=3000, budget=256), [[3000, 100, 0], [3000, 257, 0], [2999, 300, 5]]),
    ("budget_8192_lds", GQA_SMALL.with_(batch=3, n_q_heads=4, n_kv_heads=2, max_len=20000, budget=8192),
     [[20000, 5000, 8192], [19999, 8192, 8193], [20000, 8193, 12000]]),
    ("mha_64k", W.PRESETS["mha_64k"], None),
    # more than 256 instances of one head each: the 512-thread register select with the plan in its
    # tail (budgets 1024 and 2048: two and four slots per thread), lengths at, just above and below
    # the budget and zero
    ("raw_many_1024", GQA_SMALL.with_(kind="mha", batch=2, n_q_heads=136, n_kv_heads=136, n_layers=1,
                                      max_len=3000, budget=1024), [[3000, 1000], [2999, 1024], [3000, 1025]]),
    ("raw_many_2048", GQA_SMALL.with_(kind="mha", batch=2, n_q_heads=132, n_kv_heads=132, n_layers=1,
                                      max_len=4000, budget=2048), [[4000, 2048], [3999, 2049], [4000, 0]]),
    ("reg_gqa_40k", GQA_SMALL.with_(batch=2, n_q_heads=4, n_kv_heads=2, max_len=40000, budget=1024),
     [[40000, 1000], [39999, 1024], [40000, 1025]]),
    ("budget_8192", GQA_SMALL.with_(batch=1, n_q_heads=4, n_kv_heads=2, max_len=40000, budget=8192), None),
]


@pytest.mark.parametrize("name,p,lens", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_topk_and_plan_in_one_call_equal_the_two_calls(name, p, lens):
    steps = 3
    w = W.generate(p, device="cuda", seed=31, steps=steps)
    shape = shape_of(p)
    B, G, K, L = p.batch, p.n_groups, p.budget, p.max_len
    i32 = dict(dtype=torch.int32, device="cuda")

    def state():
        st = dict(sel=torch.full((B, G, K), -7, **i32), cnt=torch.full((B, G), -7, **i32),
                  sp=torch.empty((B, G, K), **i32), bm=torch.empty((B, G, (L + 31) // 32), **i32),
                  lp=torch.full((B, G, K), -7, **i32), ls=torch.full((B, G, K), -7, **i32),
                  lc=torch.full((B, G), -7, **i32))
        api.spc_elastic_reset(shape, -1, st["sp"], st["bm"])
        return st

    two, one = state(), state()
    ref_slots = [[np.full(K, -1, dtype=np.int64) for _ in range(G)] for _ in range(B)]
    for t in range(steps):
        lengths = list(w.lengths[t]) if lens is None else lens[t]
        _, logits, stats = _logits(p, w, lengths, t)
        lt = dev_lengths(lengths)
        api.spc_group_max_topk_logits(shape, logits, stats, lt, two["sel"], two["cnt"])
        api.spc_elastic_update(shape, two["sel"], two["cnt"], two["sp"], two["bm"], two["lp"], two["ls"], two["lc"],
                               flags=api.SPC_PLAN)
        api.spc_group_max_topk_plan_logits(shape, logits, stats, lt, one["sel"], one["cnt"], one["sp"], one["bm"],
                                           one["lp"], one["ls"], one["lc"])
        torch.cuda.synchronize()
        for k in two:
            np.testing.assert_array_equal(one[k].cpu().numpy(), two[k].cpu().numpy(), err_msg=f"{k} at step {t}")
        # and the selection against the fp64 oracle chain, the plan against the oracle's plan
        gsel = sel_lists(one["sel"], one["cnt"])
        ref_probs = O.retrieval_scores(f64(w.q[t], p.dtype), f64(w.dlm_k, p.dtype), lengths, p.scale)
        ref_grp = O.group_scores(ref_probs, G)
        check_topk_tolerance(gsel, O.select_all(ref_grp, lengths, K), ref_grp, K)
        lc, sp = one["lc"].cpu().numpy(), one["sp"].cpu().numpy()
        for b in range(B):
            for g in range(G):
                to_load, _, ref_slots[b][g] = O.elastic_plan(gsel[b][g], ref_slots[b][g])
                assert lc[b, g] == len(to_load)
                np.testing.assert_array_equal(sp[b, g], ref_slots[b][g])
