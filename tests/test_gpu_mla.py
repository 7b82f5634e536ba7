"""MLA variant: head-level retrieval over the latent cache, per-head Top-K, attention over the
selected latent rows, against the oracle's literal expansion of only the selected rows."""
import math

import numpy as np
import pytest
import torch

from oracle import spc_oracle as O
from speculative_kv_sparsity_amd import api
from speculative_kv_sparsity_amd import workload as W
from speculative_kv_sparsity_amd.driver import MlaDecoder
from tests.gpu_util import (ATTN_DERIVED, ATTN_MAX_ABS, PROBS_RTOL, check_topk_tolerance, dev_lengths, raw,
                            sel_lists)

pytestmark = pytest.mark.gpu


def _bf(t):
    return O.to_f64(raw(t), "bf16")


def _check_steps(p, w, steps, lengths_override=None, heads=None, batches=None):
    dec = MlaDecoder(p, w.latent, w.w_uk, w.w_uv)
    dec.stats_out = dec.tile_stats          # the step needs no tile stats; they are checked here
    T = api.spc_score_tile(dec.shape)
    C = p.latent_dim
    w_uk, w_uv = _bf(w.w_uk), _bf(w.w_uv)
    lat_all = [_bf(w.latent[b]) for b in range(p.batch)]
    heads = list(range(p.n_q_heads)) if heads is None else heads
    batches = list(range(p.batch)) if batches is None else batches
    prev = None
    overl = []
    for t in range(steps):
        lengths = list(w.lengths[t]) if lengths_override is None else lengths_override
        qn, qr = w.q_nope[t].contiguous(), w.q_rope[t].contiguous()
        dec.step(qn, qr, dev_lengths(lengths))
        torch.cuda.synchronize()
        qn64, qr64 = _bf(qn), _bf(qr)
        logits = dec.logits.cpu().numpy().astype(np.float64)
        stats = dec.tile_stats.cpu().numpy().astype(np.float64)
        gsel = sel_lists(dec.sel_idx, dec.sel_count)
        # Top-K bit-exact on the GPU's own float32 logits (one head per group: ranked as they are)
        for b in range(p.batch):
            n = int(lengths[b])
            for h in range(p.n_q_heads):
                ref = O.topk_select(np.nan_to_num(logits[b, h], nan=-np.inf), n, p.budget)
                np.testing.assert_array_equal(gsel[b][h], ref)
        # scores and selection against the literal-expansion oracle, sampled heads
        for b in batches:
            n = int(lengths[b])
            if n == 0:
                assert all(len(gsel[b][h]) == 0 for h in heads)
                assert np.all(dec.out.cpu().numpy()[b] == 0)
                continue
            lat, rope = lat_all[b][:, :C], lat_all[b][:, C:]
            ref_p = O.mla_retrieval_scores(qn64[b:b + 1], qr64[b:b + 1], lat[None], rope[None], w_uk, [n], p.scale,
                                           heads=heads)
            nt = (n + T - 1) // T
            for h in heads:
                rp = ref_p[(0, h)]
                # the probabilities exp(logit - lse), lse from the head's tile pairs
                m, sm = stats[b, h, :nt, 0], stats[b, h, :nt, 1]
                lse = np.max(m) + np.log(np.sum(sm * np.exp(m - np.max(m))))
                np.testing.assert_allclose(np.exp(logits[b, h, :n] - lse), rp, rtol=PROBS_RTOL, atol=0)
                ref_sel = O.topk_select(rp, n, p.budget)
                check_topk_tolerance([[gsel[b][h]]], [[ref_sel]], rp[None, None, :], p.budget)
                # attention + output projection over the GPU's selection, rows expanded literally
                ref_o = O.mla_sparse_attention(qn64[b, h], qr64[b, h], lat, rope, w_uk, w_uv, gsel[b][h], h, p.scale)
                err = float(np.max(np.abs(dec.out.cpu().numpy()[b, h].astype(np.float64) - ref_o)))
                assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, (t, b, h, err)
        # the per-head plan keeps the resident set equal to the selection
        sp = dec.slot_pos.cpu().numpy()
        for b in range(p.batch):
            for h in range(p.n_q_heads):
                assert set(int(x) for x in sp[b, h] if x >= 0) == set(gsel[b][h].tolist())
        if prev is not None:
            overl.append(np.mean([O.overlap(prev[b][h], gsel[b][h]) for b in range(p.batch)
                                  for h in range(p.n_q_heads) if len(gsel[b][h])]))
        prev = gsel
    return overl


def test_mla_small_ragged_all_heads():
    p = W.PRESETS["mla_32k"].with_(batch=3, n_q_heads=16, max_len=1000, budget=96)
    w = W.generate(p, device="cuda", seed=5, steps=3)
    _check_steps(p, w, 3, lengths_override=[1000, 613, 0])


def test_mla_budget_covers_everything_and_tail_tile():
    """n <= K selects every position; a length that is not a multiple of the 16-row MFMA block."""
    p = W.PRESETS["mla_32k"].with_(batch=2, n_q_heads=32, max_len=300, budget=300)
    w = W.generate(p, device="cuda", seed=6, steps=1)
    _check_steps(p, w, 1, lengths_override=[300, 77])


def test_mla_32k_full_shape_sampled_heads():
    """4 sequences, 128 heads, 32768 latent rows, budget 2048; oracle checks on sampled heads."""
    p = W.PRESETS["mla_32k"]
    w = W.generate(p, device="cuda", seed=0, steps=2)
    overl = _check_steps(p, w, 2, heads=[0, 37, 127], batches=[0, 3])
    assert overl and overl[0] > 0.3


def test_mla_32k_full_shape_all_heads_of_one_sequence():
    """Every one of the 128 heads of sequence 2 at the full 4 x 128 x 32768 shape: scores, selection and
    attention with the output projection against the oracle's literal expansion."""
    p = W.PRESETS["mla_32k"]
    w = W.generate(p, device="cuda", seed=3, steps=1)
    _check_steps(p, w, 1, batches=[2])


def test_mla_512_position_tiles_with_ragged_lengths():
    """The shape that scores on 512-position tiles (4 sequences x 64 tiles, each workgroup all 128
    heads: 8 waves of 16), with lengths that end inside a tile's last 64-row sub-tile, inside its
    first 16-row block, and at zero: logits, tile stats and Top-K against the oracle; the heads
    sampled sit in the first, fourth, fifth and last wave."""
    p = W.PRESETS["mla_32k"]
    w = W.generate(p, device="cuda", seed=4, steps=1)
    dec_shape = api.make_shape(p.batch, p.n_q_heads, 1, p.n_q_heads, p.head_dim, p.v_dim, p.max_len, p.budget, 1,
                               p.dtype, p.scale)
    assert api.spc_score_tile(dec_shape) == 512
    _check_steps(p, w, 1, lengths_override=[32768, 30001, 17, 0], heads=[0, 63, 64, 127], batches=[0, 1, 2, 3])


@pytest.mark.parametrize("B,H,dn,dv,n_layers,layer", [(1, 3, 128, 128, 1, 0), (5, 8, 100, 77, 3, 2),
                                                       (16, 2, 33, 300, 2, 1), (4, 128, 128, 128, 1, 0)])
def test_mla_helpers_match_literal_up_projections(B, H, dn, dv, n_layers, layer):
    """spc_mla_absorb_q and spc_mla_out_proj against the oracle's literal expansion.  The
    absorbed query dotted with a latent row c || r equals q_nope . (W_UK c) + q_rope . r, so the
    unit rows e_k give every entry; the output projection of o_lat equals the value part of the
    expansion of o_lat taken as a latent row, W_UV o_lat.  Odd nope and value widths, a batch of
    16 and four row groups of output rows with a ragged tail."""
    C, R = 512, 64
    gen = torch.Generator().manual_seed(7 * B + dn + dv)
    w_uk = (torch.randn(H, dn, C, generator=gen) * 0.05).to(torch.bfloat16)
    w_uv = (torch.randn(H, dv, C, generator=gen) * 0.05).to(torch.bfloat16)
    q_nope = torch.randn(B, H, dn, generator=gen).to(torch.bfloat16)
    q_rope = torch.randn(B, H, R, generator=gen).to(torch.bfloat16)
    o_lat = torch.randn(B, n_layers, H, C, generator=gen)
    shape = api.make_shape(B, H, 1, H, C + R, C, 64, 8, n_layers, "bf16", (128 + R) ** -0.5)
    dev = torch.device("cuda")
    q_abs = torch.full((B, H, C + R), float("nan"), device=dev)
    out = torch.full((B, H, dv), float("nan"), device=dev)
    api.spc_mla_absorb_q(shape, dn, w_uk.to(dev), q_nope.to(dev), q_rope.to(dev), q_abs)
    api.spc_mla_out_proj(shape, dv, w_uv.to(dev), o_lat.to(dev), layer, out)
    torch.cuda.synchronize()
    qa, got = q_abs.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64)
    wuk, wuv = _bf(w_uk), _bf(w_uv)
    qn, qr = _bf(q_nope), _bf(q_rope)
    eye = np.eye(C)
    for h in range(H):
        # keys of the unit latent rows (rope 0), then q_nope . K[k]: entry k of W_UK^T q_nope
        keys = O.mla_expand_keys(eye, np.zeros((C, R)), wuk[h:h + 1])[0][:, :dn]
        for b in range(B):
            ref_q = keys @ qn[b, h]
            # fp32 accumulation: at most dn fused multiply-adds and 16 partial sums, each rounding
            # by at most 2^-24 of the running magnitude, bounded by the sum of |terms|
            bound = (dn + 32) * 2.0 ** -24 * (np.abs(keys) @ np.abs(qn[b, h]))
            assert np.all(np.abs(qa[b, h, :C] - ref_q) <= bound), (b, h)
            np.testing.assert_array_equal(qa[b, h, C:], qr[b, h])       # the rope part widened exactly
            _, V = O.mla_expand_rows(o_lat[b, layer, h].numpy()[None].astype(np.float64), np.zeros((1, R)),
                                     wuk[h], wuv[h])
            bound = (C + 32) * 2.0 ** -24 * (np.abs(wuv[h]) @ np.abs(o_lat[b, layer, h].numpy().astype(np.float64)))
            assert np.all(np.abs(got[b, h] - V[0]) <= bound), (b, h)


def test_mla_graph_replay_equals_eager_steps():
    """The step captured once into a HIP graph and replayed over its static input buffers gives,
    step after step, the same selection, load lists, latent attention output and output projection
    as eager launches from the same state, bit for bit; eager work and a synchronize run between
    the replays."""
    p = W.PRESETS["mla_32k"].with_(batch=2, n_q_heads=32, max_len=4096, budget=256)
    steps = 4
    w = W.generate(p, device="cuda", seed=8, steps=steps)
    lens = [[4096, 3001], [4096, 3002], [10, 3003], [4096, 0]]
    dec = MlaDecoder(p, w.latent, w.w_uk, w.w_uv)
    names = ("sel_idx", "sel_count", "load_pos", "load_slot", "load_count", "slot_pos", "resident_bm", "o_lat", "out")
    start = {k: getattr(dec, k).clone() for k in names}
    eager = []
    for t in range(steps):
        dec.step(w.q_nope[t].contiguous(), w.q_rope[t].contiguous(), dev_lengths(lens[t]))
        torch.cuda.synchronize()
        eager.append({k: getattr(dec, k).clone() for k in names})
    for k in names:
        getattr(dec, k).copy_(start[k])
    dec.capture()
    for k in ("slot_pos", "resident_bm"):                 # capture leaves the state as it was
        assert torch.equal(getattr(dec, k), start[k]), k
    for t in range(steps):
        dec.step_graph(w.q_nope[t].contiguous(), w.q_rope[t].contiguous(), dev_lengths(lens[t]))
        torch.cuda.synchronize()
        junk = torch.randn(1 << 16, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k in names:
            assert torch.equal(getattr(dec, k), eager[t][k]), f"{k} at step {t}"


@pytest.mark.parametrize("kind", ["mla", "mha"])
def test_logits_without_tile_stats_are_the_same(kind):
    """With one query head per group the tile stats may be left out (NULL): the logits, and the Top-K
    taken from them, are bit-identical to a call that computes them."""
    if kind == "mla":
        p = W.PRESETS["mla_32k"].with_(batch=2, n_q_heads=32, max_len=3000, budget=128)
        w = W.generate(p, device="cuda", seed=12, steps=1)
        dec = MlaDecoder(p, w.latent, w.w_uk, w.w_uv)
        shape = dec.shape
        q = torch.empty((p.batch, p.n_q_heads, p.head_dim), dtype=torch.float32, device="cuda")
        api.spc_mla_absorb_q(shape, p.nope_dim, w.w_uk, w.q_nope[0].contiguous(), w.q_rope[0].contiguous(), q)
        k = w.latent
    else:
        p = W.PRESETS["mha_64k"].with_(batch=2, n_q_heads=4, n_kv_heads=4, max_len=5000, budget=256)
        w = W.generate(p, device="cuda", seed=12, steps=1)
        shape = api.make_shape(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.v_dim, p.max_len,
                               p.budget, 1, p.dtype, p.scale)
        q, k = w.q[0].contiguous(), w.dlm_k
    lengths = dev_lengths([p.max_len, p.max_len - 777])
    a = torch.full((p.batch, p.n_q_heads, p.max_len), float("nan"), device="cuda")
    b = a.clone()
    stats = torch.empty(api.tile_stats_shape(shape), device="cuda")
    api.spc_retrieval_logits(shape, q, k, lengths, a, stats)
    api.spc_retrieval_logits(shape, q, k, lengths, b, None)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0))
    i32 = dict(dtype=torch.int32, device="cuda")
    s1, c1 = torch.empty((p.batch, p.n_groups, p.budget), **i32), torch.empty((p.batch, p.n_groups), **i32)
    s2, c2 = s1.clone(), c1.clone()
    api.spc_group_max_topk_logits(shape, a, None, lengths, s1, c1)
    api.spc_group_max_topk_logits(shape, b, None, lengths, s2, c2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(c1, c2)


# Latent attention called directly: the absorbed float32 query against latent rows (keys: all 576
# dims, values: the first 512), with ragged per-head counts and garbage past each count.
#   whole*: budgets of <= 2048 rows with >= 512 heads -> one split per head, the output written by
#     the split kernel (no merge); 8, 4 and 2 (sequence, layer) groups, the last two shared by 2 and
#     4 XCDs (an odd number of heads in the 2-XCD case)
#   large:  a budget over 2048 rows -> splits of 1024 rows and the merge
#   small:  few heads -> splits of 256 rows, a ragged last one
LATENT_CASES = [("whole", 8, 64, 4096, 2048), ("whole_xcd2_odd", 4, 129, 3000, 1500),
                ("whole_xcd4", 2, 256, 2500, 2048), ("large", 4, 128, 4096, 3000), ("small", 2, 6, 1500, 700)]


@pytest.mark.parametrize("name,B,H,L,K", LATENT_CASES, ids=[c[0] for c in LATENT_CASES])
def test_latent_attention_matches_oracle(name, B, H, L, K):
    p = W.PRESETS["mla_32k"]
    D, DV = p.head_dim, p.v_dim
    rng = np.random.default_rng(11)
    g = torch.Generator().manual_seed(12)
    latent = torch.randn((B, L, D), generator=g).to(torch.bfloat16)
    q = (0.6 * torch.randn((B, H, D), generator=g)).float()
    counts = rng.integers(0, K + 1, size=(B, H)).astype(np.int32)
    edges = [0, 1, K, K - 1, 17, 511, 512, 513, 1023, 1025, 2047, 2049]
    for i, c in enumerate(edges):
        if c <= K:
            counts.flat[(i * 7) % counts.size] = c
    rows = np.full((B, H, K), L + 7, dtype=np.int32)          # past each count: ignored
    for b in range(B):
        for h in range(H):
            n = int(counts[b, h])
            rows[b, h, :n] = np.sort(rng.choice(L, size=n, replace=False))
    shape = api.make_shape(B, H, 1, H, D, DV, L, K, 1, "bf16", p.scale)
    args = (shape, q.cuda(), api.q_layout(H * D, 0, D), latent.cuda(), api.SpcKvLayout(L * D, 0, 0, D, 0),
            torch.from_numpy(rows).cuda(), torch.from_numpy(counts).cuda(), api.SPC_ROWS_GATHER)
    out = torch.full((B, 1, H, DV), float("nan"), device="cuda")
    api.spc_sparse_decode_attn(*args, 0, 1, out)
    # the split kernel and the merge as two calls: the same bits as the whole call
    ws = torch.empty(api.spc_workspace_size(api.SPC_CALL_ATTN, shape), dtype=torch.uint8, device="cuda")
    halves = torch.full((B, 1, H, DV), float("nan"), device="cuda")
    api.spc_attn_partial(*args, 0, 1, ws)
    api.spc_attn_merge(shape, 0, 1, ws, halves)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(halves.cpu().numpy(), out.cpu().numpy())
    got = out.cpu().numpy().astype(np.float64)[:, 0]
    lat64, q64 = _bf(latent), q.numpy().astype(np.float64)
    err = 0.0
    for b in range(B):
        for h in range(H):
            n = int(counts[b, h])
            ref = O.sparse_attention(q64[b, h], lat64[b], lat64[b][:, :DV], rows[b, h, :n], p.scale)
            if n == 0:
                assert np.all(got[b, h] == 0), (b, h)
            err = max(err, float(np.max(np.abs(got[b, h] - ref))))
    assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, err


# The attention of one MLA layer with its output projection in one call, against the two calls it
# replaces (spc_sparse_decode_attn, then spc_mla_out_proj) and against the oracle on sampled heads.
#   one_launch*: one split per head (budget <= 2048, >= 512 heads): attention and projection in
#     one launch, o_lat not written; 128 and 100 output rows per head
#   two_calls:  few heads: the attention into o_lat and the projection kernel, the same bits
#   one_launch_layer1: two layers (the second attended), 2 sequences x 2 layers x 128 heads = 512
PROJ_CASES = [("one_launch", 4, 128, 4096, 2048, 128, 1), ("one_launch_dv100", 4, 128, 3000, 1024, 100, 1),
              ("one_launch_layer1", 2, 128, 2500, 2048, 128, 2), ("two_calls", 2, 16, 1500, 700, 128, 1)]


@pytest.mark.parametrize("name,B,H,L,K,dv,NL", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_attention_with_projection_equals_the_two_calls(name, B, H, L, K, dv, NL):
    p = W.PRESETS["mla_32k"]
    D, DV = p.head_dim, p.v_dim
    rng = np.random.default_rng(21)
    g = torch.Generator().manual_seed(22)
    # [B][NL][L][D] latent rows and [B][NL][H][D] queries; the attended layer is the last one
    latent = torch.randn((B, NL, L, D), generator=g).to(torch.bfloat16)
    q = (0.6 * torch.randn((B, NL, H, D), generator=g)).float()
    layer = NL - 1
    w_uv = (torch.randn((H, dv, DV), generator=g) / math.sqrt(DV)).to(torch.bfloat16)
    counts = rng.integers(0, K + 1, size=(B, H)).astype(np.int32)
    counts[0, 0], counts[-1, -1], counts[0, -1] = 0, K, 1
    rows = np.full((B, H, K), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            n = int(counts[b, h])
            rows[b, h, :n] = np.sort(rng.choice(L, size=n, replace=False))
    shape = api.make_shape(B, H, 1, H, D, DV, L, K, NL, "bf16", p.scale)
    args = (shape, q.cuda(), api.q_layout(NL * H * D, H * D, D), latent.cuda(),
            api.SpcKvLayout(NL * L * D, L * D, 0, D, 0), torch.from_numpy(rows).cuda(),
            torch.from_numpy(counts).cuda(), api.SPC_ROWS_GATHER)
    wd = w_uv.cuda()
    nan = dict(dtype=torch.float32, device="cuda")
    o_two, out_two = torch.full((B, NL, H, DV), float("nan"), **nan), torch.full((B, H, dv), float("nan"), **nan)
    api.spc_sparse_decode_attn(*args, layer, layer + 1, o_two)
    api.spc_mla_out_proj(shape, dv, wd, o_two, layer, out_two)
    o_one, out_one = torch.full((B, NL, H, DV), float("nan"), **nan), torch.full((B, H, dv), float("nan"), **nan)
    api.spc_mla_attn_out_proj(*args, layer, dv, wd, o_one, out_one)
    torch.cuda.synchronize()
    a, z = out_one.cpu().numpy(), out_two.cpu().numpy()
    if name.startswith("two"):
        np.testing.assert_array_equal(a, z)
        np.testing.assert_array_equal(o_one.cpu().numpy(), o_two.cpu().numpy())
    else:
        # the same float32 output of each head, projected in another summation order
        np.testing.assert_allclose(a, z, rtol=1e-5, atol=1e-6)
        assert torch.isnan(o_one).all()                     # one launch: o_lat is not written
    assert np.all(a[0, 0] == 0)                             # a head without rows
    lat64, q64, w64 = _bf(latent), q.numpy().astype(np.float64), _bf(w_uv)
    err = 0.0
    for b, h in [(0, 1), (0, H - 1), (B - 1, H // 2), (B - 1, H - 1)]:
        n = int(counts[b, h])
        lb = lat64[b, layer]
        ref = w64[h] @ O.sparse_attention(q64[b, layer, h], lb, lb[:, :DV], rows[b, h, :n], p.scale)
        err = max(err, float(np.max(np.abs(a[b, h].astype(np.float64) - ref))))
    assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, err
