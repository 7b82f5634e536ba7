"""MLA in the literal form on the GPU against the oracle: each head's newly loaded latent rows
expanded into its own bf16 K/V slots (K = W_UK c || r, V = W_UV c), kept rows left as they are,
the joined query, and attention over the slots against the oracle's literal expansion."""
import numpy as np
import pytest
import torch

from oracle import spc_oracle as O
from speculative_kv_sparsity_amd import workload as W
from speculative_kv_sparsity_amd.driver import MlaDecoder, MlaLiteralDecoder
from tests.gpu_util import ATTN_DERIVED, ATTN_MAX_ABS, dev_lengths, raw, sel_lists

pytestmark = pytest.mark.gpu


def _bf(t):
    return O.to_f64(raw(t), "bf16")


def _check_rows(dec, p, lat, w_uk, w_uv, heads, batches):
    """Every filled slot of the sampled heads holds the expansion of its position."""
    C, dn, R = p.latent_dim, p.nope_dim, p.rope_dim
    sp = dec.slot_pos.cpu().numpy()
    for b in batches:
        for h in heads:
            xs = np.nonzero(sp[b, h] >= 0)[0]
            if xs.size == 0:
                continue
            pos = sp[b, h, xs]
            got = _bf(dec.kv_exp[b, h])[xs]
            c = lat[b][pos, :C]
            exact_k, exact_v = O.mla_expand_rows(c, lat[b][pos, C:], w_uk[h], w_uv[h])
            for g, e, Wm in ((got[:, :dn], exact_k[:, :dn], w_uk[h]), (got[:, dn + R:], exact_v, w_uv[h])):
                # within half a bf16 spacing of the exact value plus the float32 accumulation bound
                # (C terms: |error| <= C 2^-24 sum |c_k W_rk|)
                spacing = np.ldexp(1.0, np.frexp(np.abs(e))[1] - 8)
                acc = C * 2.0 ** -24 * (np.abs(c) @ np.abs(Wm).T)
                assert np.all(np.abs(g - e) <= 0.5 * spacing + acc), float(np.max(np.abs(g - e) / spacing))
                # equal to the oracle's stored value except where the two sums round apart
                assert np.mean(g != O.round_bf16(e)) < 0.01
            np.testing.assert_array_equal(got[:, dn:dn + R], lat[b][pos, C:])     # rotary dims copied


def _run(p, steps, seed, heads=None, batches=None, lengths_override=None):
    w = W.generate(p, device="cuda", seed=seed, steps=steps)
    dec = MlaLiteralDecoder(p, w.latent, w.w_uk, w.w_uv)
    ref_dec = MlaDecoder(p, w.latent, w.w_uk, w.w_uv)          # the absorbed form on the same inputs
    C = p.latent_dim
    w_uk, w_uv = _bf(w.w_uk), _bf(w.w_uv)
    lat = [_bf(w.latent[b]) for b in range(p.batch)]
    heads = list(range(p.n_q_heads)) if heads is None else heads
    batches = list(range(p.batch)) if batches is None else batches
    for t in range(steps):
        lengths = list(w.lengths[t]) if lengths_override is None else lengths_override
        qn, qr = w.q_nope[t].contiguous(), w.q_rope[t].contiguous()
        before = raw(dec.kv_exp).copy()
        lens = dev_lengths(lengths)
        dec.step(qn, qr, lens)
        ref_dec.step(qn, qr, lens)
        torch.cuda.synchronize()
        # the same selection as the absorbed step (same scoring and Top-K kernels)
        np.testing.assert_array_equal(dec.sel_idx.cpu().numpy(), ref_dec.sel_idx.cpu().numpy())
        # slots outside this step's load lists keep their bits
        after = raw(dec.kv_exp)
        lc = dec.load_count.cpu().numpy()
        ls = dec.load_slot.cpu().numpy()
        touched = np.zeros(after.shape[:3], dtype=bool)
        for b in range(p.batch):
            for h in range(p.n_q_heads):
                touched[b, h, ls[b, h, :lc[b, h]]] = True
        np.testing.assert_array_equal(after[~touched], before[~touched])
        # the joined query
        np.testing.assert_array_equal(raw(dec.q_exp), np.concatenate([raw(qn), raw(qr)], axis=-1))
        _check_rows(dec, p, lat, w_uk, w_uv, heads, batches)
        # attention against the oracle's literal expansion of the selected rows, stored in bf16
        gsel = sel_lists(dec.sel_idx, dec.sel_count)
        out = dec.out.cpu().numpy()[:, 0].astype(np.float64)
        qn64, qr64 = _bf(qn), _bf(qr)
        for b in batches:
            if int(lengths[b]) == 0:
                assert np.all(out[b] == 0)
                continue
            for h in heads:
                ref = O.mla_sparse_attention(qn64[b, h], qr64[b, h], lat[b][:, :C], lat[b][:, C:], w_uk, w_uv,
                                             gsel[b][h], h, p.scale, stored="bf16")
                err = float(np.max(np.abs(out[b, h] - ref)))
                assert err <= ATTN_MAX_ABS and err <= ATTN_DERIVED, (t, b, h, err)
        # and the absorbed step's output: the same attention without the bf16 storage of K/V
        d = float(np.max(np.abs(out - ref_dec.out.cpu().numpy().astype(np.float64))))
        assert d <= ATTN_MAX_ABS, d
    return dec


def test_literal_small_ragged():
    p = W.PRESETS["mla_32k"].with_(batch=3, n_q_heads=16, max_len=1000, budget=96)
    _run(p, steps=3, seed=7, lengths_override=[1000, 613, 0])


def test_literal_budget_not_multiple_of_16_and_growth():
    p = W.PRESETS["mla_32k"].with_(batch=2, n_q_heads=32, max_len=3000, budget=333)
    _run(p, steps=3, seed=8)


def test_literal_mla_32k_full_shape():
    """4 sequences, 128 heads, 32768 positions, budget 2048: the cold step expands 2048 rows per
    (sequence, head), the next ones only the changed rows (sampled heads checked)."""
    p = W.PRESETS["mla_32k"]
    _run(p, steps=2, seed=9, heads=[0, 77, 127], batches=[0, 3])
