"""Seeded synthetic inputs: determinism, shapes, growth schedule, overlap band (no GPU)."""
import numpy as np
import torch

from oracle import OracleDecoder
from oracle import spc_oracle as O
from speculative_kv_sparsity_amd import workload as W


def test_generator_is_deterministic():
    a = W.generate("tiny", seed=3, steps=2)
    b = W.generate("tiny", seed=3, steps=2)
    c = W.generate("tiny", seed=4, steps=2)
    assert torch.equal(a.dlm_k, b.dlm_k) and torch.equal(a.host_kv, b.host_kv) and torch.equal(a.q, b.q)
    assert not torch.equal(a.dlm_k, c.dlm_k)
    # fewer steps do not shift the other arrays' draws
    d = W.generate("tiny", seed=3, steps=1)
    assert torch.equal(a.dlm_k, d.dlm_k) and torch.equal(a.q[:1], d.q)


def test_shapes_and_dtypes():
    w = W.generate(W.PRESETS["b1_32k"].with_(max_len=256, n_layers=2, budget=16), steps=2)
    assert w.dlm_k.shape == (1, 8, 256, 128) and w.dlm_k.dtype == torch.bfloat16
    assert w.host_kv.shape == (1, 2, 8, 256, 2, 128)
    assert w.q.shape == (2, 1, 32, 128)
    m = W.generate(W.PRESETS["mla_32k"].with_(max_len=64, batch=2, budget=8), steps=2)
    assert m.latent.shape == (2, 64, 576) and m.w_uk.shape == (128, 128, 512)
    assert m.q_nope.shape == (2, 2, 128, 128) and m.q_rope.shape == (2, 2, 128, 64)


def test_growth_schedule():
    p = W.PRESETS["b16_grow"]
    lens = W.lengths_schedule(p, 200, seed=0)
    assert lens.shape == (200, 16)
    assert np.all(lens[0] >= 2048) and np.all(lens[0] <= 2048 + 2047)
    assert np.all(np.diff(lens, axis=0) == 1)
    full = W.lengths_schedule(p, p.steps, seed=0)
    assert full.max() == 16384 and np.all(full[-1] == 16384)


def test_boosted_structure():
    w = W.generate("tiny", seed=0, steps=1)
    m = w.boosted
    assert m[:, :, :4].all() and m[:, :, 4096 - 64:].all()
    frac = m[:, :, 4:4096 - 64].float().mean().item()
    assert 0.04 < frac < 0.06


def test_adjacent_overlap_in_pages_band():
    """Adjacent-step selections overlap in the pages' '>80%' regime (workload sanity)."""
    p = W.PRESETS["tiny"]
    w = W.generate(p, seed=0)
    dec = OracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale, p.dtype)
    k = W.to_numpy_raw(w.dlm_k)
    ovl, prev = [], None
    for t in range(w.steps):
        _, sel = dec.select(W.to_numpy_raw(w.q[t]), k, w.lengths[t])
        if prev is not None:
            ovl += [O.overlap(prev[0][r], sel[0][r]) for r in range(p.n_groups)]
        prev = sel
    assert 0.75 <= float(np.mean(ovl)) <= 0.95
