"""Checks that pin the front-end oracle (oracle/front.py) to facts fixed outside of it.

As in pins.py, each check takes the oracle functions it pins as arguments, so
test_oracle_front.py runs it against the oracle and against broken copies.

Sources of truth, none of them the oracle's formula retyped:
  * closed forms (RMS norm of constant and two-element vectors);
  * an independent formulation: the rotation of each dimension pair as a complex
    multiplication by exp(i p theta) (NumPy complex arithmetic);
  * invariants of rotary embeddings (relative position, norm preservation,
    position 0 is the identity);
  * the defining limits of YaRN's interpolation: unchanged high-frequency
    dimensions, fully interpolated (theta / s) low-frequency dimensions, plain
    rotary embedding at s = 1, and the temperature 0.1 ln(s) + 1 at known s;
  * identity projection weights, which expose the head / dimension layout.
"""
from __future__ import annotations

import math

import numpy as np


def check_rms_norm(rms_norm):
    # constant vector: mean(x^2) = c^2
    for c, eps in ((2.5, 0.0), (-3.0, 0.0), (0.5, 1e-2)):
        x = np.full(64, c)
        np.testing.assert_allclose(rms_norm(x, np.ones(64), eps), np.full(64, c / math.sqrt(c * c + eps)),
                                   rtol=1e-14)
    # (3, 4): mean square 12.5
    np.testing.assert_allclose(rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0),
                               np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=1e-14)
    rng = np.random.default_rng(0)
    x = rng.standard_normal(256)
    g = rng.standard_normal(256)
    # scale invariance (eps = 0) and gamma applied element-wise after the normalisation
    np.testing.assert_allclose(rms_norm(7.0 * x, np.ones(256), 0.0), rms_norm(x, np.ones(256), 0.0), rtol=1e-12)
    np.testing.assert_allclose(rms_norm(x, g, 1e-5), g * rms_norm(x, np.ones(256), 1e-5), rtol=1e-12)


def check_rope_frequencies(rope_inv_freq):
    d, base = 128, 500000.0
    th = rope_inv_freq(d, base)
    assert th.shape == (d // 2,)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[:-1] / th[1:], np.full(d // 2 - 1, base ** (2.0 / d)), rtol=1e-12)
    np.testing.assert_allclose(th[-1], base ** (-(d - 2) / d), rtol=1e-12)


def check_rope_rotation(apply_rope, rope_inv_freq):
    """Against complex multiplication: z_i = x_i + j x_{i+d/2} goes to z_i exp(j p theta_i)."""
    rng = np.random.default_rng(1)
    d = 16
    th = rope_inv_freq(d, 10000.0)
    x = rng.standard_normal((3, d))
    for p in (0.0, 1.0, 7.0, 12345.0):
        z = (x[:, :d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * p * th)
        want = np.concatenate([z.real, z.imag], axis=-1)
        np.testing.assert_allclose(apply_rope(x, p, th), want, rtol=1e-9, atol=1e-12)
    # mscale multiplies the rotated vector
    np.testing.assert_allclose(apply_rope(x, 5.0, th, 1.5), 1.5 * apply_rope(x, 5.0, th), rtol=1e-12)


def check_rope_relative(apply_rope, rope_inv_freq):
    """q.k after rotation depends on the position difference only; pair norms are kept."""
    rng = np.random.default_rng(2)
    d = 32
    th = rope_inv_freq(d, 10000.0)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = apply_rope(q, 100.0, th) @ apply_rope(k, 37.0, th)
    b = apply_rope(q, 1100.0, th) @ apply_rope(k, 1037.0, th)
    assert abs(a - b) < 1e-9 * max(1.0, abs(a))
    r = apply_rope(q, 321.0, th)
    np.testing.assert_allclose(r[:d // 2] ** 2 + r[d // 2:] ** 2, q[:d // 2] ** 2 + q[d // 2:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(apply_rope(q, 0.0, th), q, rtol=0, atol=0)


def check_yarn(yarn_inv_freq, yarn_mscale, rope_inv_freq):
    d, base, orig = 128, 500000.0, 2048
    th = rope_inv_freq(d, base)
    np.testing.assert_allclose(yarn_inv_freq(d, base, 1.0, orig), th, rtol=0, atol=0)
    for s in (4.0, 16.0):
        y = yarn_inv_freq(d, base, s, orig, 32.0, 1.0)
        wavelength = 2.0 * math.pi / th
        fast = orig / wavelength > 32.0          # many rotations over the original context
        slow = orig / wavelength < 1.0           # less than one rotation
        assert fast.any() and slow.any()
        np.testing.assert_allclose(y[fast], th[fast], rtol=1e-15)
        np.testing.assert_allclose(y[slow], th[slow] / s, rtol=1e-12)
        mid = ~fast & ~slow
        assert np.all(y[mid] <= th[mid] * (1 + 1e-12)) and np.all(y[mid] >= th[mid] / s * (1 - 1e-12))
        assert np.all(np.diff(y) < 0)            # frequencies keep their order
    assert yarn_mscale(1.0) == 1.0 and yarn_mscale(0.5) == 1.0
    assert abs(yarn_mscale(math.e) - 1.1) < 1e-12
    assert abs(yarn_mscale(math.e ** 5) - 1.5) < 1e-12


def check_qk_layout(retrieval_head_qk, apply_rope, yarn_inv_freq, yarn_mscale):
    """Identity projections expose the layout: row h*d + i of W_q is dimension i of head h."""
    hidden, Hq, Hkv, d = 8, 2, 1, 4
    rng = np.random.default_rng(3)
    emb = rng.standard_normal((5, hidden))
    gamma = np.ones(hidden)
    wq = np.eye(hidden)
    wk = np.eye(hidden)[4:8]
    q, k = retrieval_head_qk([3, 1, 9], [0, 0, 0], emb, gamma, wq, wk, Hq, Hkv, d, 0.0, 10000.0, 1.0, 2048)
    for b, t in enumerate((3, 1)):
        xh = emb[t] / math.sqrt(np.mean(emb[t] ** 2))
        np.testing.assert_allclose(q[b], xh.reshape(Hq, d), rtol=1e-12)
        np.testing.assert_allclose(k[b, 0], xh[4:8], rtol=1e-12)
    assert np.all(q[2] == 0) and np.all(k[2] == 0)      # a token outside the vocabulary
    # rotation at the token's own position, with the YaRN frequencies and temperature
    s, orig = 8.0, 64
    q2, k2 = retrieval_head_qk([3], [50], emb, gamma, wq, wk, Hq, Hkv, d, 0.0, 10000.0, s, orig)
    q0, k0 = retrieval_head_qk([3], [0], emb, gamma, wq, wk, Hq, Hkv, d, 0.0, 10000.0, s, orig)
    inv = yarn_inv_freq(d, 10000.0, s, orig)
    ms = yarn_mscale(s)
    np.testing.assert_allclose(q0[0], ms * q[0], rtol=1e-12)
    np.testing.assert_allclose(q2[0], apply_rope(q[0], 50.0, inv, ms), rtol=1e-12)
    np.testing.assert_allclose(k2[0], apply_rope(k[0], 50.0, inv, ms), rtol=1e-12)


def check_append(append_keys):
    cache = np.arange(2 * 1 * 5 * 3, dtype=np.float64).reshape(2, 1, 5, 3)
    new = -np.ones((2, 1, 3)) * np.array([[[1.0]], [[2.0]]])
    out = append_keys(cache, new, [4, 5])
    np.testing.assert_array_equal(out[0, 0, 4], [-1.0, -1.0, -1.0])
    np.testing.assert_array_equal(out[0, 0, :4], cache[0, 0, :4])
    np.testing.assert_array_equal(out[1], cache[1])           # position 5 is past the cache
    np.testing.assert_array_equal(cache.ravel()[:3], [0.0, 1.0, 2.0])   # input untouched
