"""The front-end oracle against its pins, and each pin against a planted mistake (CPU only)."""
import math

import numpy as np
import pytest

from oracle import front as F
from tests import pins_front as P


def test_rms_norm():
    P.check_rms_norm(F.rms_norm)


def test_rope_frequencies():
    P.check_rope_frequencies(F.rope_inv_freq)


def test_rope_rotation_is_complex_multiplication():
    P.check_rope_rotation(F.apply_rope, F.rope_inv_freq)


def test_rope_relative_position():
    P.check_rope_relative(F.apply_rope, F.rope_inv_freq)


def test_yarn_limits():
    P.check_yarn(F.yarn_inv_freq, F.yarn_mscale, F.rope_inv_freq)


def test_qk_projection_layout():
    P.check_qk_layout(F.retrieval_head_qk, F.apply_rope, F.yarn_inv_freq, F.yarn_mscale)


def test_append():
    P.check_append(F.append_keys)


def test_bf16_rounding():
    # exact values stay, halfway cases go to even, one ulp above 1 in bf16 is 2^-7
    bits = F.to_bf16_bits(np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0, 0.0]))
    np.testing.assert_array_equal(bits, [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000])


# ----------------------------------------------------------------------------- planted mistakes

def _fails(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def test_pins_catch_rms_mistakes():
    def eps_outside(x, g, eps):
        x = np.asarray(x, dtype=np.float64)
        return g * x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)

    def sum_not_mean(x, g, eps):
        x = np.asarray(x, dtype=np.float64)
        return g * x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)

    def gamma_before(x, g, eps):
        y = np.asarray(g, dtype=np.float64) * x
        return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)

    for bad in (eps_outside, sum_not_mean, gamma_before):
        _fails(P.check_rms_norm, bad)


def test_pins_catch_rope_mistakes():
    def interleaved(x, pos, th, ms=1.0):
        x = np.asarray(x, dtype=np.float64)
        a, b = x[..., 0::2], x[..., 1::2]
        c, s = np.cos(pos * th), np.sin(pos * th)
        out = np.empty_like(x)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
        return ms * out

    def backwards(x, pos, th, ms=1.0):
        return F.apply_rope(x, -pos, th, ms)

    def freq_off_by_one(d, base):
        return base ** (-2.0 * (np.arange(d // 2) + 1) / d)

    _fails(P.check_rope_rotation, interleaved, F.rope_inv_freq)
    _fails(P.check_rope_rotation, backwards, F.rope_inv_freq)
    _fails(P.check_rope_frequencies, freq_off_by_one)


def test_pins_catch_yarn_mistakes():
    def ramp_reversed(d, base, factor, orig, bf=32.0, bs=1.0):
        th = F.rope_inv_freq(d, base)
        if factor <= 1.0:
            return th
        r = orig / (2 * math.pi / th)
        g = np.clip((r - bs) / (bf - bs), 0.0, 1.0)
        return (1 - g) * th + g * th / factor

    def log10_mscale(s):
        return 0.1 * math.log10(s) + 1.0 if s > 1.0 else 1.0

    _fails(P.check_yarn, ramp_reversed, F.yarn_mscale, F.rope_inv_freq)
    _fails(P.check_yarn, F.yarn_inv_freq, log10_mscale, F.rope_inv_freq)


def test_pins_catch_layout_mistakes():
    def head_minor(tokens, positions, emb, gamma, wq, wk, Hq, Hkv, d, eps, base, factor, orig, bf=32.0, bs=1.0):
        q, k = F.retrieval_head_qk(tokens, positions, emb, gamma, wq, wk, Hq, Hkv, d, eps, base, factor, orig,
                                   bf, bs)
        # row i*H + h read as head h, dimension i
        B = q.shape[0]
        return q.reshape(B, d, Hq).transpose(0, 2, 1), k

    def no_temperature(tokens, positions, emb, gamma, wq, wk, Hq, Hkv, d, eps, base, factor, orig, bf=32.0,
                       bs=1.0):
        q, k = F.retrieval_head_qk(tokens, positions, emb, gamma, wq, wk, Hq, Hkv, d, eps, base, factor, orig,
                                   bf, bs)
        m = F.yarn_mscale(factor)
        return q / m, k / m

    _fails(P.check_qk_layout, head_minor, F.apply_rope, F.yarn_inv_freq, F.yarn_mscale)
    _fails(P.check_qk_layout, no_temperature, F.apply_rope, F.yarn_inv_freq, F.yarn_mscale)
