"""Plain CPU oracle (NumPy, float64) of the retrieval head's front end.

TEST INFRASTRUCTURE ONLY, like ``spc_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` may use it, and it
imports nothing from the product path.

The retrieval head keeps, of the distilled model's single decoder layer, the
token embedding and the Query/Key projections that produce attention weights
(SpeContext blog, section 5 "C1"; paper summary sections 4.1 and 4.3).  Per
decode step and sequence b, with the new token t_b at position p_b:

  F1  x_b   = E[t_b]                                        embedding row
  F2  x̂_b   = gamma * x_b / sqrt(mean(x_b^2) + eps)          RMS normalisation of
      the layer input (the decoder layer's own input norm: a reading, the pages
      name only "embedding + QK projection")
  F3  q_b   = W_q x̂_b  -> [H_q][d];   k_b = W_k x̂_b -> [H_kv][d]
  F4  rotary position embedding at p_b, with the frequencies extended by YaRN
      (paper summary section 4.1: the DLM's 2K context is extended with
      training-free YaRN), applied to q and k
  F5  q_b is the step's retrieval query; k_b joins the DLM key cache at row p_b
      (it becomes a candidate from the next step on, when the length covers it)

q and k are stored in the cache's element type (bf16 workloads: round to
nearest even), which is what the scoring stage and the key cache hold.

YaRN as published (Peng, Quesnelle, Fan, Shippole, 2023, "YaRN: Efficient
Context Window Extension of Large Language Models"): "NTK-by-parts" interpolation
of the rotary frequencies plus an attention temperature.  For a rotary frequency
theta_i with wavelength lambda_i = 2 pi / theta_i and r_i = L_orig / lambda_i
rotations over the original context,
  gamma_i = clamp((r_i - beta_slow) / (beta_fast - beta_slow), 0, 1)
  theta'_i = gamma_i theta_i + (1 - gamma_i) theta_i / s
(high-frequency dimensions keep theta_i, low-frequency ones are interpolated by
the scale s), and q and k are both multiplied by 0.1 ln(s) + 1, so the logits
carry its square.  s <= 1 gives plain rotary embedding.

Rotary convention: the d dimensions of a head are two halves; dimension i and
i + d/2 form the pair rotated by angle p * theta_i (the "rotate half" layout of
the Llama family the distilled model comes from).
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest even, via float32); returns uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """F2: gamma * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + eps)


def rope_inv_freq(d: int, base: float) -> np.ndarray:
    """Rotary frequencies theta_i = base^(-2i/d), i < d/2."""
    i = np.arange(d // 2, dtype=np.float64)
    return base ** (-2.0 * i / d)


def yarn_inv_freq(d: int, base: float, factor: float, orig_max_pos: int,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """YaRN "NTK-by-parts" frequencies (see the module docstring); factor <= 1: plain RoPE."""
    theta = rope_inv_freq(d, base)
    if factor <= 1.0:
        return theta
    wavelength = 2.0 * math.pi / theta
    r = orig_max_pos / wavelength
    gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return gamma * theta + (1.0 - gamma) * theta / factor


def yarn_mscale(factor: float) -> float:
    """YaRN attention temperature applied to q and k: 0.1 ln(s) + 1 (1 for s <= 1)."""
    return 0.1 * math.log(factor) + 1.0 if factor > 1.0 else 1.0


def apply_rope(x: np.ndarray, pos: float, inv_freq: np.ndarray, mscale: float = 1.0) -> np.ndarray:
    """F4 on the last axis (d): pairs (i, i + d/2) rotated by pos * inv_freq[i], times mscale."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = pos * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return mscale * np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def retrieval_head_qk(tokens: Sequence[int], positions: Sequence[int], emb: np.ndarray, gamma: np.ndarray,
                      wq: np.ndarray, wk: np.ndarray, n_q_heads: int, n_kv_heads: int, head_dim: int,
                      eps: float, base: float, factor: float, orig_max_pos: int,
                      beta_fast: float = 32.0, beta_slow: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """F1-F4 for a batch: q [B][H_q][d] and k [B][H_kv][d] in float64 (before storage rounding).

    emb: [vocab][hidden]; gamma: [hidden]; wq: [H_q * d][hidden]; wk: [H_kv * d][hidden]
    (row h*d + i produces dimension i of head h).  A token outside [0, vocab) gives
    zero q and k (a reading: no embedding row, nothing to project).
    """
    inv = yarn_inv_freq(head_dim, base, factor, orig_max_pos, beta_fast, beta_slow)
    ms = yarn_mscale(factor)
    B = len(tokens)
    q = np.zeros((B, n_q_heads, head_dim))
    k = np.zeros((B, n_kv_heads, head_dim))
    for b in range(B):
        t = int(tokens[b])
        if not 0 <= t < emb.shape[0]:
            continue
        xh = rms_norm(emb[t].astype(np.float64), gamma, eps)
        qb = (wq @ xh).reshape(n_q_heads, head_dim)
        kb = (wk @ xh).reshape(n_kv_heads, head_dim)
        q[b] = apply_rope(qb, float(positions[b]), inv, ms)
        k[b] = apply_rope(kb, float(positions[b]), inv, ms)
    return q, k


def append_keys(dlm_k: np.ndarray, k_new: np.ndarray, positions: Sequence[int]) -> np.ndarray:
    """F5: a copy of the key cache [B][H_kv][L][d] with k_new[b] written at row positions[b]
    (positions outside [0, L) write nothing)."""
    out = np.array(dlm_k, copy=True)
    L = out.shape[2]
    for b, p in enumerate(positions):
        if 0 <= int(p) < L:
            out[b, :, int(p)] = k_new[b]
    return out
