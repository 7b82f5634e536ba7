"""Plain CPU oracle (NumPy, float64) of SpeContext's per-step sparse-KV decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its binding) never imports, calls or links it, and this
module imports nothing from the product path.

Every stage follows the pages' description step by step, in the pages'
notation, with no blocking, fusion or reordering:

  O1  retrieval scores      softmax(q K^T / sqrt(d)) per query head
      (SpeContext blog, section 2 "why only part of the KV cache is needed",
       the AttentionWeight formula; paper summary section 2.1)
  O2  group score           element-wise max over the query heads of a GQA
      group; MQA = one group; MHA = each head on its own
      (blog section 5 "C1 retrieval head"; paper summary section 4.3)
  O3  Top-K selection       the K positions with the largest group score
      (blog section 2, "KV budget"; blog section 4 pseudocode, topk(k=kv_budget))
  O4  elastic plan          to_load = S_now - S_last, written in place into the
      slots freed by positions that left the selection
      (blog section 4 pseudocode; blog section 6 worked example
       {1,8,21,35} -> {1,8,21,50}; paper summary section 5.4 / Figure 7)
  O5  elastic copy          host row -> device slot for every (pos, slot) pair
      (blog section 4 pseudocode: only the rows to load are prefetched)
  O6  sparse attention      softmax(q K_S^T / sqrt(d)) V_S over the selected
      positions only, read from the host store BY POSITION
      (blog section 4 pseudocode llm.forward(..., sparse_kv=resident_kv);
       AttentionWeight formula of blog section 2)
  O6m MLA                   select latent rows, expand ONLY the selected rows to
      per-head K/V with the up-projections, then attend
      (blog section 5 last paragraph; paper summary section 4.3, MLA bullet)
  O7  statistics            adjacent-step overlap, bytes moved vs full reload
      (blog section 6; paper summary sections 1 and 5.3)

Readings taken where the pages are silent:
  * lower index wins a tie in the Top-K;
  * the i-th ascending position to load goes to the i-th ascending freed slot;
  * a sequence with n <= K valid positions selects all n; n = 0 selects none
    and its attention output is zero;
  * query head i belongs to KV head / group i // (H_q / H_kv) (consecutive
    heads share a KV head);
  * MLA scale is 1/sqrt(128 + 64) for scoring and attention.

Inputs are NumPy arrays.  bf16 tensors are passed as their raw uint16 bit
patterns together with ``dtype="bf16"``; ``to_f64`` widens them exactly.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# widening of stored inputs
# ----------------------------------------------------------------------------


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored input array to float64.

    ``dtype`` is ``"f32"`` (float32 values) or ``"bf16"`` (uint16 bit patterns:
    a bfloat16 is the upper half of an IEEE float32, so shifting its 16 bits
    into the top of a 32-bit word gives the float32 with the same value).
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# O1: retrieval scores  (AttentionWeight = softmax(Q K^T / sqrt(d)))
# ----------------------------------------------------------------------------


def softmax(x: np.ndarray) -> np.ndarray:
    """softmax of a 1-D vector, computed with the usual max shift."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return x.copy()
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def retrieval_scores(q: np.ndarray, k: np.ndarray, lengths: Sequence[int],
                     scale: float) -> np.ndarray:
    """Per-head attention weights of the retrieval head over the cached keys.

    q: [B][H_q][d] float64, the retrieval head's query of the new token.
    k: [B][H_kv][L_max][d] float64, the cached DLM keys.
    lengths[b]: number of valid cached positions n of sequence b.
    Returns probs [B][H_q][L_max]: probs[b, i, j] = softmax_j(scale * q_i . k_{g(i), j})
    over j < n, and 0 for j >= n.  g(i) = i // (H_q / H_kv).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    L = k.shape[2]
    assert Hq % Hkv == 0
    per_kv = Hq // Hkv
    probs = np.zeros((B, Hq, L), dtype=np.float64)
    for b in range(B):
        n = int(min(max(int(lengths[b]), 0), L))
        if n == 0:
            continue
        for i in range(Hq):
            g = i // per_kv
            logits = (k[b, g, :n, :] @ q[b, i, :]) * scale
            probs[b, i, :n] = softmax(logits)
    return probs


# ----------------------------------------------------------------------------
# O2: group score (element-wise max over the query heads of a group)
# ----------------------------------------------------------------------------


def group_scores(probs: np.ndarray, n_groups: int) -> np.ndarray:
    """probs [B][H_q][L] -> group scores [B][n_groups][L].

    Group r holds the consecutive query heads r*G .. r*G+G-1, G = H_q / n_groups;
    its score at position j is the element-wise max of those heads' weights.
    GQA: n_groups = H_kv.  MQA: n_groups = 1.  MHA / MLA: n_groups = H_q.
    """
    B, Hq, L = probs.shape
    assert Hq % n_groups == 0
    G = Hq // n_groups
    out = np.empty((B, n_groups, L), dtype=np.float64)
    for b in range(B):
        for r in range(n_groups):
            out[b, r] = np.max(probs[b, r * G:(r + 1) * G, :], axis=0)
    return out


# ----------------------------------------------------------------------------
# O3: Top-K selection
# ----------------------------------------------------------------------------


def topk_select(scores: np.ndarray, n: int, budget: int) -> np.ndarray:
    """The first min(K, n) positions of [0, n) ordered by (score desc, index asc).

    scores: 1-D array of length >= n.  Returns the selected positions sorted
    ascending (int64).  The order is a full sort of the candidates; the lower
    index wins among equal scores.
    """
    n = int(n)
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    s = np.asarray(scores[:n], dtype=np.float64)
    idx = np.arange(n)
    order = np.lexsort((idx, -s))  # primary key: -score; secondary: index
    chosen = order[:min(int(budget), n)]
    return np.sort(chosen).astype(np.int64)


def select_all(group: np.ndarray, lengths: Sequence[int], budget: int) -> List[List[np.ndarray]]:
    """Top-K of every (b, group) instance: returns sel[b][r] (ascending arrays)."""
    B, Gn, _ = group.shape
    return [[topk_select(group[b, r], int(lengths[b]), budget) for r in range(Gn)]
            for b in range(B)]


# ----------------------------------------------------------------------------
# O4: elastic plan (set difference, in-place slot reuse)
# ----------------------------------------------------------------------------


def elastic_plan(selected: Sequence[int], slot_pos: Sequence[int]) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One (b, group) instance of the elastic-loading plan.

    selected: the new selection S_now (any order).
    slot_pos: the resident slot map before the step: slot x holds position
              slot_pos[x], or -1 if empty.  Its non-empty entries are S_last.
    Returns (to_load, load_slot, new_slot_pos):
      to_load   = sorted(S_now - S_last), the positions to copy in;
      freed     = sorted slots that are empty or hold a position not in S_now;
      load_slot = freed[:len(to_load)]: to_load[i] is written into freed[i];
      new_slot_pos: slot map after the step; kept positions never move,
      freed slots left over become -1.
    """
    S_now = set(int(p) for p in selected)
    slots = [int(p) for p in slot_pos]
    S_last = set(p for p in slots if p != -1)
    to_load = sorted(S_now - S_last)
    freed = sorted(x for x in range(len(slots)) if slots[x] == -1 or slots[x] not in S_now)
    assert len(to_load) <= len(freed), "budget exceeded: more positions to load than free slots"
    new = list(slots)
    for i, pos in enumerate(to_load):
        new[freed[i]] = pos
    for x in freed[len(to_load):]:
        new[x] = -1
    return (np.asarray(to_load, dtype=np.int64),
            np.asarray(freed[:len(to_load)], dtype=np.int64),
            np.asarray(new, dtype=np.int64))


def elastic_plan_lag1(current: Sequence[int], nxt: Sequence[int], slot_pos: Sequence[int]
                      ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """The elastic plan of the pipelined loop (blog section 4: while the target model attends over
    the sparse KV loaded in the previous iteration, the retrieval head already selects the positions
    for the following one).

    current: S_t, the selection the target model attends over in this step (loaded in the previous one);
    nxt:     S_t+1, the selection the retrieval head just made for the next step;
    slot_pos: the pool's slot map before the step (-1 = empty).
    A slot may be overwritten only if its position is in neither selection: the current one is
    being read by this step's attention, the next one will be (paper summary section 5.4 keeps three
    sets: the previous selection, the current one and what is resident).  Returns (to_load, load_slot, new_slot_pos,
    attend_slots): to_load = sorted(S_t+1 - resident) into the ascending free slots, leftover free
    slots emptied, and the ascending slots holding S_t after the update.
    """
    keep = set(int(p) for p in current) | set(int(p) for p in nxt)
    slots = [int(p) for p in slot_pos]
    resident = set(p for p in slots if p != -1)
    to_load = sorted(set(int(p) for p in nxt) - resident)
    free = sorted(x for x in range(len(slots)) if slots[x] == -1 or slots[x] not in keep)
    assert len(to_load) <= len(free), "pool exceeded: more positions to load than free slots"
    new = list(slots)
    for i, pos in enumerate(to_load):
        new[free[i]] = pos
    for x in free[len(to_load):]:
        new[x] = -1
    cur = set(int(p) for p in current)
    attend = sorted(x for x in range(len(new)) if new[x] in cur)
    return (np.asarray(to_load, dtype=np.int64), np.asarray(free[:len(to_load)], dtype=np.int64),
            np.asarray(new, dtype=np.int64), np.asarray(attend, dtype=np.int64))


# ----------------------------------------------------------------------------
# O5: elastic copy
# ----------------------------------------------------------------------------


def elastic_copy(host_rows: np.ndarray, dev_rows: np.ndarray,
                 to_load: Sequence[int], load_slot: Sequence[int]) -> None:
    """dev_rows[slot] <- host_rows[pos] for every (pos, slot) pair (any dtype, exact)."""
    for pos, slot in zip(to_load, load_slot):
        dev_rows[int(slot)] = host_rows[int(pos)]


# ----------------------------------------------------------------------------
# O6: sparse decode attention over the selected positions
# ----------------------------------------------------------------------------


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     positions: Sequence[int], scale: float) -> np.ndarray:
    """softmax(scale * q . K[j]) weighted sum of V[j] over j in positions.

    q: [d]; K: [L][d]; V: [L][dv]; returns [dv] (zeros if positions is empty).
    """
    pos = np.asarray(list(positions), dtype=np.int64)
    if pos.size == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    logits = (K[pos] @ q) * scale
    w = softmax(logits)
    return w @ V[pos]


def sparse_decode_layer(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                        sel: List[List[np.ndarray]], n_groups: int, scale: float) -> np.ndarray:
    """All query heads of one target layer.

    q: [B][H_q][d]; K, V: [B][H_kv][L][d] (read by position);
    sel[b][r]: selected positions of group r, shared by its query heads.
    Query head i reads group r = i // (H_q / n_groups) and KV head
    i // (H_q / H_kv).  Returns [B][H_q][dv].
    """
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    Gq = Hq // n_groups
    per_kv = Hq // Hkv
    out = np.zeros((B, Hq, V.shape[-1]), dtype=np.float64)
    for b in range(B):
        for i in range(Hq):
            r = i // Gq
            g = i // per_kv
            out[b, i] = sparse_attention(q[b, i], K[b, g], V[b, g], sel[b][r], scale)
    return out


# ----------------------------------------------------------------------------
# O1/O6 for MLA: latent cache, literal expansion of the selected rows
# ----------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits), ties to even,
    returned as float64.  For finite values in bf16's normal range: x = m 2^e with
    0.5 <= |m| < 1 (frexp); the 8 significant bits are m 2^8 rounded half to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def mla_expand_rows(latent_rows: np.ndarray, rope_rows: np.ndarray, W_UK_h: np.ndarray, W_UV_h: np.ndarray,
                    stored: str | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """One head's literal expansion of latent rows (SpeContext blog section 5, last
    paragraph; paper summary section 4.3, MLA bullet: 512 -> 128 x 128 K/V up-projection):
    K[j] = (W_UK_h c_j) || r_j and V[j] = W_UV_h c_j.

    latent_rows: [n][C]; rope_rows: [n][R]; W_UK_h: [dn][C]; W_UV_h: [dv][C].
    stored="bf16": the up-projected parts are rounded to bf16 (nearest, ties to even) as a
    bf16 K/V cache holds them; the rotary dims are cache values already.  Returns (K, V).
    """
    Kn = np.asarray(latent_rows, dtype=np.float64) @ np.asarray(W_UK_h, dtype=np.float64).T
    V = np.asarray(latent_rows, dtype=np.float64) @ np.asarray(W_UV_h, dtype=np.float64).T
    if stored == "bf16":
        Kn, V = round_bf16(Kn), round_bf16(V)
    elif stored is not None:
        raise ValueError(stored)
    return np.concatenate([Kn, np.asarray(rope_rows, dtype=np.float64)], axis=1), V


def mla_expand_keys(latent: np.ndarray, rope: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """Per-head keys of the given latent rows: K_h[j] = (W_UK[h] c_j) || r_j.

    latent: [n][C]; rope: [n][R]; W_UK: [H][dn][C].  Returns [H][n][dn + R].
    """
    H = W_UK.shape[0]
    n = latent.shape[0]
    out = np.empty((H, n, W_UK.shape[1] + rope.shape[1]), dtype=np.float64)
    for h in range(H):
        out[h, :, :W_UK.shape[1]] = latent @ W_UK[h].T
        out[h, :, W_UK.shape[1]:] = rope
    return out


def mla_retrieval_scores(q_nope: np.ndarray, q_rope: np.ndarray, latent: np.ndarray,
                         rope: np.ndarray, W_UK: np.ndarray, lengths: Sequence[int],
                         scale: float, heads: Sequence[int] | None = None) -> Dict[Tuple[int, int], np.ndarray]:
    """Head-level retrieval scores over the MLA latent cache, keys expanded literally.

    q_nope: [B][H][dn]; q_rope: [B][H][R]; latent: [B][L][C]; rope: [B][L][R];
    W_UK: [H][dn][C].  Returns {(b, h): probs over the n valid positions}.
    ``heads`` restricts the heads evaluated (all by default).
    """
    B, H, _ = q_nope.shape
    out = {}
    hs = range(H) if heads is None else heads
    for b in range(B):
        n = int(lengths[b])
        for h in hs:
            if n <= 0:
                out[(b, h)] = np.zeros(0)
                continue
            Kh = np.concatenate([latent[b, :n] @ W_UK[h].T, rope[b, :n]], axis=1)
            qh = np.concatenate([q_nope[b, h], q_rope[b, h]])
            out[(b, h)] = softmax((Kh @ qh) * scale)
    return out


def mla_sparse_attention(q_nope: np.ndarray, q_rope: np.ndarray, latent: np.ndarray,
                         rope: np.ndarray, W_UK: np.ndarray, W_UV: np.ndarray,
                         positions: Sequence[int], h: int, scale: float,
                         stored: str | None = None) -> np.ndarray:
    """One MLA head over its selected latent rows, expanding ONLY those rows.

    K_h[j] = (W_UK[h] c_j) || r_j,  V_h[j] = W_UV[h] c_j, for j in positions
    (mla_expand_rows; stored="bf16" rounds them as a bf16 cache of expanded rows holds them);
    then out = softmax(scale * q . K_h[j]) weighted sum of V_h[j].
    q_nope: [dn]; q_rope: [R]; latent: [L][C]; rope: [L][R]; W_UK, W_UV: [H][d][C].
    """
    pos = np.asarray(list(positions), dtype=np.int64)
    if pos.size == 0:
        return np.zeros(W_UV.shape[1], dtype=np.float64)
    K, V = mla_expand_rows(latent[pos], rope[pos], W_UK[h], W_UV[h], stored)
    q = np.concatenate([q_nope, q_rope])
    w = softmax((K @ q) * scale)
    return w @ V


# ----------------------------------------------------------------------------
# O7: statistics the pages quote
# ----------------------------------------------------------------------------


def overlap(prev: Sequence[int], now: Sequence[int]) -> float:
    """|S_now intersect S_prev| / |S_now| (1.0 for an empty S_now)."""
    now = set(int(x) for x in now)
    if not now:
        return 1.0
    return len(now & set(int(x) for x in prev)) / len(now)


def transfer_fraction(n_loaded: int, n_full: int) -> float:
    """Rows moved by elastic loading over the rows a full reload would move."""
    return n_loaded / n_full if n_full else 0.0


def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int,
                   seq_len: int, batch: int = 1) -> int:
    """Size of a full K+V cache: layers x KV heads x d x (K and V) x bytes x L x B."""
    return n_layers * n_kv_heads * head_dim * 2 * elem_bytes * seq_len * batch


def default_scale(head_dim: int) -> float:
    """1/sqrt(d), the scale of the AttentionWeight formula."""
    return 1.0 / math.sqrt(head_dim)


# ----------------------------------------------------------------------------
# Adaptive memory management: per-layer offload thresholds
# (blog section 7 "C3"; paper summary sections 6.1-6.2.1)
# ----------------------------------------------------------------------------

INT32_MAX = 2 ** 31 - 1


def memory_bytes(seq_len: int, n_offloaded: int, fixed_bytes: int, token_bytes: int, n_layers: int, batch: int,
                 n_kv_heads: int, head_dim: int, v_dim: int, budget: int, elem_bytes: int) -> int:
    """GPU memory at sequence length L with the last c layers offloaded: everything independent of L,
    the per-position state outside the target KV, the full K/V of the layers kept on the GPU, and the
    budget-sized working set of each offloaded layer (the pages' four inputs: the model's weights and
    layers, KV heads and head dimension, the requests and the KV budget)."""
    per_layer_token = batch * n_kv_heads * (head_dim + v_dim) * elem_bytes
    return (fixed_bytes + seq_len * token_bytes + (n_layers - n_offloaded) * seq_len * per_layer_token
            + n_offloaded * budget * per_layer_token)


def offload_thresholds(gpu_bytes: int, **model) -> List[int]:
    """threshold[c] for c = 0..n_layers: the first sequence length at which c offloaded layers no
    longer fit in gpu_bytes (0: not even an empty cache fits; INT32_MAX: never within int32).
    Found by bisection on the plain memory sum."""
    out = []
    for c in range(model["n_layers"] + 1):
        if memory_bytes(0, c, **model) > gpu_bytes:
            out.append(0)
            continue
        if memory_bytes(INT32_MAX - 1, c, **model) <= gpu_bytes:
            out.append(INT32_MAX)
            continue
        lo, hi = 0, INT32_MAX - 1            # fits at lo, not at hi
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if memory_bytes(mid, c, **model) <= gpu_bytes:
                lo = mid
            else:
                hi = mid
        out.append(hi)
    return out


def offloaded_layers(seq_len: int, thresholds: Sequence[int], n_offloaded: int = 0) -> int:
    """The pages' runtime loop: while the length reaches the threshold of the current count,
    offload one more layer (the last one still on the GPU)."""
    c = n_offloaded
    while c < len(thresholds) - 1 and seq_len >= thresholds[c]:
        c += 1
    return c
