"""Each pin must catch a plausible mistake: plant one in a copy of an oracle
function (on the CPU) and check that the matching pin fails."""
import math

import numpy as np
import pytest

from oracle import spc_oracle as O
from tests import pins


def _scores(q, k, lengths, scale, *, sign=1.0, scale_pow=1.0, head_map="div", mask_len=True):
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    per_kv = Hq // Hkv
    probs = np.zeros((B, Hq, L))
    for b in range(B):
        n = int(lengths[b]) if mask_len else L
        if n == 0:
            continue
        for i in range(Hq):
            g = i // per_kv if head_map == "div" else i % Hkv
            logits = sign * (k[b, g, :n] @ q[b, i]) * scale ** scale_pow
            probs[b, i, :n] = O.softmax(logits)
    return probs


def _fails(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def test_pins_catch_score_mistakes():
    _fails(pins.check_scores_closed_form, lambda *a: _scores(*a, sign=-1.0))
    _fails(pins.check_scores_closed_form, lambda *a: _scores(*a, scale_pow=2.0))
    _fails(pins.check_scores_vs_library, lambda *a: _scores(*a, head_map="mod"))
    _fails(pins.check_scores_length_masking, lambda *a: _scores(*a, mask_len=False))


def test_pins_catch_group_mistakes():
    def mean_groups(p, n_groups):
        B, Hq, L = p.shape
        G = Hq // n_groups
        return p.reshape(B, n_groups, G, L).mean(axis=2)

    def strided_groups(p, n_groups):
        B, Hq, L = p.shape
        return np.stack([p[:, r::n_groups].max(axis=1) for r in range(n_groups)], axis=1)

    _fails(pins.check_group_max_is_max_of_per_head, O.retrieval_scores, mean_groups)
    _fails(pins.check_group_max_is_max_of_per_head, O.retrieval_scores, strided_groups)
    _fails(pins.check_group_modes, mean_groups)


def test_pins_catch_topk_mistakes():
    def high_index_wins(s, n, k):
        if n <= 0:
            return np.zeros(0, dtype=np.int64)
        order = np.lexsort((-np.arange(n), -np.asarray(s[:n])))
        return np.sort(order[:min(k, n)])

    def ascending_scores(s, n, k):
        if n <= 0:
            return np.zeros(0, dtype=np.int64)
        order = np.lexsort((np.arange(n), np.asarray(s[:n])))
        return np.sort(order[:min(k, n)])

    def unsorted_output(s, n, k):
        if n <= 0:
            return np.zeros(0, dtype=np.int64)
        return np.lexsort((np.arange(n), -np.asarray(s[:n])))[:min(k, n)]

    def ignores_length(s, n, k):
        return O.topk_select(s, len(s), k)[:min(k, n)] if n > 0 else np.zeros(0, dtype=np.int64)

    def signed_zeros_apart(s, n, k):       # ranks +0.0 above -0.0, as a key made of the float's bits would
        x = np.asarray(s, dtype=np.float64)
        x = np.where((x == 0) & np.signbit(x), -1e-300, x)
        return O.topk_select(x, n, k)

    for bad in (high_index_wins, ascending_scores, unsorted_output):
        _fails(pins.check_topk_bruteforce, bad)
        _fails(pins.check_topk_python_sorted, bad)
    _fails(pins.check_topk_edge_cases, ignores_length)
    _fails(pins.check_topk_edge_cases, signed_zeros_apart)


def test_pins_catch_plan_mistakes():
    def rebuild_slots(selected, slot_pos):
        # loads everything again into slots 0.. (no reuse, no in-place)
        S = sorted(int(p) for p in selected)
        new = np.full(len(slot_pos), -1); new[:len(S)] = S
        return np.asarray(S), np.arange(len(S)), new

    def descending_freed(selected, slot_pos):
        S = set(int(p) for p in selected)
        slots = [int(p) for p in slot_pos]
        to_load = sorted(S - set(p for p in slots if p != -1))
        freed = sorted((x for x in range(len(slots)) if slots[x] == -1 or slots[x] not in S), reverse=True)
        new = list(slots)
        for i, p in enumerate(to_load):
            new[freed[i]] = p
        for x in freed[len(to_load):]:
            new[x] = -1
        return np.asarray(to_load), np.asarray(freed[:len(to_load)]), np.asarray(new)

    def union_not_difference(selected, slot_pos):
        t, s, new = O.elastic_plan(selected, slot_pos)
        return np.asarray(sorted(int(p) for p in selected)), s, new

    _fails(pins.check_plan_worked_example, rebuild_slots)
    _fails(pins.check_plan_invariants, rebuild_slots)
    _fails(pins.check_plan_invariants, descending_freed)
    _fails(pins.check_plan_worked_example, union_not_difference)


def test_pins_catch_attention_mistakes():
    def no_scale(q, K, V, positions, scale):
        return O.sparse_attention(q, K, V, positions, 1.0)

    def keys_as_values(q, K, V, positions, scale):
        pos = np.asarray(list(positions), dtype=np.int64)
        if pos.size == 0:
            return np.zeros(V.shape[1])
        return O.softmax(K[pos] @ q * scale) @ K[pos][:, :V.shape[1]] if K.shape[1] >= V.shape[1] \
            else O.softmax(K[pos] @ q * scale) @ np.resize(K[pos], (pos.size, V.shape[1]))

    def wrong_head_layer(q, K, V, sel, n_groups, scale):
        B, Hq, _ = q.shape
        Hkv = K.shape[1]
        out = np.zeros((B, Hq, V.shape[-1]))
        for b in range(B):
            for i in range(Hq):
                g = i % Hkv
                out[b, i] = O.sparse_attention(q[b, i], K[b, g], V[b, g], sel[b][g], scale)
        return out

    _fails(pins.check_attention_subset_vs_masked_library, no_scale)
    _fails(pins.check_attention_subset_vs_masked_library, keys_as_values)
    _fails(pins.check_attention_full_budget, O.topk_select, wrong_head_layer)


def test_pins_catch_mla_mistakes():
    def keys_from_value_proj(q_nope, q_rope, latent, rope, W_UK, W_UV, positions, h, scale):
        return O.mla_sparse_attention(q_nope, q_rope, latent, rope, W_UV, W_UV, positions, h, scale)

    def dropped_rope(q_nope, q_rope, latent, rope, W_UK, W_UV, positions, h, scale):
        return O.mla_sparse_attention(q_nope, 0 * q_rope, latent, rope, W_UK, W_UV, positions, h, scale)

    _fails(pins.check_mla_literal_vs_absorbed, keys_from_value_proj, O.mla_retrieval_scores)
    _fails(pins.check_mla_literal_vs_absorbed, dropped_rope, O.mla_retrieval_scores)


def test_pins_catch_size_mistakes():
    _fails(pins.check_kv_cache_size, lambda l, h, d, e, s, b=1: l * h * d * e * s * b)   # forgot K and V


def test_pins_catch_offload_mistakes():
    def last_fitting(gpu, **m):            # the last length that fits instead of the first that does not
        return [t - 1 if 0 < t < 2 ** 31 - 1 else t for t in O.offload_thresholds(gpu, **m)]

    def no_working_set(L, c, **m):         # offloaded layers keep nothing on the GPU
        per = m["batch"] * m["n_kv_heads"] * (m["head_dim"] + m["v_dim"]) * m["elem_bytes"]
        return m["fixed_bytes"] + L * m["token_bytes"] + (m["n_layers"] - c) * L * per

    def strict_loop(L, th, c=0):           # offloads only once the length passes the threshold
        while c < len(th) - 1 and L > th[c]:
            c += 1
        return c

    _fails(pins.check_offload_golden, last_fitting, O.offloaded_layers)
    _fails(pins.check_offload_golden, O.offload_thresholds, strict_loop)
    _fails(pins.check_offload_invariants, O.offload_thresholds, no_working_set)


def test_pins_catch_lag1_plan_mistakes():
    def frees_current(cur, nxt, slots):          # reuses the slots the current step still reads
        return O.elastic_plan_lag1(nxt, nxt, slots)

    def attend_before_update(cur, nxt, slots):   # attended slots taken from the map before the loads
        a, b, new, _ = O.elastic_plan_lag1(cur, nxt, slots)
        c = set(int(p) for p in cur)
        return a, b, new, np.asarray([x for x, p in enumerate(slots) if p in c], dtype=np.int64)

    _fails(pins.check_plan_lag1_worked_example, frees_current)
    _fails(pins.check_plan_lag1_invariants, frees_current)
    _fails(pins.check_plan_lag1_reduces_to_lag0, attend_before_update, O.elastic_plan)


def test_pins_catch_bf16_and_expansion_mistakes():
    from oracle.front import to_bf16_bits

    def half_up(x):                                   # ties away from zero instead of to even
        m, e = np.frexp(np.asarray(x, dtype=np.float64))
        return np.ldexp(np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5), e - 8)

    def truncate(x):
        m, e = np.frexp(np.asarray(x, dtype=np.float64))
        return np.ldexp(np.trunc(m * 256.0), e - 8)

    def seven_bits(x):
        m, e = np.frexp(np.asarray(x, dtype=np.float64))
        return np.ldexp(np.rint(m * 128.0), e - 7)

    _fails(pins.check_round_bf16, half_up, to_bf16_bits)
    _fails(pins.check_round_bf16, truncate, to_bf16_bits)
    _fails(pins.check_round_bf16, seven_bits, to_bf16_bits)

    def swapped(lat, rope, W_UK_h, W_UV_h, stored=None):
        return O.mla_expand_rows(lat, rope, W_UV_h[:W_UK_h.shape[0]] if W_UV_h.shape[0] >= W_UK_h.shape[0]
                                 else np.resize(W_UV_h, W_UK_h.shape), W_UK_h[:W_UV_h.shape[0]], stored)

    def transposed_rows(lat, rope, W_UK_h, W_UV_h, stored=None):
        K, V = O.mla_expand_rows(lat, rope, W_UK_h, W_UV_h, stored)
        return K, V[::-1]                                # rows of V misassigned

    def no_rounding(lat, rope, W_UK_h, W_UV_h, stored=None):
        return O.mla_expand_rows(lat, rope, W_UK_h, W_UV_h, None)

    _fails(pins.check_mla_expand_exact, swapped)
    _fails(pins.check_mla_expand_exact, transposed_rows)
    _fails(pins.check_mla_expand_exact, no_rounding)
