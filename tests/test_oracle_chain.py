"""The oracle's chaining code against what the pages and the library fix (no GPU), and planted
mistakes in copies of it (on the CPU), each of which a pin must catch."""
import copy

import numpy as np
import pytest

from oracle import spc_oracle as O
from oracle.decoder import LagOneOracleDecoder, OracleDecoder
from tests import pins_chain as C


# ----------------------------------------------------------------------------- the real oracle

def test_decoder_attention_matches_masked_library_attention():
    C.check_decoder_attend_vs_library(OracleDecoder)


def test_decoder_steps_reproduce_the_pages_worked_example():
    C.check_decoder_step_worked_example(OracleDecoder)


def test_lag1_decoder_warm_up_and_worked_example():
    C.check_lag1_decoder_worked_example(LagOneOracleDecoder)


def test_select_all_respects_each_sequence_length():
    C.check_select_all_ragged(O.select_all)


def test_decoder_steps_match_the_stage_functions_composed_by_hand():
    C.check_decoder_matches_stage_composition(OracleDecoder, O)


def test_mla_expand_keys_integer_brute_force():
    C.check_mla_expand_keys_exact(O.mla_expand_keys)


def test_mla_expand_keys_match_the_row_expansion():
    C.check_mla_expand_keys_match_rows(O.mla_expand_keys, O.mla_expand_rows)


# ----------------------------------------------------------------------------- planted mistakes

def _fails(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def _attend_with(dec, q_raw, host_kv_raw, sel, layers, group_of, kv_of, layer_of=lambda li, layer: layer):
    """The decoder's attention loop with the head -> group, head -> KV head and layer maps given."""
    q = O.to_f64(q_raw, dec.dtype)
    out = np.zeros((dec.B, len(layers), dec.Hq, dec.d))
    for li, layer in enumerate(layers):
        for b in range(dec.B):
            for i in range(dec.Hq):
                pos = np.asarray(sel[b][group_of(dec, i)], dtype=np.int64)
                rows = O.to_f64(host_kv_raw[b, layer_of(li, layer), kv_of(dec, i)][pos], dec.dtype)
                out[b, li, i] = O.sparse_attention(q[b, i], rows[:, 0, :], rows[:, 1, :], np.arange(len(pos)),
                                                   dec.scale)
    return out


class _KVSwapped(OracleDecoder):
    def attend(self, q_raw, host_kv_raw, sel, layers):
        return super().attend(q_raw, host_kv_raw[..., ::-1, :], sel, layers)


class _GroupByKVHead(OracleDecoder):          # group index taken from the KV head map
    def attend(self, q_raw, host_kv_raw, sel, layers):
        return _attend_with(self, q_raw, host_kv_raw, sel, layers,
                            lambda d, i: min(i // (d.Hq // d.Hkv), d.G - 1), lambda d, i: i // (d.Hq // d.Hkv))


class _StridedKVHeads(OracleDecoder):         # query head i on KV head i mod H_kv
    def attend(self, q_raw, host_kv_raw, sel, layers):
        return _attend_with(self, q_raw, host_kv_raw, sel, layers,
                            lambda d, i: i // (d.Hq // d.G), lambda d, i: i % d.Hkv)


class _LayerByListIndex(OracleDecoder):       # the position in the layer list used as the layer
    def attend(self, q_raw, host_kv_raw, sel, layers):
        return _attend_with(self, q_raw, host_kv_raw, sel, layers,
                            lambda d, i: i // (d.Hq // d.G), lambda d, i: i // (d.Hq // d.Hkv),
                            layer_of=lambda li, layer: li)


class _SlotMapsNotCarried(OracleDecoder):     # each plan starts from the state before the first step
    def plan(self, sel):
        before = copy.deepcopy(self.slot_pos)
        plans = super().plan(sel)
        self.slot_pos = before
        return plans


class _GroupsOfKVHeads(OracleDecoder):        # the group max taken over the KV heads' groups
    def select(self, q_raw, dlm_k_raw, lengths):
        probs = O.retrieval_scores(O.to_f64(q_raw, self.dtype), O.to_f64(dlm_k_raw, self.dtype), lengths, self.scale)
        return probs, O.select_all(O.group_scores(probs, self.Hkv), lengths, self.K)


class _FirstLengthForAll(OracleDecoder):      # every sequence selected with the first one's length
    def select(self, q_raw, dlm_k_raw, lengths):
        probs = O.retrieval_scores(O.to_f64(q_raw, self.dtype), O.to_f64(dlm_k_raw, self.dtype), lengths, self.scale)
        return probs, O.select_all(O.group_scores(probs, self.G), [lengths[0]] * len(lengths), self.K)


class _NoWarmUp(LagOneOracleDecoder):          # the first step attends an empty previous selection
    def plan_lag1(self, nxt):
        if self.current is None:
            self.current = [[np.zeros(0, dtype=np.int64) for _ in row] for row in nxt]
        return super().plan_lag1(nxt)


class _CurrentNotAdvanced(LagOneOracleDecoder):  # the warm-up selection is served at every step
    def plan_lag1(self, nxt):
        first = self.current
        plans, cur = super().plan_lag1(nxt)
        if first is not None:
            self.current = first
        return plans, cur


def test_pins_catch_decoder_attention_mistakes():
    for bad in (_KVSwapped, _GroupByKVHead, _StridedKVHeads, _LayerByListIndex):
        _fails(C.check_decoder_attend_vs_library, bad)
    _fails(C.check_decoder_matches_stage_composition, _KVSwapped, O)
    _fails(C.check_decoder_matches_stage_composition, _LayerByListIndex, O)


def test_pins_catch_decoder_state_and_selection_mistakes():
    _fails(C.check_decoder_step_worked_example, _SlotMapsNotCarried)
    _fails(C.check_decoder_matches_stage_composition, _SlotMapsNotCarried, O)
    _fails(C.check_decoder_matches_stage_composition, _GroupsOfKVHeads, O)
    _fails(C.check_decoder_matches_stage_composition, _FirstLengthForAll, O)


def test_pins_catch_lag1_warm_up_mistakes():
    _fails(C.check_lag1_decoder_worked_example, _NoWarmUp)
    _fails(C.check_lag1_decoder_worked_example, _CurrentNotAdvanced)


def test_pins_catch_select_all_mistakes():
    def first_length(group, lengths, budget):
        return O.select_all(group, [lengths[0]] * len(lengths), budget)

    def whole_rows(group, lengths, budget):
        return O.select_all(group, [group.shape[2]] * len(lengths), budget)

    def one_past(group, lengths, budget):
        return O.select_all(group, [min(int(n) + 1, group.shape[2]) for n in lengths], budget)

    for bad in (first_length, whole_rows, one_past):
        _fails(C.check_select_all_ragged, bad)


def test_pins_catch_mla_key_expansion_mistakes():
    def heads_shifted(latent, rope, W_UK):
        return O.mla_expand_keys(latent, rope, np.roll(W_UK, 1, axis=0))

    def rope_dropped(latent, rope, W_UK):
        return O.mla_expand_keys(latent, np.zeros_like(rope), W_UK)

    def rope_rows_reversed(latent, rope, W_UK):
        return O.mla_expand_keys(latent, rope[::-1], W_UK)

    def weights_summed_over_heads(latent, rope, W_UK):
        return O.mla_expand_keys(latent, rope, np.broadcast_to(W_UK.sum(axis=0), W_UK.shape))

    for bad in (heads_shifted, rope_dropped, rope_rows_reversed, weights_summed_over_heads):
        _fails(C.check_mla_expand_keys_exact, bad)
        _fails(C.check_mla_expand_keys_match_rows, bad, O.mla_expand_rows)
