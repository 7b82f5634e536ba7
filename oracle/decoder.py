"""Step-by-step CPU oracle of one whole decode step (O1 -> O6), with state.

TEST INFRASTRUCTURE ONLY (see spc_oracle.py).  It chains the per-stage
definitions of spc_oracle in the order of the SpeContext blog's section 4
pseudocode: retrieval head scores and Top-K, to_load = selected - resident,
prefetch of to_load, attention over the resident sparse KV, resident = selected.

The selection of step t is used by the attention of step t (the retrieval head
runs before the target model on the same input, paper summary section 5.1).
Attention reads the selected positions straight from the host store, never
from the slots, so a wrong slot assignment on the device side cannot hide.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import spc_oracle as O


class OracleDecoder:
    """Keeps the slot maps of every (b, group) and runs O1..O6 per step.

    host_kv: raw array [B][layers][H_kv][L][2][d] (K at [...,0,:], V at [...,1,:]).
    All raw arrays are widened with ``dtype`` ("f32" or "bf16").
    """

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, n_groups: int,
                 head_dim: int, budget: int, scale: float, dtype: str):
        self.B, self.Hq, self.Hkv, self.G = batch, n_q_heads, n_kv_heads, n_groups
        self.d, self.K, self.scale, self.dtype = head_dim, budget, scale, dtype
        self.slot_pos = [[np.full(budget, -1, dtype=np.int64) for _ in range(n_groups)]
                         for _ in range(batch)]
        self.prev_sel: Optional[List[List[np.ndarray]]] = None

    def select(self, q_raw: np.ndarray, dlm_k_raw: np.ndarray, lengths: Sequence[int]):
        """O1 -> O3: returns (probs [B][Hq][L], sel[b][r])."""
        q = O.to_f64(q_raw, self.dtype)
        k = O.to_f64(dlm_k_raw, self.dtype)
        probs = O.retrieval_scores(q, k, lengths, self.scale)
        grp = O.group_scores(probs, self.G)
        sel = O.select_all(grp, lengths, self.K)
        return probs, sel

    def plan(self, sel: List[List[np.ndarray]]):
        """O4 on every instance; updates the slot maps; returns plans[b][r] = (to_load, load_slot)."""
        plans = []
        for b in range(self.B):
            row = []
            for r in range(self.G):
                to_load, load_slot, new = O.elastic_plan(sel[b][r], self.slot_pos[b][r])
                self.slot_pos[b][r] = new
                row.append((to_load, load_slot))
            plans.append(row)
        return plans

    def attend(self, q_raw: np.ndarray, host_kv_raw: np.ndarray, sel: List[List[np.ndarray]],
               layers: Sequence[int]) -> np.ndarray:
        """O6 for the given layers, K/V read by position from the host store.

        Returns out [B][len(layers)][Hq][d].
        """
        q = O.to_f64(q_raw, self.dtype)
        out = np.zeros((self.B, len(layers), self.Hq, self.d), dtype=np.float64)
        Gq = self.Hq // self.G
        per_kv = self.Hq // self.Hkv
        for li, layer in enumerate(layers):
            for b in range(self.B):
                for i in range(self.Hq):
                    r, g = i // Gq, i // per_kv
                    pos = np.asarray(sel[b][r], dtype=np.int64)
                    rows = O.to_f64(host_kv_raw[b, layer, g][pos], self.dtype)   # [n][2][d]
                    out[b, li, i] = O.sparse_attention(q[b, i], rows[:, 0, :], rows[:, 1, :],
                                                       np.arange(len(pos)), self.scale)
        return out

    def step(self, q_raw, dlm_k_raw, lengths, host_kv_raw, layers: Sequence[int]):
        probs, sel = self.select(q_raw, dlm_k_raw, lengths)
        plans = self.plan(sel)
        out = self.attend(q_raw, host_kv_raw, sel, layers)
        stats = None
        if self.prev_sel is not None:
            stats = [[O.overlap(self.prev_sel[b][r], sel[b][r]) for r in range(self.G)]
                     for b in range(self.B)]
        self.prev_sel = sel
        return dict(probs=probs, sel=sel, plans=plans, out=out, overlap=stats)


class LagOneOracleDecoder(OracleDecoder):
    """The pipelined loop of the blog's section 4: at step t the retrieval head's selection S_t+1
    (from token t) is loaded while the target model attends over S_t, the selection made at the
    previous step.  The first step has no previous selection: it attends over its own (the
    pipeline's warm-up, which the blog's pseudocode omits).  The slots form a pool of ``pool``
    entries per (b, group) (the union of two selections must fit)."""

    def __init__(self, batch, n_q_heads, n_kv_heads, n_groups, head_dim, budget, scale, dtype, pool: int):
        super().__init__(batch, n_q_heads, n_kv_heads, n_groups, head_dim, budget, scale, dtype)
        self.slot_pos = [[np.full(pool, -1, dtype=np.int64) for _ in range(n_groups)] for _ in range(batch)]
        self.current: Optional[List[List[np.ndarray]]] = None

    def plan_lag1(self, nxt: List[List[np.ndarray]]):
        """O4 of the pipelined loop; returns (plans[b][r] = (to_load, load_slot, attend_slots), current)."""
        cur = nxt if self.current is None else self.current
        plans = []
        for b in range(self.B):
            row = []
            for r in range(self.G):
                to_load, load_slot, new, attend = O.elastic_plan_lag1(cur[b][r], nxt[b][r], self.slot_pos[b][r])
                self.slot_pos[b][r] = new
                row.append((to_load, load_slot, attend))
            plans.append(row)
        self.current = nxt
        return plans, cur
