"""One sparse-KV decode step ordered on HIP streams (host-side ordering only).

SpeContext's dataflow (blog section 4; paper summary section 5.1): the
retrieval head runs first on the step's input, its Top-K selection drives the
elastic load of the missing K/V rows, and the target model's attention
consumes the resident sparse KV while later layers are still loading.  Here:

  main stream : scores -> group max / Top-K -> plan -> copy(chunk 0) -ev_copy[0]-> copy(chunk 1) ... copy(last)
                -> attention(last chunk) -> wait ev_attn
  side stream :                   wait ev_copy[c] -> attention(chunk c) ... -> ev_attn   (every chunk but the last)

The copy is on the critical path, so it runs on the stream of the stages it
depends on and starts without a cross-stream hand-off; the attention of the
earlier layer chunks overlaps the remaining copies on the side stream.  The
last chunk is the short one (its attention is the only compute left after the
last copy).  The next step's scores are ordered after every attention of this
step (the next query depends on this step's output), and so is the next plan,
which frees slots those attentions read.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import api
from .workload import FrontWeights, Preset


class RetrievalHead:
    """The retrieval head's front end: the new token of each sequence -> the stage-1 query; its key
    is appended to the DLM key cache at the token's position (SpeContext blog section 5 "C1")."""

    def __init__(self, shape, fw: FrontWeights):
        self.shape = shape
        self.fw = fw
        self.rope = api.rope_params(fw.rope_base, fw.rope_factor, fw.rope_orig)
        self.ws = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_FRONT, shape)), dtype=torch.uint8,
                              device=fw.emb.device)

    def __call__(self, tokens: torch.Tensor, positions: torch.Tensor, q_out: torch.Tensor, dlm_k: torch.Tensor,
                 stream=None) -> None:
        fw = self.fw
        api.spc_retrieval_head_qk(self.shape, fw.hidden, self.rope, fw.eps, tokens, positions, fw.emb, fw.gamma,
                                  fw.wq, fw.wk, q_out, dlm_k, ws=self.ws, stream=stream)


class SparseDecoder:
    """Device buffers, state and streams of the sparse decode path for one workload.

    dlm_k:   device [B][H_kv][L][d]  retrieval-head key cache
    host_kv: pinned host [B][layers][H_kv][L][2][d]  full target K/V store

    ``thresholds`` (optional, from ``api.spc_offload_thresholds``) turns on adaptive offloading
    (SpeContext blog section 7 "C3"; paper summary section 6.2): the decoder starts with every
    layer's full K/V on the GPU and offloads the last layer still there each time the sequence
    length reaches the next threshold (``offload_for``).  GPU-resident layers attend over the
    selected positions gathered from their full cache; offloaded layers use the elastic slots.
    Without thresholds every layer is offloaded from the start (the host-resident workloads).
    """

    def __init__(self, p: Preset, dlm_k: torch.Tensor, host_kv: torch.Tensor, layer_chunks: int = 2,
                 tail_layers: Optional[int] = None, device: Optional[torch.device] = None,
                 thresholds: Optional[List[int]] = None):
        assert p.kind in ("gqa", "mha", "mqa"), "MLA uses MlaDecoder"
        self.p = p
        dev = device or dlm_k.device
        self.device = dev
        B, Hq, Hkv, G, d, L, K = p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.max_len, p.budget
        self.shape = api.make_shape(B, Hq, Hkv, G, d, p.v_dim, L, K, p.n_layers, p.dtype, p.scale)
        self.dlm_k = dlm_k
        self.host_kv = host_kv
        self.host_l = api.kv_layout(host_kv)
        i32 = dict(dtype=torch.int32, device=dev)
        # stage 1 in log-domain form: logits + per-tile (max, sum exp); stage 2 ranks them directly.
        # With one query head per group the ranking needs no stats, and stage 1 computes none
        self.logits = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
        self.tile_stats = torch.empty(api.tile_stats_shape(self.shape), dtype=torch.float32, device=dev)
        self.stats_out = self.tile_stats if Hq > G else None
        self.sel_idx = torch.empty((B, G, K), **i32)
        self.sel_count = torch.empty((B, G), **i32)
        self.slot_pos = torch.empty((B, G, K), **i32)
        self.resident_bm = torch.empty((B, G, (L + 31) // 32), **i32)
        self.load_pos = torch.empty((B, G, K), **i32)
        self.load_slot = torch.empty((B, G, K), **i32)
        self.load_count = torch.empty((B, G), **i32)
        self.dev_kv = torch.zeros((B, p.n_layers, Hkv, K, 2, d), dtype=p.torch_dtype, device=dev)
        self.dev_l = api.kv_layout(self.dev_kv)
        self.out = torch.zeros((B, p.n_layers, Hq, p.v_dim), dtype=torch.float32, device=dev)
        self.ws_topk = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_TOPK, self.shape)),
                                   dtype=torch.uint8, device=dev)
        self.q_l = api.q_layout(Hq * d, 0, d)   # the same query serves every layer
        self.layer_chunks, self.tail_layers = layer_chunks, tail_layers
        self.thresholds = list(thresholds) if thresholds is not None else None
        if self.thresholds is None:
            self.n_off = p.n_layers
            self.full_kv = None
        else:
            # every layer's full K/V on the GPU to start with (the prefill's cache)
            self.n_off = 0
            self.full_kv = torch.empty((B, p.n_layers, Hkv, L, 2, d), dtype=p.torch_dtype, device=dev)
            self.full_kv.copy_(host_kv)
            self.full_l = api.kv_layout(self.full_kv)
            # a full reload of an offloaded layer: every slot x from host row slot_pos[x]
            self.all_slots = torch.arange(K, dtype=torch.int32, device=dev).repeat(B, G, 1).contiguous()
            self.all_count = torch.full((B, G), K, **i32)
        self.main = torch.cuda.current_stream(dev)
        self.side = torch.cuda.Stream(device=dev)
        self.ev_sel = torch.cuda.Event()
        self.ev_attn = torch.cuda.Event()
        self._layout()
        self.reset()

    def _layout(self) -> None:
        """Layer chunks of the offloaded layers [n_res, n_layers) and the events / workspaces they need."""
        p = self.p
        self.n_res = p.n_layers - self.n_off
        self.chunks: List[tuple] = []
        if self.n_off:
            self.chunks = [(self.n_res + a, self.n_res + z)
                           for a, z in layer_chunk_bounds(self.n_off, self.layer_chunks, self.tail_layers)]
        self.ev_copy = [torch.cuda.Event() for _ in self.chunks]
        # one attention workspace per call that may run concurrently: the resident layers + each chunk
        n_ws = len(self.chunks) + 1
        if not hasattr(self, "ws_attn") or len(self.ws_attn) < n_ws:
            self.ws_attn = [torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_ATTN, self.shape)),
                                        dtype=torch.uint8, device=self.device) for _ in range(n_ws)]

    def reset(self, batch_index: int = -1) -> None:
        api.spc_elastic_reset(self.shape, batch_index, self.slot_pos, self.resident_bm, stream=self.main)

    def offload_for(self, seq_len: int) -> int:
        """The pages' rule: while seq_len reaches the threshold of the current count, offload the last
        layer still on the GPU.  A newly offloaded layer's slots are filled with the rows of the
        current resident set (the next plan then loads only what changes).  Returns the count."""
        if self.thresholds is None:
            return self.n_off
        c = self.n_off
        while c < self.p.n_layers and seq_len >= self.thresholds[c]:
            c += 1
        if c > self.n_off:
            a, z = self.p.n_layers - c, self.p.n_layers - self.n_off
            api.spc_elastic_update(self.shape, None, None, None, None, self.slot_pos, self.all_slots, self.all_count,
                                   self.host_kv, self.host_l, self.dev_kv, self.dev_l, a, z, flags=api.SPC_COPY,
                                   plan_stream=self.main, copy_stream=self.main)
            self.n_off = c
            self._layout()
        return self.n_off

    # --- the four stages --------------------------------------------------------------
    def scores(self, q: torch.Tensor, lengths: torch.Tensor) -> None:
        api.spc_retrieval_logits(self.shape, q, self.dlm_k, lengths, self.logits, self.stats_out, stream=self.main)

    def topk(self, lengths: torch.Tensor) -> None:
        api.spc_group_max_topk_logits(self.shape, self.logits, self.tile_stats, lengths, self.sel_idx,
                                      self.sel_count, ws=self.ws_topk, stream=self.main)

    def select(self, q: torch.Tensor, lengths: torch.Tensor) -> None:
        self.scores(q, lengths)
        self.topk(lengths)

    def plan(self) -> None:
        api.spc_elastic_update(self.shape, self.sel_idx, self.sel_count, self.slot_pos, self.resident_bm,
                               self.load_pos, self.load_slot, self.load_count, flags=api.SPC_PLAN,
                               plan_stream=self.main)

    def topk_plan(self, lengths: torch.Tensor) -> None:
        """Top-K and the elastic plan in one call (the plan at the end of the Top-K's last kernel)."""
        api.spc_group_max_topk_plan_logits(self.shape, self.logits, self.tile_stats, lengths, self.sel_idx,
                                           self.sel_count, self.slot_pos, self.resident_bm, self.load_pos,
                                           self.load_slot, self.load_count, ws=self.ws_topk, stream=self.main)

    def copy_chunk(self, c: int) -> None:
        a, z = self.chunks[c]
        api.spc_elastic_update(self.shape, None, None, None, None, self.load_pos, self.load_slot, self.load_count,
                               self.host_kv, self.host_l, self.dev_kv, self.dev_l, a, z, flags=api.SPC_COPY,
                               plan_stream=self.main, copy_stream=self.main)

    def _attend(self, q, kv, kv_l, rows, count, mode, a, z, ws, stream, mark, name) -> None:
        """One attention call; with `mark`, the same two kernels as two calls (split, then merge) with
        an event between them, so the split kernel's own time can be read."""
        st = self.main if stream is None else stream
        if mark is None:
            api.spc_sparse_decode_attn(self.shape, q, self.q_l, kv, kv_l, rows, count, mode, a, z, self.out, ws=ws,
                                       stream=st)
        else:
            api.spc_attn_partial(self.shape, q, self.q_l, kv, kv_l, rows, count, mode, a, z, ws, stream=st)
            mark(name + "_merge", st)
            api.spc_attn_merge(self.shape, a, z, ws, self.out, stream=st)

    def attend_chunk(self, q: torch.Tensor, c: int, stream=None, mark=None) -> None:
        a, z = self.chunks[c]
        self._attend(q, self.dev_kv, self.dev_l, self.slot_pos, None, api.SPC_ROWS_SLOTS, a, z, self.ws_attn[c + 1],
                     stream, mark, f"attn{c}")

    def attend_resident(self, q: torch.Tensor, stream=None, mark=None) -> None:
        """Layers still on the GPU: the selected positions gathered from their full cache."""
        self._attend(q, self.full_kv, self.full_l, self.sel_idx, self.sel_count, api.SPC_ROWS_GATHER, 0, self.n_res,
                     self.ws_attn[0], stream, mark, "attn_res")

    # --- one step -----------------------------------------------------------------------
    def step_tokens(self, head: RetrievalHead, tokens: torch.Tensor, lengths: torch.Tensor,
                    timer: Optional["StageTimer"] = None) -> torch.Tensor:
        """The step from the new tokens: the front end writes the query (and appends each token's
        key at position lengths[b], a candidate from the next step on), then the four stages.
        Returns the query buffer."""
        if not hasattr(self, "q_front"):
            p = self.p
            self.q_front = torch.empty((p.batch, p.n_q_heads, p.head_dim), dtype=p.torch_dtype, device=self.device)
        mark = timer.mark if timer is not None else (lambda name, stream: None)
        mark("front", self.main)
        head(tokens, lengths, self.q_front, self.dlm_k, stream=self.main)
        self.step(self.q_front, lengths, timer)
        return self.q_front

    def step(self, q: torch.Tensor, lengths: torch.Tensor, timer: Optional["StageTimer"] = None) -> None:
        """q: device [B][H_q][d]; lengths: device int32 [B].  Asynchronous.

        ``timer`` (optional) brackets every stage call with events on the
        stream the stage runs on, and splits each attention call at its merge."""
        mark = timer.mark if timer is not None else (lambda name, stream: None)
        split = timer.mark if timer is not None else None
        mark("scores", self.main)
        self.scores(q, lengths)
        mark("topk", self.main)
        self.topk_plan(lengths)
        mark("plan_end", self.main)
        side_used = False
        if self.n_res:
            if self.chunks:                       # overlap the resident layers with the copies
                self.ev_sel.record(self.main)
                self.side.wait_event(self.ev_sel)
                mark("attn_res", self.side)
                self.attend_resident(q, self.side, split)
                mark("attn_res_end", self.side)
                side_used = True
            else:
                mark("attn_res", self.main)
                self.attend_resident(q, mark=split)
                mark("attn_res_end", self.main)
        last = len(self.chunks) - 1
        for c in range(len(self.chunks)):
            mark(f"copy{c}", self.main)
            self.copy_chunk(c)
            mark(f"copy{c}_end", self.main)
            if c < last:
                self.ev_copy[c].record(self.main)
                self.side.wait_event(self.ev_copy[c])
                mark(f"attn{c}", self.side)
                self.attend_chunk(q, c, self.side, split)
                mark(f"attn{c}_end", self.side)
                side_used = True
        if self.chunks:
            mark(f"attn{last}", self.main)
            self.attend_chunk(q, last, mark=split)
            mark(f"attn{last}_end", self.main)
        if side_used:
            self.ev_attn.record(self.side)
            self.main.wait_event(self.ev_attn)


class LagOneDecoder:
    """The pipelined loop of the SpeContext blog's section 4: at step t the retrieval head selects
    the positions of step t+1 and their missing rows are copied on the side stream, while the
    target model attends over the selection made at step t-1 (loaded by the previous copy).

      main : scores(t) -> Top-K(t) -> plan(cur=S_t, next=S_t+1) -ev_plan-> wait ev_copy(t-1) -> attention(S_t)
      side :                                  wait ev_plan -> copy(S_t+1 - resident) -> ev_copy(t)

    The slots form a pool of ``pool`` (default 2K) rows per (b, group): a slot is reused only if it
    holds neither selection, so the copy of step t never touches the rows the attention of step t
    reads, and it starts after the attention of step t-1 (stream order on main).  In steady state the
    copies run back to back and everything else overlaps them.  The first step has no previous
    selection and attends over its own, after its copy (warm-up).
    """

    def __init__(self, p: Preset, dlm_k: torch.Tensor, host_kv: torch.Tensor, pool: Optional[int] = None):
        assert p.kind in ("gqa", "mha", "mqa")
        self.p = p
        dev = dlm_k.device
        self.device = dev
        B, Hq, Hkv, G, d, L, K = p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.max_len, p.budget
        P = 2 * K if pool is None else pool
        self.P = P
        self.shape = api.make_shape(B, Hq, Hkv, G, d, p.v_dim, L, K, p.n_layers, p.dtype, p.scale)
        self.pool_shape = api.make_shape(B, Hq, Hkv, G, d, p.v_dim, L, P, p.n_layers, p.dtype, p.scale)
        self.dlm_k, self.host_kv = dlm_k, host_kv
        self.host_l = api.kv_layout(host_kv)
        i32 = dict(dtype=torch.int32, device=dev)
        # stage 1 in log-domain form: logits + per-tile (max, sum exp); stage 2 ranks them directly.
        # With one query head per group the ranking needs no stats, and stage 1 computes none
        self.logits = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
        self.tile_stats = torch.empty(api.tile_stats_shape(self.shape), dtype=torch.float32, device=dev)
        self.stats_out = self.tile_stats if Hq > G else None
        self.sel = [torch.empty((B, G, K), **i32) for _ in range(2)]
        self.cnt = [torch.empty((B, G), **i32) for _ in range(2)]
        self.slot_pos = torch.empty((B, G, P), **i32)
        self.resident_bm = torch.empty((B, G, (L + 31) // 32), **i32)
        self.load_pos = [torch.empty((B, G, P), **i32) for _ in range(2)]
        self.load_slot = [torch.empty((B, G, P), **i32) for _ in range(2)]
        self.load_count = [torch.zeros((B, G), **i32) for _ in range(2)]
        self.attend_rows = torch.empty((B, G, K), **i32)
        self.attend_count = torch.empty((B, G), **i32)
        self.dev_kv = torch.zeros((B, p.n_layers, Hkv, P, 2, d), dtype=p.torch_dtype, device=dev)
        self.dev_l = api.kv_layout(self.dev_kv)
        self.out = torch.zeros((B, p.n_layers, Hq, p.v_dim), dtype=torch.float32, device=dev)
        self.ws_topk = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_TOPK, self.shape)),
                                   dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_ATTN, self.shape)),
                                   dtype=torch.uint8, device=dev)
        self.q_l = api.q_layout(Hq * d, 0, d)
        self.main = torch.cuda.current_stream(dev)
        self.side = torch.cuda.Stream(device=dev)
        self.ev_plan = torch.cuda.Event()
        self.ev_copy = [torch.cuda.Event() for _ in range(2)]
        self.t = 0
        api.spc_elastic_reset(self.pool_shape, -1, self.slot_pos, self.resident_bm, stream=self.main)

    def step(self, q: torch.Tensor, lengths: torch.Tensor, timer: Optional["StageTimer"] = None) -> None:
        mark = timer.mark if timer is not None else (lambda name, stream: None)
        nx = self.t % 2
        cur = nx if self.t == 0 else 1 - nx
        mark("scores", self.main)
        api.spc_retrieval_logits(self.shape, q, self.dlm_k, lengths, self.logits, self.stats_out, stream=self.main)
        mark("topk", self.main)
        api.spc_group_max_topk_logits(self.shape, self.logits, self.tile_stats, lengths, self.sel[nx],
                                      self.cnt[nx], ws=self.ws_topk, stream=self.main)
        mark("plan", self.main)
        api.spc_elastic_plan_lag1(self.pool_shape, self.p.budget, self.sel[cur], self.cnt[cur], self.sel[nx],
                                  self.cnt[nx], self.slot_pos, self.resident_bm, self.load_pos[nx],
                                  self.load_slot[nx], self.load_count[nx], self.attend_rows, self.attend_count,
                                  stream=self.main)
        mark("plan_end", self.main)
        self.ev_plan.record(self.main)
        self.side.wait_event(self.ev_plan)
        mark("copy", self.side)
        api.spc_elastic_update(self.pool_shape, None, None, None, None, self.load_pos[nx], self.load_slot[nx],
                               self.load_count[nx], self.host_kv, self.host_l, self.dev_kv, self.dev_l, 0,
                               self.p.n_layers, flags=api.SPC_COPY, plan_stream=self.side, copy_stream=self.side)
        mark("copy_end", self.side)
        self.ev_copy[nx].record(self.side)
        # this step attends over S_t, loaded by the previous step's copy (the warm-up step by its own)
        self.main.wait_event(self.ev_copy[nx if self.t == 0 else cur])
        mark("attn", self.main)
        api.spc_sparse_decode_attn(self.shape, q, self.q_l, self.dev_kv, self.dev_l, self.attend_rows,
                                   self.attend_count, api.SPC_ROWS_GATHER, 0, self.p.n_layers, self.out,
                                   ws=self.ws_attn, stream=self.main)
        mark("attn_end", self.main)
        self.t += 1


def layer_chunk_bounds(n_layers: int, n_chunks: int, tail_layers: Optional[int] = None) -> List[tuple]:
    """Layer ranges [a, z) of the copy/attention pipeline.

    The last chunk holds ``tail_layers`` layers (default n_layers // 8, at least
    one): its attention is the only work left once the last copy ends, and its
    copy must outlast the attention of the chunks before it.  The other layers
    are split evenly over the first n_chunks - 1 chunks."""
    n = max(1, min(n_chunks, n_layers))
    if n == 1:
        return [(0, n_layers)]
    tail = max(1, n_layers // 8) if tail_layers is None else tail_layers
    tail = max(1, min(tail, n_layers - (n - 1)))
    head = n_layers - tail
    step = -(-head // (n - 1))
    out = [(a, min(a + step, head)) for a in range(0, head, step)]
    return out + [(head, n_layers)]


class StageTimer:
    """Events recorded around each stage call of a step, on that stage's stream."""

    def __init__(self):
        self.events = {}

    def mark(self, name: str, stream) -> None:
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        self.events[name] = ev

    def ms(self, a: str, b: str) -> float:
        return self.events[a].elapsed_time(self.events[b])


class MlaDecoder:
    """The MLA variant of the step: one shared latent head (512 latent + 64 rope dims) in HBM.

    Per step: absorbed query -> head-level scores over the latent cache (MFMA) -> per-head
    Top-K -> elastic plan (the resident-set bookkeeping of each head; the latent stays in
    HBM, so there is nothing to copy) -> attention over the selected latent rows -> output
    projection.  latent: device [B][L][576]; w_uk, w_uv: device [H][dv][512].
    """

    def __init__(self, p: Preset, latent: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor):
        assert p.kind == "mla"
        self.p = p
        dev = latent.device
        B, H, L, K = p.batch, p.n_q_heads, p.max_len, p.budget
        self.shape = api.make_shape(B, H, 1, H, p.head_dim, p.v_dim, L, K, 1, p.dtype, p.scale)
        self.latent, self.w_uk, self.w_uv = latent, w_uk, w_uv
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.q_abs = torch.empty((B, H, p.head_dim), **f32)
        self.logits = torch.empty((B, H, L), **f32)
        self.tile_stats = torch.empty(api.tile_stats_shape(self.shape), **f32)
        self.stats_out = None       # one head per group: the Top-K ranks the logits, no stats needed
        self.sel_idx = torch.empty((B, H, K), **i32)
        self.sel_count = torch.empty((B, H), **i32)
        self.slot_pos = torch.empty((B, H, K), **i32)
        self.resident_bm = torch.empty((B, H, (L + 31) // 32), **i32)
        self.load_pos = torch.empty((B, H, K), **i32)
        self.load_slot = torch.empty((B, H, K), **i32)
        self.load_count = torch.empty((B, H), **i32)
        self.o_lat = torch.zeros((B, 1, H, p.latent_dim), **f32)
        self.out = torch.zeros((B, H, p.nope_dim), **f32)
        self.ws_topk = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_TOPK, self.shape)),
                                   dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_ATTN, self.shape)),
                                   dtype=torch.uint8, device=dev)
        self.q_l = api.q_layout(H * p.head_dim, 0, p.head_dim)          # float32 elements
        self.lat_l = api.SpcKvLayout(L * p.head_dim, 0, 0, p.head_dim, 0)  # V = first 512 dims of the row
        self.main = torch.cuda.current_stream(dev)
        api.spc_elastic_reset(self.shape, -1, self.slot_pos, self.resident_bm, stream=self.main)

    def step(self, q_nope: torch.Tensor, q_rope: torch.Tensor, lengths: torch.Tensor,
             timer: Optional["StageTimer"] = None) -> None:
        """q_nope: device [B][H][dn]; q_rope: device [B][H][R]; lengths: device int32 [B].  Asynchronous."""
        mark = timer.mark if timer is not None else (lambda name, stream: None)
        s, st = self.shape, self.main
        mark("absorb", st)
        api.spc_mla_absorb_q(s, self.p.nope_dim, self.w_uk, q_nope, q_rope, self.q_abs, stream=st)
        mark("scores", st)
        api.spc_retrieval_logits(s, self.q_abs, self.latent, lengths, self.logits, self.stats_out, stream=st)
        mark("topk", st)
        api.spc_group_max_topk_plan_logits(s, self.logits, None, lengths, self.sel_idx, self.sel_count,
                                           self.slot_pos, self.resident_bm, self.load_pos, self.load_slot,
                                           self.load_count, ws=self.ws_topk, stream=st)
        mark("attn", st)                 # attention and output projection (one launch where it fits)
        api.spc_mla_attn_out_proj(s, self.q_abs, self.q_l, self.latent, self.lat_l, self.sel_idx, self.sel_count,
                                  api.SPC_ROWS_GATHER, 0, self.p.nope_dim, self.w_uv, self.o_lat, self.out,
                                  ws=self.ws_attn, stream=st)
        mark("end", st)

    def capture(self) -> None:
        """Capture one step into a HIP graph over static input buffers (the query parts and the
        lengths), so that a serving loop launches the whole step at once: step_graph() copies a
        step's inputs into those buffers and replays it.  The warm-up step that capture needs runs
        on zero-length inputs, and the resident-set state is restored after it."""
        p, dev = self.p, self.latent.device
        B, H = p.batch, p.n_q_heads
        self.g_qn = torch.zeros((B, H, p.nope_dim), dtype=p.torch_dtype, device=dev)
        self.g_qr = torch.zeros((B, H, p.rope_dim), dtype=p.torch_dtype, device=dev)
        self.g_len = torch.zeros((B,), dtype=torch.int32, device=dev)
        main = self.main
        state = (self.slot_pos, self.resident_bm, self.load_pos, self.load_slot, self.load_count, self.sel_idx,
                 self.sel_count)
        saved = [t.clone() for t in state]
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(main)
        self.main = cap
        try:
            with torch.cuda.stream(cap):
                self.step(self.g_qn, self.g_qr, self.g_len)      # warm-up on the capture stream
                for t, v in zip(state, saved):                   # which must leave the state as it was
                    t.copy_(v)
            cap.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph, stream=cap):
                self.step(self.g_qn, self.g_qr, self.g_len)
        finally:
            self.main = main
        torch.cuda.synchronize(dev)

    def step_graph(self, q_nope: torch.Tensor, q_rope: torch.Tensor, lengths: torch.Tensor) -> None:
        """One step through the captured graph (capture() first); inputs as for step()."""
        self.g_qn.copy_(q_nope)
        self.g_qr.copy_(q_rope)
        self.g_len.copy_(lengths)
        self.graph.replay()

    def attend(self, stream=None) -> None:
        """Attention of every head over its selected latent rows (gathered by position).  One call:
        where the budget fits one split per head the library runs it as a single launch, so the
        step is timed as it runs, without a split at the merge."""
        st = self.main if stream is None else stream
        api.spc_sparse_decode_attn(self.shape, self.q_abs, self.q_l, self.latent, self.lat_l, self.sel_idx,
                                   self.sel_count, api.SPC_ROWS_GATHER, 0, 1, self.o_lat, ws=self.ws_attn,
                                   stream=st)


class MlaLiteralDecoder(MlaDecoder):
    """The MLA step in the literal form: each head keeps its own expanded K/V slots.

    Per step: absorbed query -> head-level scores over the latent cache -> per-head Top-K ->
    elastic plan -> the rows each head newly loads expanded into its slots, K = W_UK c || r and
    V = W_UV c in bf16 (spc_mla_expand, MFMA), with the head's query joined as q_nope || q_rope
    -> attention of every head over its slots (head_dim 192, v_dim 128).  Rows a head keeps are
    not expanded again.  The output is the heads' attention output itself, [B][1][H][dv].
    """

    def __init__(self, p: Preset, latent: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor):
        super().__init__(p, latent, w_uk, w_uv)
        B, H, L, K = p.batch, p.n_q_heads, p.max_len, p.budget
        dn, R, dv = p.nope_dim, p.rope_dim, w_uv.shape[1]
        dev = latent.device
        self.row = dn + R + dv
        self.kv_exp = torch.zeros((B, H, K, self.row), dtype=torch.bfloat16, device=dev)
        self.q_exp = torch.empty((B, H, dn + R), dtype=torch.bfloat16, device=dev)
        self.exp_shape = api.make_shape(B, H, H, H, dn + R, dv, L, K, 1, p.dtype, p.scale)
        self.exp_l = api.SpcKvLayout(H * K * self.row, 0, K * self.row, self.row, dn + R)
        self.exp_q_l = api.q_layout(H * (dn + R), 0, dn + R)
        self.out = torch.zeros((B, 1, H, dv), dtype=torch.float32, device=dev)
        self.ws_exp_attn = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_ATTN, self.exp_shape)),
                                       dtype=torch.uint8, device=dev)

    def step(self, q_nope: torch.Tensor, q_rope: torch.Tensor, lengths: torch.Tensor,
             timer: Optional["StageTimer"] = None) -> None:
        """q_nope: device [B][H][dn]; q_rope: device [B][H][R]; lengths: device int32 [B].  Asynchronous."""
        mark = timer.mark if timer is not None else (lambda name, stream: None)
        s, st = self.shape, self.main
        mark("absorb", st)
        api.spc_mla_absorb_q(s, self.p.nope_dim, self.w_uk, q_nope, q_rope, self.q_abs, stream=st)
        mark("scores", st)
        api.spc_retrieval_logits(s, self.q_abs, self.latent, lengths, self.logits, self.stats_out, stream=st)
        mark("topk", st)
        api.spc_group_max_topk_plan_logits(s, self.logits, None, lengths, self.sel_idx, self.sel_count,
                                           self.slot_pos, self.resident_bm, self.load_pos, self.load_slot,
                                           self.load_count, ws=self.ws_topk, stream=st)
        mark("expand", st)
        self.expand(q_nope, q_rope, st)
        mark("attn", st)
        self.attend(st)
        mark("end", st)

    def expand(self, q_nope: torch.Tensor, q_rope: torch.Tensor, stream=None) -> None:
        api.spc_mla_expand(self.shape, self.p.nope_dim, self.w_uv.shape[1], self.latent, self.w_uk, self.w_uv,
                           self.load_pos, self.load_slot, self.load_count, self.kv_exp, q_nope, q_rope, self.q_exp,
                           stream=self.main if stream is None else stream)

    def attend(self, stream=None) -> None:
        """Every head over its expanded slots (slot x attended iff it holds a position)."""
        api.spc_sparse_decode_attn(self.exp_shape, self.q_exp, self.exp_q_l, self.kv_exp, self.exp_l, self.slot_pos,
                                   None, api.SPC_ROWS_SLOTS, 0, 1, self.out, ws=self.ws_exp_attn,
                                   stream=self.main if stream is None else stream)
