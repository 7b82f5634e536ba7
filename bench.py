"""Benchmark of the sparse-KV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 60] [--warmup 4] [--config b1_32k]
                    (--config tiny | b1_32k | b16_grow | mha_64k | mla_32k)

A step is one pass of the whole path over one batch of synthetic input:
retrieval scores -> group max / Top-K -> elastic plan -> elastic copy (per
layer chunk) -> sparse decode attention (per layer chunk, overlapping the
copies of the later chunks on a second stream).  The
default workload is the Llama3.1-8B-shaped 32K step (batch 1, 32 layers,
32 q-heads / 8 KV heads, d=128, bf16, budget 2048, target K/V in pinned host
memory).  Inputs are resident (HBM / pinned host) before timing starts.
The other configurations run the same way; the MLA one runs its own step
(absorbed query -> scores over the latent cache -> per-head Top-K -> plan ->
attention over the selected latent rows -> output projection; the latent
stays in HBM, so nothing is copied).

Prints one JSON line: steps/s from a clean timed pass (events only at its two
ends); per-stage times inside steps from a second, instrumented pass (events
around every stage call on its own stream); per-call kernel times from a third,
isolated phase (each stage call launched back to back, events only at the ends
of the run, on the stream the call uses), which the rooflines of the attention,
scoring and elastic-copy kernels use; and the CPU oracle timed on a bounded
sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import itertools
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
HOST_LINK_PEAK_GBS = 63.0      # PCIe Gen5 x16 per direction: 32 GT/s x 16 x 128/130 / 8
LLC_BYTES = 256 << 20          # MI355X last-level cache (Infinity Cache)
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published

WORKLOADS = {
    "tiny": "tiny: 1 sequence, 1 layer, 32 q-heads / 8 KV heads, d=128, fp32, 4096 cached tokens, budget 256",
    "b1_32k": "b1_32k: Llama3.1-8B-shaped decode step",
    "b16_grow": "b16_grow: batch 16 reasoning growth, 32 layers, ragged lengths growing to 16384, budget 1024",
    "mha_64k": "mha_64k: MHA 32 q-heads = 32 KV heads, 65536 cached tokens, batch 2, budget 4096, 1 layer",
    "mla_32k": "mla_32k: MLA 128 heads, latent 512 + rope 64, 32768 cached tokens, batch 4, budget 2048, 1 layer",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default="b1_32k")
    ap.add_argument("--retrieval", default="head", choices=("head", "batch"),
                    help="head: one selection per KV head (GQA group; the path as built); batch: one selection "
                         "per sequence shared by every head (the comparison the pages draw)")
    ap.add_argument("--graph", action="store_true",
                    help="MLA: time the steps as HIP-graph replays instead of eager launches")
    ap.add_argument("--layer-chunks", type=int, default=2)
    ap.add_argument("--tail-layers", type=int, default=None,
                    help="layers in the last chunk (default n_layers // 8)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--hbm-gb", type=float, default=None,
                    help="adaptive offloading: GPU memory (GB) for the model; layers whose full K/V fits stay on "
                         "the GPU (default: every layer offloaded, the K/V store in pinned host memory)")
    ap.add_argument("--lag", type=int, default=0, choices=(0, 1),
                    help="1: the pipelined loop (the step attends over the previous step's selection while the "
                         "next one loads)")
    ap.add_argument("--mla-literal", action="store_true",
                    help="MLA: the literal form (each head expands its newly loaded rows into its own K/V slots) "
                         "instead of the absorbed one")
    ap.add_argument("--weights-gb", type=float, default=16.0,
                    help="target-model weights counted against --hbm-gb (8B parameters in bf16)")
    ap.add_argument("--t0", type=int, default=None,
                    help="first step of the measured window in the length schedule (default 0; batch-16 "
                         "growth: the last steps, where every sequence has reached 16384)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--iso-reps", type=int, default=30, help="launches per stage in the isolated phase")
    ap.add_argument("--kv-heads-per-gpu", type=int, default=None,
                    help="GQA/MHA: run one tensor-parallel shard of the workload, with this many KV heads (and "
                         "their query heads) of the model's; every stage is independent per KV head, so a shard "
                         "is the whole per-GPU path of a multi-GPU step")
    ap.add_argument("--budget-sweep", default=None,
                    help="comma-separated KV budgets: per budget, one layer's prefetch (a full reload and the "
                         "elastic load of a steady step) against one layer's sparse attention")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with three 256 MiB device-to-device copies (counter calibration)")
    return ap.parse_args()


def measured_traffic(workload: str, layer_chunks: int):
    """HBM traffic per launch from the committed counter summary, while the kernels are unchanged.

    profiles/hbm_traffic_<workload>.md carries the scaled FETCH_SIZE / WRITE_SIZE bytes per launch
    of each stage call and the hashes of the sources they were taken with; any mismatch gives None.
    """
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return {}
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return {}
    data = json.loads(m.group(1))
    if data.get("workload") != workload or data.get("layer_chunks") != layer_chunks:
        return {}
    out = {}
    csrc = os.path.join(ROOT, "speculative_kv_sparsity_amd", "csrc")
    for call, rec in data["calls"].items():
        ok = all(hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()[:16] == h
                 for f, h in rec["sources"].items())
        out[call] = rec["read_bytes"] + rec["write_bytes"] if ok else None
    return out


ISO_WARM_MS = 10.0      # back-to-back replays before the timed ones (steady clocks, see iso())
ISO_TIMED_REPLAYS = 3


def iso(torch, call, reps):
    """Average time of one call: `reps` launches captured once into a HIP graph (host launch
    overhead out of the bracket), replayed between two events on the stream the calls use.

    The timed replays follow at least ISO_WARM_MS of back-to-back replays of the same graph, with no
    idle gap in between: after the PCIe-bound copies of the steps the part needs a few milliseconds
    of HBM-bound work before its clocks settle (the 32K attention kernel reads 44-45 us in its first
    replay and 42 us from the fifth on, over the same rotating inputs), and a serving loop runs these
    kernels back to back."""
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        call(st)
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for _ in range(reps):
                call(st)
        with torch.cuda.stream(st):        # replay is enqueued on the current stream
            a.record(st)
            g.replay()
            z.record(st)
            torch.cuda.synchronize()
            n_warm = max(2, int(np.ceil(ISO_WARM_MS / max(a.elapsed_time(z), 1e-3))))
            for _ in range(n_warm):
                g.replay()
            a.record(st)
            for _ in range(ISO_TIMED_REPLAYS):
                g.replay()
            z.record(st)
        n = reps * ISO_TIMED_REPLAYS
    except Exception:          # capture refused: time eager launches instead
        torch.cuda.synchronize()
        a.record(st)
        for _ in range(reps):
            call(st)
        z.record(st)
        n = reps
    torch.cuda.synchronize()
    return a.elapsed_time(z) / n


def roof(bound, amount, ms, peak, unit, kernel, calls, traffic=None):
    """Roofline record of one call: `amount` algorithmic bytes (GB/s units) or flops (TFLOP/s)."""
    scale = 1e9 if unit == "GB/s" else 1e12
    ach = amount / (ms * 1e-3) / scale
    rec = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
           "traffic": traffic, "kernel": kernel, "avg_launch_us": round(ms * 1e3, 2), "launches_per_step": calls}
    rec["bytes_per_launch" if unit == "GB/s" else "flop_per_launch"] = int(amount)
    return rec


def resident(*ts):
    """rotation()'s counterpart for inputs that a step keeps in the last-level cache: always the same
    tensors."""
    return lambda: ts


def rotation(*ts, min_bytes=2 * LLC_BYTES):
    """A function that hands out, call by call in turn, copies of the given device tensors, with
    enough copies that one round touches min_bytes.  An isolated call replayed over them reads its
    inputs from HBM, as in a step (the step's other traffic has pushed them out of the last-level
    cache by their next use), instead of from the cache a replay of one buffer would hit."""
    size = sum(t.numel() * t.element_size() for t in ts)
    n = max(2, -(-min_bytes // size))
    it = itertools.cycle([ts] + [tuple(t.clone() for t in ts) for _ in range(n - 1)])
    return lambda: next(it)


def topk_plan_call(api, shape, logits, tile_stats, lengths, dec):
    """A launcher of the fused Top-K + plan call on copies of the decoder's selection, state and plan
    buffers (a replay must not change the decoder's own load lists, which the copy's timing reads)."""
    sel, cnt = dec.sel_idx.clone(), dec.sel_count.clone()
    sp, bm = dec.slot_pos.clone(), dec.resident_bm.clone()
    lp, ls, lc = dec.load_pos.clone(), dec.load_slot.clone(), dec.load_count.clone()
    return lambda st: api.spc_group_max_topk_plan_logits(shape, logits, tile_stats, lengths, sel, cnt, sp, bm, lp,
                                                         ls, lc, ws=dec.ws_topk, stream=st)


def probs_call(torch, api, shape, q, k, lengths, inputs=rotation):
    """A launcher of the probability form of stage 1 (spc_retrieval_scores: logits, then the
    normalize pass), with its own output and workspace, over rotating (or resident) copies of the
    keys.  The step ranks the log-domain form; this one is measured beside it."""
    probs = torch.empty((shape.batch, shape.n_q_heads, shape.max_len), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, api.spc_workspace_size(api.SPC_CALL_SCORES, shape)), dtype=torch.uint8, device="cuda")
    kr = inputs(k)
    return lambda st: api.spc_retrieval_scores(shape, q, kr()[0], lengths, probs, ws=ws, stream=st)


def calibration_copies(torch):
    """Three 256 MiB device-to-device copies: the known-size reference of the counter passes."""
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def selection_coverage(torch, p, q, dlm_k, host_kv, lengths, sel_idx, sel_count):
    """How much attention weight the step's selection covers, averaged over (sequence, query head):
    of the retrieval head's own weights, and of layer 0's target weights (dense softmax over every
    cached position, the same query).  A statistic of the run, computed after the timed passes with
    plain tensor operations; the pages compare it between head-level and batch-level selection."""
    B, Hq, Hkv, d = p.batch, p.n_q_heads, p.n_kv_heads, p.head_dim
    per_kv, per_g = Hq // Hkv, Hq // p.n_groups
    lens = lengths.tolist()
    sel, cnt = sel_idx.cpu(), sel_count.cpu()
    out = {"retrieval_head": [], "target_layer0": []}
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        qb = q[b].float()
        for name, keys in (("retrieval_head", dlm_k[b, :, :n].float()),
                           ("target_layer0", host_kv[b, 0, :, :n, 0].to("cuda").float())):
            kh = keys.repeat_interleave(per_kv, dim=0).contiguous()             # [Hq][n][d] float32
            wts = torch.softmax(torch.bmm(kh, qb[:, :, None].contiguous())[:, :, 0] * p.scale, dim=-1)
            for i in range(Hq):
                g = i // per_g
                idx = sel[b, g, :int(cnt[b, g])].long().to("cuda")
                out[name].append(float(wts[i, idx].sum()))
    return {k: round(float(np.mean(v)), 4) for k, v in out.items()}


def cpu_baseline(p, w, t0, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same workload."""
    from oracle import OracleDecoder
    from speculative_kv_sparsity_amd.workload import to_numpy_raw
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    dec = OracleDecoder(p.batch, p.n_q_heads, p.n_kv_heads, p.n_groups, p.head_dim, p.budget, p.scale, p.dtype)
    k = to_numpy_raw(w.dlm_k)
    kv = to_numpy_raw(w.host_kv)
    layers = list(range(p.n_layers))
    n, start = 0, time.perf_counter()
    t = t0
    while True:
        dec.step(to_numpy_raw(w.q[t]), k, w.lengths[t], kv, layers)
        n += 1
        t = min(t + 1, w.steps - 1)
        if time.perf_counter() - start >= budget_s:
            break
    el = time.perf_counter() - start
    return {"value": n / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "nproc": usable, "host_cpus": os.cpu_count(),
            "sample": f"{n} consecutive decode steps of the same workload (all {p.n_layers} layers, "
                      f"fp64 NumPy), {el:.1f} s; cores = the BLAS threads the oracle ran with, nproc = the "
                      f"CPUs this process may use"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures the path on one GPU only; --gpus {args.gpus} is not supported "
              "(the per-sequence / per-KV-head sharding across GPUs is described, not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    from speculative_kv_sparsity_amd import workload as W

    torch.cuda.set_device(0)
    p = W.PRESETS[args.config]
    if args.kv_heads_per_gpu is not None:
        if p.kind not in ("gqa", "mha") or not 0 < args.kv_heads_per_gpu <= p.n_kv_heads or \
                p.n_kv_heads % args.kv_heads_per_gpu:
            print(f"--kv-heads-per-gpu must divide the {p.n_kv_heads} KV heads of a GQA/MHA workload",
                  file=sys.stderr)
            sys.exit(2)
        g = p.n_q_heads // p.n_kv_heads
        p = p.with_(n_kv_heads=args.kv_heads_per_gpu, n_q_heads=g * args.kv_heads_per_gpu)
    if args.retrieval == "batch":
        if p.kind not in ("gqa", "mha"):
            print("--retrieval batch applies to GQA/MHA workloads", file=sys.stderr)
            sys.exit(2)
        p = p.with_(kind="mqa")          # one group over every query head of a sequence
    if args.budget_sweep:
        result = bench_budget_sweep(args, p, torch, W)
    elif p.kind == "mla":
        result = bench_mla_literal(args, p, torch, W) if args.mla_literal else bench_mla(args, p, torch, W)
    elif args.lag == 1:
        result = bench_lag1(args, p, torch, W)
    else:
        result = bench_gqa(args, p, torch, W)
    print(json.dumps(result), flush=True)


def _header(args, p, ms_per_step, config):
    return {
        "metric": "sparse decode steps/s (score+TopK+elastic load+attn) and % HBM peak at 32K",
        "value": round(1e3 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": config,
    }


def bench_gqa(args, p, torch, W):
    from speculative_kv_sparsity_amd import api
    from speculative_kv_sparsity_amd.driver import RetrievalHead, SparseDecoder, StageTimer

    K_, Wm = args.steps, args.warmup
    total = Wm + 2 * K_
    t0 = args.t0
    if t0 is None:
        t0 = p.steps - total if p.name == "b16_grow" else 0
    t0 = max(0, min(t0, p.steps - total)) if p.steps >= total else 0
    w = W.generate(p, device="cuda", seed=args.seed, steps=max(total, t0 + total), pin_host=True)
    thresholds = None
    if args.hbm_gb is not None:
        # memory model: weights; per position the DLM key, the probabilities and the Top-K key of every
        # head; per layer and position the target K and V (the four inputs the pages name)
        thresholds = api.spc_offload_thresholds(
            int(args.hbm_gb * 1e9), int(args.weights_gb * 1e9),
            p.batch * (p.n_kv_heads * p.head_dim * p.elem_bytes + p.n_q_heads * 4 + p.n_groups * 4), p.n_layers,
            p.batch, p.n_kv_heads, p.head_dim, p.v_dim, p.budget, p.elem_bytes)
    dec = SparseDecoder(p, w.dlm_k, w.host_kv, layer_chunks=args.layer_chunks, tail_layers=args.tail_layers,
                        thresholds=thresholds)
    seq_len = [int(x) for x in w.lengths.max(axis=1)]

    def step(t, timer=None):
        dec.offload_for(seq_len[t])
        dec.step(qs[t], lens[t], timer)
    lens = torch.as_tensor(w.lengths, device="cuda")
    qs = w.q.contiguous()
    torch.cuda.synchronize()

    for t in range(t0, t0 + Wm):                 # the first step is the cold full-budget load
        step(t)
    torch.cuda.synchronize()

    # clean timed pass
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(dec.main)
    for t in range(t0 + Wm, t0 + Wm + K_):
        step(t)
    e1.record(dec.main)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / K_

    # instrumented pass: K more steps, launched back to back like the timed ones (no synchronize
    # between steps), with events around every stage call and inside each attention call at its
    # merge; the rows moved are summed on the device and read at the end
    timers = []
    moved = torch.zeros((K_, 2), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    for i, t in enumerate(range(t0 + Wm + K_, t0 + total)):
        tm = StageTimer()
        step(t, tm)
        moved[i, 0] = dec.load_count.sum()
        moved[i, 1] = dec.sel_count.sum()
        timers.append(tm)
    torch.cuda.synchronize()
    nch = len(dec.chunks)
    # rows per KV head: a group spanning several KV heads (batch-level retrieval) loads and holds its
    # selected rows in every one of them
    hpg = max(1, p.n_kv_heads // p.n_groups)
    loaded_rows, sel_rows = [x * hpg for x in moved[:, 0].tolist()], [x * hpg for x in moved[:, 1].tolist()]
    spans = {"scores": ("scores", "topk"), "topk_plan": ("topk", "plan_end")}
    for c in range(nch):
        spans.update({f"copy{c}": (f"copy{c}", f"copy{c}_end"), f"attn{c}": (f"attn{c}", f"attn{c}_end"),
                      f"attn{c}_split": (f"attn{c}", f"attn{c}_merge")})
    if dec.n_res:
        spans.update({"attn_resident": ("attn_res", "attn_res_end"), "attn_resident_split": ("attn_res",
                                                                                              "attn_res_merge")})
    avg = {k: float(np.mean([tm.ms(a, z) for tm in timers])) for k, (a, z) in spans.items()}

    # isolated phase: each stage call launched back to back.  Where one step moves more than the
    # last-level cache holds (keys, logits, every layer's selected K/V rows, the rows copied in), a
    # stage's inputs are gone from the cache by its next use, so the HBM-bound calls are replayed over
    # rotating copies of their inputs; a smaller step keeps them resident and replays the same ones
    tq, tl = qs[t0 + total - 1], lens[t0 + total - 1]
    R = args.iso_reps
    n_step = float(np.mean(w.lengths[t0 + Wm + K_:t0 + total].sum(axis=1)))
    step_bytes = (n_step * (p.n_kv_heads * p.head_dim * p.elem_bytes + p.n_q_heads * 4)
                  + float(np.mean(sel_rows)) * p.n_layers * 2 * p.head_dim * p.elem_bytes
                  + float(np.mean(loaded_rows)) * (p.n_layers - dec.n_res) * 2 * p.head_dim * p.elem_bytes)
    inputs = rotation if step_bytes > LLC_BYTES else resident
    dk = inputs(dec.dlm_k)
    iso_ms = {
        "scores": iso(torch, lambda st: api.spc_retrieval_logits(dec.shape, tq, dk()[0], tl, dec.logits,
                                                                 dec.stats_out, stream=st), R),
        "topk": iso(torch, lambda st: api.spc_group_max_topk_logits(dec.shape, dec.logits, dec.tile_stats, tl,
                                                                    dec.sel_idx, dec.sel_count, ws=dec.ws_topk,
                                                                    stream=st), R),
        "topk_plan": iso(torch, topk_plan_call(api, dec.shape, dec.logits, dec.tile_stats, tl, dec), R),
        "scores_probs": iso(torch, probs_call(torch, api, dec.shape, tq, dec.dlm_k, tl, inputs), R),
    }
    if nch:
        c0a, c0z = dec.chunks[0]
        kv = inputs(dec.dev_kv)
        iso_ms["attn"] = iso(torch, lambda st: api.spc_sparse_decode_attn(
            dec.shape, tq, dec.q_l, kv()[0], dec.dev_l, dec.slot_pos, None, api.SPC_ROWS_SLOTS, c0a, c0z,
            dec.out, ws=dec.ws_attn[0], stream=st), R)
        iso_ms["attn_partial"] = iso(torch, lambda st: api.spc_attn_partial(
            dec.shape, tq, dec.q_l, kv()[0], dec.dev_l, dec.slot_pos, None, api.SPC_ROWS_SLOTS, c0a, c0z,
            dec.ws_attn[0], stream=st), R)
        iso_ms["copy"] = iso(torch, lambda st: api.spc_elastic_update(
            dec.shape, None, None, None, None, dec.load_pos, dec.load_slot, dec.load_count, dec.host_kv, dec.host_l,
            dec.dev_kv, dec.dev_l, c0a, c0z, flags=api.SPC_COPY, plan_stream=st, copy_stream=st),
            max(5, R // 3))   # rewrites the same slots
    else:                     # every layer on the GPU: the gather from the full cache is the attention
        c0a, c0z = 0, dec.n_res
        fk = inputs(dec.full_kv)
        iso_ms["attn"] = iso(torch, lambda st: api.spc_sparse_decode_attn(
            dec.shape, tq, dec.q_l, fk()[0], dec.full_l, dec.sel_idx, dec.sel_count, api.SPC_ROWS_GATHER, 0,
            dec.n_res, dec.out, ws=dec.ws_attn[0], stream=st), R)
        iso_ms["attn_partial"] = iso(torch, lambda st: api.spc_attn_partial(
            dec.shape, tq, dec.q_l, fk()[0], dec.full_l, dec.sel_idx, dec.sel_count, api.SPC_ROWS_GATHER, 0,
            dec.n_res, dec.ws_attn[0], stream=st), R)
    # the retrieval head's front end (upstream of the step): new tokens -> query, key appended
    fw = W.generate_front(p, device="cuda", seed=args.seed, steps=1)
    heads = inputs(fw.wq, fw.wk)
    ncopy = max(2, -(-2 * LLC_BYTES // (fw.wq.nbytes + fw.wk.nbytes))) if inputs is rotation else 1
    heads = [RetrievalHead(dec.shape, dataclasses.replace(fw, wq=wq, wk=wk)) for wq, wk in (heads() for _ in range(ncopy))]
    head = itertools.cycle(heads)
    q_front = torch.empty((p.batch, p.n_q_heads, p.head_dim), dtype=p.torch_dtype, device="cuda")
    tok = torch.as_tensor(fw.tokens[0], device="cuda")
    iso_ms["front"] = iso(torch, lambda st: next(head)(tok, tl, q_front, dec.dlm_k, stream=st), R)

    eb = p.elem_bytes
    lay0 = c0z - c0a
    B, Hkv, Hq, d, K = p.batch, p.n_kv_heads, p.n_q_heads, p.head_dim, p.budget
    n_valid = float(np.mean(w.lengths[t0 + Wm + K_:t0 + total].sum(axis=1)))
    row = 2 * d * eb                                             # one K||V row
    sel_per_group = float(np.mean(sel_rows)) / (B * p.n_kv_heads)       # rows per (sequence, KV head)
    # algorithmic bytes per call (one launch of the stage)
    kv_bytes = B * lay0 * Hkv * sel_per_group * row                         # K/V rows read (split kernel)
    attn_bytes = kv_bytes + B * lay0 * Hq * d * 4                             # + out write (the whole call)
    score_bytes = n_valid * Hkv * d * eb + n_valid * Hq * 4              # keys read + logits (probs) write
    front_bytes = ((Hq + Hkv) * d * fw.hidden + B * fw.hidden + fw.hidden + B * (Hq + Hkv) * d) * eb
    full_reload = float(np.mean(sel_rows)) * p.n_layers * row
    off = p.n_layers - dec.n_res                                 # offloaded layers at the end of the run

    shard = args.kv_heads_per_gpu is not None
    traffic = measured_traffic(p.name, nch) if thresholds is None and not shard else {}
    config = {"workload": WORKLOADS.get(p.name, p.name), "batch": B, "layers": p.n_layers, "q_heads": Hq,
              "kv_heads": Hkv, "head_dim": d, "cached_tokens": p.max_len,
              "mean_length": round(n_valid / B, 1), "first_step": t0, "kv_budget": K, "layer_chunks": nch,
              "chunk_layers": [z - a for a, z in dec.chunks], "parallelism": "single GPU"}
    if p.kind == "mqa":
        config["retrieval"] = "batch-level: one selection per sequence shared by all query heads"
    if thresholds is not None:
        config.update({"hbm_gb": args.hbm_gb, "weights_gb": args.weights_gb, "offloaded_layers": off,
                       "offload_thresholds": thresholds})
    if shard:
        full = W.PRESETS[p.name].n_kv_heads
        config["parallelism"] = (f"one of {full // p.n_kv_heads} tensor-parallel shards over KV heads "
                                 f"({p.n_kv_heads} of {full} per GPU), single GPU")
    result = _header(args, p, ms_per_step, config)
    rows_of = (", slots of the offloaded layers" if nch else
               ", selected rows gathered from the GPU-resident full cache")
    cold = ("; isolated launches over rotating copies of its inputs, cold in the last-level cache as in a step"
            if inputs is rotation else "")
    result["roofline"] = roof("hbm", kv_bytes, iso_ms["attn_partial"], HBM_PEAK_GBS, "GB/s",
                              "attn_split_kernel (the dominant kernel: split-K partial attention" + rows_of +
                              ", first layer chunk, timed alone through spc_attn_partial" + cold + ")", max(nch, 1),
                              traffic.get("attn_partial"))
    result["roofline_attn_call"] = roof("hbm", attn_bytes, iso_ms["attn"], HBM_PEAK_GBS, "GB/s",
                                        "attn_split_kernel + attn_combine_kernel (spc_sparse_decode_attn: the "
                                        "whole stage-4 call" + rows_of + cold + ")", max(nch, 1), traffic.get("attn"))
    result["roofline_scores"] = roof("hbm", score_bytes, iso_ms["scores"], HBM_PEAK_GBS, "GB/s",
                                     "scores_logits_kernel (stage 1 as the step runs it: logits and per-tile "
                                     "max / sum exp in one pass over the DLM keys" + cold + ")", 1,
                                     traffic.get("scores"))
    result["roofline_scores_probs"] = roof("hbm", score_bytes, iso_ms["scores_probs"], HBM_PEAK_GBS, "GB/s",
                                           "scores_logits_kernel + scores_normalize_kernel (spc_retrieval_scores: "
                                           "the probabilities written; not on the step's path)", 0,
                                           traffic.get("scores_probs"))
    if nch:
        copy_bytes = float(np.mean(loaded_rows)) * lay0 * row            # host reads per chunk
        result["roofline_host_link"] = roof("host_link", copy_bytes, iso_ms["copy"], HOST_LINK_PEAK_GBS, "GB/s",
                                            "copy_kernel (elastic host->HBM gather, first layer chunk)", nch,
                                            traffic.get("copy"))
    result["roofline_front_end"] = roof("hbm", front_bytes, iso_ms["front"], HBM_PEAK_GBS, "GB/s",
                                        "front_gemv_kernel + front_finish_kernel (retrieval-head front end: "
                                        f"embedding, input norm, Q/K projection of hidden {fw.hidden}, YaRN rotary, "
                                        "key append; upstream of the step, not in value)", 1, traffic.get("front"))
    result["stage_us_in_step"] = {k: round(v * 1e3, 2) for k, v in avg.items()}
    result["call_us_isolated"] = {k: round(v * 1e3, 2) for k, v in iso_ms.items()}
    result["isolated_inputs"] = {"step_bytes": int(step_bytes), "last_level_cache_bytes": LLC_BYTES,
                                 "replayed_over": "rotating copies" if inputs is rotation else "the same buffers"}
    result["elastic"] = {"rows_loaded_per_step": float(np.mean(loaded_rows)),
                         "rows_selected_per_step": float(np.mean(sel_rows)),
                         "transfer_fraction_vs_full_reload":
                             round(float(np.mean(loaded_rows)) * p.n_layers * row / full_reload, 4),
                         "adjacent_overlap": round(1.0 - float(np.mean(loaded_rows)) / float(np.mean(sel_rows)), 4),
                         "rows_counted_per": "(sequence, layer, KV head)",
                         "host_link_bytes_per_step": int(float(np.mean(loaded_rows)) * off * row)}
    result["retrieval"] = {"level": "head" if p.kind != "mqa" else "batch", "groups": p.n_groups,
                           "coverage": selection_coverage(torch, p, tq, dec.dlm_k, w.host_kv, tl, dec.sel_idx,
                                                          dec.sel_count)}
    if args.calibrate_copy:
        calibration_copies(torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, w, t0 + Wm, args.cpu_seconds)
    return result


def bench_budget_sweep(args, p, torch, W):
    """Per KV budget: the time to prefetch one layer's selected rows (all of them, as on the cold first
    step, and the elastic load of a steady step) against one layer's sparse attention over them.
    The copy and the attention of all layers run as one chunk and are divided by the layer count."""
    from speculative_kv_sparsity_amd import api
    from speculative_kv_sparsity_amd.driver import SparseDecoder, StageTimer

    budgets = [int(x) for x in args.budget_sweep.split(",")]
    if p.kind not in ("gqa", "mha") or any(not 0 < k <= p.max_len for k in budgets):
        print("--budget-sweep takes budgets in (0, max_len] of a GQA/MHA workload", file=sys.stderr)
        sys.exit(2)
    steps = 8
    w = W.generate(p, device="cuda", seed=args.seed, steps=steps, pin_host=True)
    lens = torch.as_tensor(w.lengths, device="cuda")
    qs = w.q.contiguous()
    L, row = p.n_layers, 2 * p.head_dim * p.elem_bytes
    rows = []
    for K in budgets:
        pk = p.with_(budget=K)
        dec = SparseDecoder(pk, w.dlm_k, w.host_kv, layer_chunks=1)
        times = []
        moved = []
        for t in range(steps):
            tm = StageTimer()
            dec.step(qs[t], lens[t], tm)
            torch.cuda.synchronize()
            times.append((tm.ms("copy0", "copy0_end"), tm.ms("attn0", "attn0_merge")))
            moved.append(int(dec.load_count.sum().item()))
        cold_copy = times[0][0] / L
        warm = times[2:]
        el_copy = float(np.mean([c for c, _ in warm])) / L
        attn = float(np.mean([a for _, a in warm])) / L
        full_bytes = moved[0] * row                               # every selected row of one layer
        el_bytes = float(np.mean(moved[2:])) * row
        rows.append({"budget": K, "full_reload_us_per_layer": round(cold_copy * 1e3, 2),
                     "full_reload_MB_per_layer": round(full_bytes / 1e6, 3),
                     "elastic_us_per_layer": round(el_copy * 1e3, 2),
                     "elastic_MB_per_layer": round(el_bytes / 1e6, 3),
                     "attention_us_per_layer": round(attn * 1e3, 2)})
        del dec
        torch.cuda.empty_cache()
    config = {"workload": WORKLOADS.get(p.name, p.name), "batch": p.batch, "layers": L, "q_heads": p.n_q_heads,
              "kv_heads": p.n_kv_heads, "head_dim": p.head_dim, "cached_tokens": p.max_len,
              "budgets": budgets, "parallelism": "single GPU"}
    return {"mode": "budget sweep (one layer's prefetch against one layer's sparse attention)",
            "data": "synthetic", "config": config, "budget_sweep": rows}


def bench_lag1(args, p, torch, W):
    """The pipelined loop: step t's copy loads step t+1's rows while step t attends over the rows
    loaded for it one step earlier."""
    from speculative_kv_sparsity_amd import api
    from speculative_kv_sparsity_amd.driver import LagOneDecoder, StageTimer

    K_, Wm = args.steps, args.warmup
    total = Wm + 2 * K_
    t0 = args.t0
    if t0 is None:
        t0 = p.steps - total if p.name == "b16_grow" else 0
    t0 = max(0, min(t0, p.steps - total)) if p.steps >= total else 0
    w = W.generate(p, device="cuda", seed=args.seed, steps=max(total, t0 + total), pin_host=True)
    dec = LagOneDecoder(p, w.dlm_k, w.host_kv)
    lens = torch.as_tensor(w.lengths, device="cuda")
    qs = w.q.contiguous()
    torch.cuda.synchronize()
    for t in range(t0, t0 + Wm):
        dec.step(qs[t], lens[t])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(dec.main)
    for t in range(t0 + Wm, t0 + Wm + K_):
        dec.step(qs[t], lens[t])
    e1.record(dec.main)
    dec.side.synchronize()
    torch.cuda.synchronize()
    # the last step's copy (of the rows of a step not run) is outside the bracket; it overlapped the
    # attention of that step, as every copy overlaps the next step's work
    ms_per_step = e0.elapsed_time(e1) / K_
    stage = {k: [] for k in ("scores", "topk", "plan", "copy", "attn")}
    loaded, sel_rows = [], []
    for t in range(t0 + Wm + K_, t0 + total):
        nx = dec.t % 2
        tm = StageTimer()
        dec.step(qs[t], lens[t], timer=tm)
        torch.cuda.synchronize()
        for a, z in (("scores", "topk"), ("topk", "plan"), ("plan", "plan_end"), ("copy", "copy_end"),
                     ("attn", "attn_end")):
            stage[a].append(tm.ms(a, z))
        loaded.append(int(dec.load_count[nx].sum().item()))
        sel_rows.append(int(dec.cnt[nx].sum().item()))
    avg = {k: float(np.mean(v)) for k, v in stage.items()}
    tq, tl = qs[t0 + total - 1], lens[t0 + total - 1]
    R = args.iso_reps
    nx = (dec.t - 1) % 2
    dk, kv = rotation(dec.dlm_k), rotation(dec.dev_kv)
    iso_ms = {
        "scores": iso(torch, lambda st: api.spc_retrieval_logits(dec.shape, tq, dk()[0], tl, dec.logits,
                                                                 dec.stats_out, stream=st), R),
        "topk": iso(torch, lambda st: api.spc_group_max_topk_logits(dec.shape, dec.logits, dec.tile_stats, tl,
                                                                    dec.sel[nx], dec.cnt[nx], ws=dec.ws_topk,
                                                                    stream=st), R),
        "attn": iso(torch, lambda st: api.spc_sparse_decode_attn(
            dec.shape, tq, dec.q_l, kv()[0], dec.dev_l, dec.attend_rows, dec.attend_count, api.SPC_ROWS_GATHER,
            0, p.n_layers, dec.out, ws=dec.ws_attn, stream=st), R),
        "attn_partial": iso(torch, lambda st: api.spc_attn_partial(
            dec.shape, tq, dec.q_l, kv()[0], dec.dev_l, dec.attend_rows, dec.attend_count, api.SPC_ROWS_GATHER,
            0, p.n_layers, dec.ws_attn, stream=st), R),
        "copy": iso(torch, lambda st: api.spc_elastic_update(
            dec.pool_shape, None, None, None, None, dec.load_pos[nx], dec.load_slot[nx], dec.load_count[nx],
            dec.host_kv, dec.host_l, dec.dev_kv, dec.dev_l, 0, p.n_layers, flags=api.SPC_COPY, plan_stream=st,
            copy_stream=st), max(5, R // 3)),
    }
    eb = p.elem_bytes
    B, Hkv, Hq, d, K = p.batch, p.n_kv_heads, p.n_q_heads, p.head_dim, p.budget
    n_valid = float(np.mean(w.lengths[t0 + Wm + K_:t0 + total].sum(axis=1)))
    row = 2 * d * eb
    sel_per_group = float(np.mean(sel_rows)) / (B * p.n_groups)
    kv_bytes = B * p.n_layers * Hkv * sel_per_group * row
    attn_bytes = kv_bytes + B * p.n_layers * Hq * d * 4
    score_bytes = n_valid * Hkv * d * eb + n_valid * Hq * 4
    copy_bytes = float(np.mean(loaded)) * p.n_layers * row
    config = {"workload": WORKLOADS.get(p.name, p.name), "batch": B, "layers": p.n_layers, "q_heads": Hq,
              "kv_heads": Hkv, "head_dim": d, "cached_tokens": p.max_len, "mean_length": round(n_valid / B, 1),
              "first_step": t0, "kv_budget": K, "pipeline": "lag 1 (attention over the previous step's selection)",
              "slot_pool": dec.P, "parallelism": "single GPU"}
    result = _header(args, p, ms_per_step, config)
    result["roofline"] = roof("hbm", kv_bytes, iso_ms["attn_partial"], HBM_PEAK_GBS, "GB/s",
                              "attn_split_kernel (the dominant kernel: the pool's rows of the current selection, "
                              "gathered; timed alone through spc_attn_partial)", 1)
    result["roofline_attn_call"] = roof("hbm", attn_bytes, iso_ms["attn"], HBM_PEAK_GBS, "GB/s",
                                        "attn_split_kernel + attn_combine_kernel (the whole stage-4 call)", 1)
    result["roofline_scores"] = roof("hbm", score_bytes, iso_ms["scores"], HBM_PEAK_GBS, "GB/s",
                                     "scores_logits_kernel (logits and per-tile max / sum exp, one pass)", 1)
    result["roofline_host_link"] = roof("host_link", copy_bytes, iso_ms["copy"], HOST_LINK_PEAK_GBS, "GB/s",
                                        "copy_kernel (elastic host->HBM gather, every layer in one launch)", 1)
    result["stage_us_in_step"] = {k: round(v * 1e3, 2) for k, v in avg.items()}
    result["call_us_isolated"] = {k: round(v * 1e3, 2) for k, v in iso_ms.items()}
    result["elastic"] = {"rows_loaded_per_step": float(np.mean(loaded)),
                         "rows_selected_per_step": float(np.mean(sel_rows)),
                         "transfer_fraction_vs_full_reload": round(float(np.mean(loaded)) / float(np.mean(sel_rows)),
                                                                   4),
                         "host_link_bytes_per_step": int(copy_bytes)}
    return result


def bench_mla(args, p, torch, W):
    from speculative_kv_sparsity_amd import api
    from speculative_kv_sparsity_amd.driver import MlaDecoder, StageTimer

    K_, Wm = args.steps, args.warmup
    total = Wm + 2 * K_
    w = W.generate(p, device="cuda", seed=args.seed, steps=total)
    dec = MlaDecoder(p, w.latent, w.w_uk, w.w_uv)
    lens = torch.as_tensor(w.lengths, device="cuda")
    qn, qr = w.q_nope.contiguous(), w.q_rope.contiguous()
    torch.cuda.synchronize()
    for t in range(Wm):
        dec.step(qn[t], qr[t], lens[t])
    torch.cuda.synchronize()

    # the timed steps: eager launches, or with --graph HIP-graph replays of one captured step (its
    # inputs copied into the graph's static buffers, inside the timed region); the other launch
    # mode is timed too, over the same steps replayed from the same state, and reported beside it.
    # Eager launches run ahead of the GPU here, so the graph gains nothing (it measures slower)
    state = (dec.slot_pos, dec.resident_bm, dec.load_pos, dec.load_slot, dec.load_count, dec.sel_idx,
             dec.sel_count)
    saved = [t.clone() for t in state]
    dec.capture()

    def timed(graph):
        for t, v in zip(state, saved):
            t.copy_(v)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(dec.main)
        for t in range(Wm, Wm + K_):
            if graph:
                dec.step_graph(qn[t], qr[t], lens[t])
            else:
                dec.step(qn[t], qr[t], lens[t])
        e1.record(dec.main)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K_

    ms_eager = timed(False)
    ms_graph = timed(True)
    ms_per_step = ms_graph if args.graph else ms_eager

    # instrumented pass: K more steps launched back to back (no synchronize between steps), events
    # around every stage call and at the attention's merge; counts summed on the device
    names = ("absorb", "scores", "topk", "attn", "end")       # "attn": attention + output projection
    timers = []
    moved = torch.zeros((K_, 3), dtype=torch.int64, device="cuda")
    mark = torch.zeros((p.batch, p.max_len + 1), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for i, t in enumerate(range(Wm + K_, total)):
        tm = StageTimer()
        dec.step(qn[t], qr[t], lens[t], timer=tm)
        moved[i, 0] = dec.load_count.sum()
        moved[i, 1] = dec.sel_count.sum()
        # distinct latent rows selected by any head of a sequence: what the attention must read at least once
        idx = torch.where(dec.sel_idx >= 0, dec.sel_idx, p.max_len).reshape(p.batch, -1).long()
        mark.zero_()
        mark.scatter_(1, idx, 1)
        moved[i, 2] = mark[:, :p.max_len].sum()
        timers.append(tm)
    torch.cuda.synchronize()
    churn, sel_rows, union_rows = (moved[:, j].tolist() for j in range(3))
    spans = dict(zip(names[:-1], zip(names[:-1], names[1:])))
    avg = {k: float(np.mean([tm.ms(a, z) for tm in timers])) for k, (a, z) in spans.items()}

    tq, tr, tl = qn[total - 1], qr[total - 1], lens[total - 1]
    R = args.iso_reps
    s = dec.shape
    # what one step moves: the latent rows, the logits and the two up-projections.  At 32K that is
    # about 250 MB, which the 256 MB last-level cache holds from one step to the next (the kernels'
    # durations inside the timed steps match warm replays), so the isolated calls replay resident
    # inputs; a larger working set gets rotating copies, cold like the GQA steps
    n_step = float(np.mean(w.lengths[Wm + K_:total].sum(axis=1)))
    step_bytes = (n_step * p.head_dim * p.elem_bytes + n_step * p.n_q_heads * 4 + dec.w_uk.nbytes
                  + dec.w_uv.nbytes)
    inputs = rotation if step_bytes > LLC_BYTES else resident
    uk, uv, lat = inputs(dec.w_uk), inputs(dec.w_uv), inputs(dec.latent)
    iso_ms = {
        "absorb": iso(torch, lambda st: api.spc_mla_absorb_q(s, p.nope_dim, uk()[0], tq, tr, dec.q_abs,
                                                             stream=st), R),
        "scores": iso(torch, lambda st: api.spc_retrieval_logits(s, dec.q_abs, lat()[0], tl, dec.logits,
                                                                 dec.stats_out, stream=st), R),
        "topk": iso(torch, lambda st: api.spc_group_max_topk_logits(s, dec.logits, None, tl, dec.sel_idx,
                                                                    dec.sel_count, ws=dec.ws_topk, stream=st), R),
        "topk_plan": iso(torch, topk_plan_call(api, s, dec.logits, None, tl, dec), R),
        "scores_probs": iso(torch, probs_call(torch, api, s, dec.q_abs, dec.latent, tl, inputs), R),
        "attn": iso(torch, lambda st: api.spc_sparse_decode_attn(
            s, dec.q_abs, dec.q_l, lat()[0], dec.lat_l, dec.sel_idx, dec.sel_count, api.SPC_ROWS_GATHER, 0, 1,
            dec.o_lat, ws=dec.ws_attn, stream=st), R),
        "attn_partial": iso(torch, lambda st: api.spc_attn_partial(
            s, dec.q_abs, dec.q_l, lat()[0], dec.lat_l, dec.sel_idx, dec.sel_count, api.SPC_ROWS_GATHER, 0, 1,
            dec.ws_attn, stream=st), R),
        "out_proj": iso(torch, lambda st: api.spc_mla_out_proj(s, p.nope_dim, uv()[0], dec.o_lat, 0, dec.out,
                                                               stream=st), R),
        "attn_out_proj": iso(torch, lambda st: api.spc_mla_attn_out_proj(
            s, dec.q_abs, dec.q_l, lat()[0], dec.lat_l, dec.sel_idx, dec.sel_count, api.SPC_ROWS_GATHER, 0,
            p.nope_dim, uv()[0], dec.o_lat, dec.out, ws=dec.ws_attn, stream=st), R),
    }
    B, H, L, D = p.batch, p.n_q_heads, p.max_len, p.head_dim
    n_valid = float(np.mean(w.lengths[Wm + K_:total].sum(axis=1)))
    sel = float(np.mean(sel_rows))
    union = float(np.mean(union_rows))
    row = D * p.elem_bytes                                      # one latent row: 512 latent + 64 rope dims
    lat_bytes = union * row                                      # every selected row once (split kernel)
    attn_bytes = lat_bytes + B * H * p.latent_dim * 4            # + o_lat writes (the whole call)
    gathered = sel * row                                         # each head's own gather (L2 / last-level cache)
    score_flop = 2.0 * n_valid * H * D                           # every head against every valid latent row
    score_bytes = n_valid * row + n_valid * H * 4               # latent read once + logits (probs) write
    traffic = measured_traffic(p.name, 1)
    config = {"workload": WORKLOADS["mla_32k"] if p.name == "mla_32k" else p.name, "batch": B, "layers": 1,
              "q_heads": H, "latent_dim": p.latent_dim, "rope_dim": p.rope_dim, "nope_dim": p.nope_dim,
              "cached_tokens": L, "kv_budget": p.budget, "parallelism": "single GPU"}
    result = _header(args, p, ms_per_step, config)
    result.update({
        "step_launch": "hip_graph" if args.graph else "eager",
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": round(ms_graph, 4),
        "roofline": dict(roof("hbm", lat_bytes, iso_ms["attn_partial"], HBM_PEAK_GBS, "GB/s",
                              "attn_split_latent_kernel (the dominant kernel, timed alone through spc_attn_partial: "
                              "each head gathers its selected latent rows; a row selected by several heads is "
                              "counted once here)", 1,
                              traffic.get("attn_partial")),
                         gathered_bytes_per_launch=int(gathered),
                         gathered_GBs=round(gathered / (iso_ms["attn_partial"] * 1e-3) / 1e9, 1)),
        "roofline_attn_call": roof("hbm", attn_bytes, iso_ms["attn"], HBM_PEAK_GBS, "GB/s",
                                   "spc_sparse_decode_attn, the whole stage-4 call: one attn_split_latent_kernel "
                                   "launch that writes the output where each head's budget fits one split (up to "
                                   "2048 rows, 512 or more heads), else the split kernel + attn_combine_kernel", 1,
                                   traffic.get("attn")),
        "roofline_scores": roof("mfma", score_flop, iso_ms["scores"], MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
                                "mla_scores_kernel (logits and per-tile max / sum exp; bf16 MFMA, fp32 query as "
                                "a hi/lo bf16 pair: 2 MFMAs per product)", 1),
        "roofline_scores_hbm": roof("hbm", score_bytes, iso_ms["scores"], HBM_PEAK_GBS, "GB/s",
                                    "mla_scores_kernel", 1, traffic.get("scores")),
        "roofline_scores_probs": roof("hbm", score_bytes, iso_ms["scores_probs"], HBM_PEAK_GBS, "GB/s",
                                      "mla_scores_kernel + scores_normalize_kernel (spc_retrieval_scores: the "
                                      "probabilities written; not on the step's path)", 0,
                                      traffic.get("scores_probs")),
        "stage_us_in_step": {k: round(v * 1e3, 2) for k, v in avg.items()},
        "call_us_isolated": {k: round(v * 1e3, 2) for k, v in iso_ms.items()},
        "isolated_inputs": {"step_bytes": int(step_bytes), "last_level_cache_bytes": LLC_BYTES,
                            "replayed_over": "rotating copies" if inputs is rotation else "the same buffers"},
        "elastic": {"rows_selected_per_step": sel, "distinct_rows_per_step": union,
                    "rows_changed_per_step": float(np.mean(churn)),
                    "resident_churn": round(float(np.mean(churn)) / sel, 4) if sel else None,
                    "host_link_bytes_per_step": 0},
    })
    if args.calibrate_copy:
        calibration_copies(torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_mla(p, w, Wm, args.cpu_seconds)
    return result


def bench_mla_literal(args, p, torch, W):
    """The MLA step in the literal form: per-head K/V slots, only the rows a head newly loads
    expanded (MFMA), attention over the slots; the absorbed step is timed beside it."""
    from speculative_kv_sparsity_amd import api
    from speculative_kv_sparsity_amd.driver import MlaDecoder, MlaLiteralDecoder, StageTimer

    K_, Wm = args.steps, args.warmup
    total = Wm + 2 * K_
    w = W.generate(p, device="cuda", seed=args.seed, steps=total)
    dec = MlaLiteralDecoder(p, w.latent, w.w_uk, w.w_uv)
    lens = torch.as_tensor(w.lengths, device="cuda")
    qn, qr = w.q_nope.contiguous(), w.q_rope.contiguous()
    torch.cuda.synchronize()
    for t in range(Wm):
        dec.step(qn[t], qr[t], lens[t])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(dec.main)
    for t in range(Wm, Wm + K_):
        dec.step(qn[t], qr[t], lens[t])
    e1.record(dec.main)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / K_

    names = ("absorb", "scores", "topk", "expand", "attn", "end")
    stage = {k: [] for k in names[:-1]}
    loaded, sel_rows = [], []
    for t in range(Wm + K_, total):
        tm = StageTimer()
        dec.step(qn[t], qr[t], lens[t], timer=tm)
        torch.cuda.synchronize()
        for a, z in zip(names[:-1], names[1:]):
            stage[a].append(tm.ms(a, z))
        loaded.append(int(dec.load_count.sum().item()))
        sel_rows.append(int(dec.sel_count.sum().item()))
    avg = {k: float(np.mean(v)) for k, v in stage.items()}

    tq, tr, tl = qn[total - 1], qr[total - 1], lens[total - 1]
    R = args.iso_reps
    xs = dec.exp_shape
    # one step reads every head's expanded slots (671 MB at 32K), past the last-level cache: the
    # attention calls are replayed over rotating copies of the slot store, the expansion over rotating
    # copies of the latent cache and the up-projections
    kx = rotation(dec.kv_exp)
    lx = rotation(dec.latent, dec.w_uk, dec.w_uv)

    def expand(st):
        lat, uk, uv = lx()
        api.spc_mla_expand(dec.shape, p.nope_dim, uv.shape[1], lat, uk, uv, dec.load_pos, dec.load_slot,
                           dec.load_count, kx()[0], tq, tr, dec.q_exp, stream=st)

    iso_ms = {
        "expand": iso(torch, expand, R),
        "attn": iso(torch, lambda st: api.spc_sparse_decode_attn(
            xs, dec.q_exp, dec.exp_q_l, kx()[0], dec.exp_l, dec.slot_pos, None, api.SPC_ROWS_SLOTS, 0, 1, dec.out,
            ws=dec.ws_exp_attn, stream=st), R),
        "attn_partial": iso(torch, lambda st: api.spc_attn_partial(
            xs, dec.q_exp, dec.exp_q_l, kx()[0], dec.exp_l, dec.slot_pos, None, api.SPC_ROWS_SLOTS, 0, 1,
            dec.ws_exp_attn, stream=st), R),
    }
    # the absorbed step on the same inputs, for comparison
    ab = MlaDecoder(p, w.latent, w.w_uk, w.w_uv)
    for t in range(Wm):
        ab.step(qn[t], qr[t], lens[t])
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(ab.main)
    for t in range(Wm, Wm + K_):
        ab.step(qn[t], qr[t], lens[t])
    a1.record(ab.main)
    torch.cuda.synchronize()
    absorbed_ms = a0.elapsed_time(a1) / K_

    B, H, L = p.batch, p.n_q_heads, p.max_len
    sel = float(np.mean(sel_rows))
    rows_new = float(np.mean(loaded))
    dn, dr, dv, C = p.nope_dim, p.rope_dim, w.w_uv.shape[1], p.latent_dim
    row_exp = (dn + dr + dv) * p.elem_bytes                       # one expanded K||V slot row
    kv_bytes = sel * row_exp                                       # every selected slot read once
    exp_flop = 2.0 * rows_new * C * (dn + dv)                      # K and V up-projection of the new rows
    exp_bytes = rows_new * ((C + dr) * p.elem_bytes + row_exp) + 2 * H * dn * C * p.elem_bytes
    config = {"workload": "mla_32k, literal expansion: " + WORKLOADS["mla_32k"] if p.name == "mla_32k" else p.name,
              "batch": B, "layers": 1, "q_heads": H, "latent_dim": C, "rope_dim": dr, "nope_dim": dn,
              "cached_tokens": L, "kv_budget": p.budget, "form": "literal (per-head expanded K/V slots)",
              "parallelism": "single GPU"}
    result = _header(args, p, ms_per_step, config)
    result.update({
        "roofline": roof("hbm", kv_bytes, iso_ms["attn_partial"], HBM_PEAK_GBS, "GB/s",
                         "attn_split_kernel<bf16, 192, 128> (the dominant kernel: every head over its expanded "
                         "slots, timed alone through spc_attn_partial)", 1),
        "roofline_attn_call": roof("hbm", kv_bytes + B * H * dv * 4, iso_ms["attn"], HBM_PEAK_GBS, "GB/s",
                                   "attn_split_kernel + attn_combine_kernel (the whole stage-4 call)", 1),
        "roofline_expand": roof("mfma", exp_flop, iso_ms["expand"], MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
                                "mla_expand_kernel (the newly loaded rows of every head up-projected to K and V "
                                "on bf16 MFMA)", 1),
        "roofline_expand_hbm": roof("hbm", exp_bytes, iso_ms["expand"], HBM_PEAK_GBS, "GB/s",
                                    "mla_expand_kernel (each new latent row read once + its K||V slot row "
                                    "written + W_UK and W_UV)", 1),
        "stage_us_in_step": {k: round(v * 1e3, 2) for k, v in avg.items()},
        "call_us_isolated": {k: round(v * 1e3, 2) for k, v in iso_ms.items()},
        "absorbed_form": {"ms_per_step": round(absorbed_ms, 4), "steps_per_s": round(1e3 / absorbed_ms, 2)},
        "elastic": {"rows_selected_per_step": sel, "rows_expanded_per_step": rows_new,
                    "expanded_fraction": round(rows_new / sel, 4) if sel else None, "host_link_bytes_per_step": 0},
    })
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_mla(p, w, Wm, args.cpu_seconds)
    return result


def cpu_baseline_mla(p, w, t, budget_s):
    """The CPU oracle's MLA step (literal expansion of the keys and of the selected rows), timed
    per (sequence, head) on a bounded sample and scaled to whole steps of all heads and sequences."""
    from oracle import spc_oracle as O
    from speculative_kv_sparsity_amd.workload import to_numpy_raw
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    C = p.latent_dim
    lat = O.to_f64(to_numpy_raw(w.latent), "bf16")
    w_uk = O.to_f64(to_numpy_raw(w.w_uk), "bf16")
    w_uv = O.to_f64(to_numpy_raw(w.w_uv), "bf16")
    qn = O.to_f64(to_numpy_raw(w.q_nope[t]), "bf16")
    qr = O.to_f64(to_numpy_raw(w.q_rope[t]), "bf16")
    n_done, start = 0, time.perf_counter()
    b = 0
    h = 0
    while True:
        n = int(w.lengths[t][b])
        probs = O.mla_retrieval_scores(qn[b:b + 1], qr[b:b + 1], lat[b:b + 1, :, :C], lat[b:b + 1, :, C:], w_uk,
                                       [n], p.scale, heads=[h])[(0, h)]
        sel = O.topk_select(probs, n, p.budget)
        O.mla_sparse_attention(qn[b, h], qr[b, h], lat[b, :, :C], lat[b, :, C:], w_uk, w_uv, sel, h, p.scale)
        n_done += 1
        h = (h + 1) % p.n_q_heads
        if time.perf_counter() - start >= budget_s:
            break
    el = time.perf_counter() - start
    per_step = el / n_done * p.batch * p.n_q_heads
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "nproc": usable, "host_cpus": os.cpu_count(),
            "sample": f"{n_done} (sequence 0, head) scoring + Top-K + attention evaluations of one step "
                      f"(fp64 NumPy, keys expanded literally), {el:.1f} s, scaled by "
                      f"{p.batch} x {p.n_q_heads} to whole steps"}


if __name__ == "__main__":
    main()
