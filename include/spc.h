/*
 * spc.h - C ABI of the MI355X (gfx950) sparse-KV decode path of SpeContext
 * ("speculative context sparsity", Xu et al.).
 *
 * One decode step is four stages; each is a call below and runs as
 * hand-written HIP kernels on the caller's stream(s):
 *
 *   spc_retrieval_scores     per-head attention weights softmax(q K^T / sqrt(d))
 *                            of the retrieval head over every cached key
 *   spc_group_max_topk       element-wise max over each GQA group, then the
 *                            Top-K positions per group (the KV budget)
 *   spc_elastic_update       to_load = selected - resident; copy only those
 *                            K/V rows, in place, from pinned host memory into
 *                            the freed device slots
 *   spc_sparse_decode_attn   decode attention over the resident sparse KV only
 *
 * Conventions shared by every call:
 *   - All calls are asynchronous on the given HIP stream(s) (void* holding a
 *     hipStream_t; NULL = the null stream).  None allocates device memory,
 *     frees, or synchronizes.  Device faults surface at the caller's next
 *     synchronization.
 *   - The caller owns every buffer.  Device buffers are plain device pointers.
 *     Scratch space is the caller's `ws` buffer of at least
 *     spc_workspace_size(call, shape) bytes; ws contents need no
 *     initialization and are not preserved between calls.
 *   - Every argument is validated on the host before anything is launched;
 *     a call that returns an error has launched nothing.
 *   - Device pointers of vector data must be 16-byte aligned.
 *   - Errors are returned as spc_status; spc_last_error() gives a
 *     thread-local message for the last failing call.  Nothing aborts or
 *     prints across the ABI.
 *   - lengths[b] (valid cached positions of sequence b) are clamped to
 *     [0, max_len] on the device.
 *   - Head maps: query head i reads KV head i / (n_q_heads / n_kv_heads) and
 *     belongs to selection group i / (n_q_heads / n_groups) (consecutive
 *     heads share).  GQA: n_groups = n_kv_heads; MQA: n_groups = 1;
 *     MHA: n_groups = n_q_heads = n_kv_heads; MLA (one shared latent KV
 *     head): n_kv_heads = 1, n_groups = n_q_heads.  One of n_groups and
 *     n_kv_heads divides the other: a group lies within one KV head, or a KV
 *     head within one group.  The second case includes the batch-level
 *     selection the SpeContext blog (section 5, "C1") and the paper summary
 *     (section 4.2) set against head-level retrieval: n_groups = 1 over several
 *     KV heads, one selection shared by every head of the sequence, ranked by
 *     the element-wise max over all of its query heads.
 */
#ifndef SPC_H
#define SPC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: adds spc_mla_attn_out_proj */
#define SPC_ABI_VERSION 3

typedef enum spc_status {
  SPC_OK = 0,
  SPC_ERR_INVALID_ARG = 1,  /* null pointer, bad size, head counts that do not divide, misalignment */
  SPC_ERR_UNSUPPORTED = 2,  /* a dtype / head_dim combination this library does not build */
  SPC_ERR_WORKSPACE = 3,    /* ws smaller than spc_workspace_size() */
  SPC_ERR_NOT_MAPPED = 4,   /* host KV pointer is not pinned, device-mapped memory */
  SPC_ERR_HIP = 5           /* a HIP runtime call or launch failed; see spc_last_error() */
} spc_status;

typedef enum spc_dtype { SPC_F32 = 0, SPC_BF16 = 1 } spc_dtype;

/* Problem shape, shared by all calls. */
typedef struct spc_shape {
  int32_t batch;       /* B: sequences */
  int32_t n_q_heads;   /* H_q */
  int32_t n_kv_heads;  /* H_kv: key heads of the scored cache (MLA: 1) */
  int32_t n_groups;    /* selection groups (see head maps above) */
  int32_t head_dim;    /* d of the scored keys: 128 (MLA: 512 latent + 64 rope = 576) */
  int32_t v_dim;       /* value dimension: 128 (MLA: 512) */
  int32_t max_len;     /* L_max: capacity of the position axis */
  int32_t budget;      /* K: KV budget per group, 1 <= K <= max_len */
  int32_t n_layers;    /* target layers held in the KV stores */
  int32_t dtype;       /* spc_dtype of q, keys and K/V */
  float scale;         /* logit scale, 1/sqrt(d) (MLA: 1/sqrt(192)) */
} spc_shape;

/* Element strides (not bytes) of a K/V store, host or device.  A K row of
 * head_dim elements and a V row of v_dim elements are each contiguous
 * (unit stride).  Row `r` of layer `l`, KV head `h`, sequence `b`:
 *   K at  base + b*s_b + l*s_layer + h*s_head + r*s_row
 *   V at  the same + s_kv
 * s_kv = 0 reads V from the first v_dim elements of the K row (MLA latent). */
typedef struct spc_kv_layout {
  int64_t s_b, s_layer, s_head, s_row, s_kv;
} spc_kv_layout;

/* Element strides of the per-layer target queries q[b][layer][head][0..d).
 * s_layer = 0 lets every layer read the same query. */
typedef struct spc_q_layout {
  int64_t s_b, s_layer, s_head;
} spc_q_layout;

/* which_call for spc_workspace_size */
enum { SPC_CALL_SCORES = 1, SPC_CALL_TOPK = 2, SPC_CALL_ELASTIC = 3, SPC_CALL_ATTN = 4, SPC_CALL_FRONT = 5 };

/* Rotary position embedding of the retrieval head (spc_retrieval_head_qk): frequencies
 * theta_i = base^(-2i/d) on the dimension pairs (i, i + d/2), extended by YaRN when
 * factor > 1 (Peng et al. 2023, "NTK-by-parts"): with r_i = orig_max_pos * theta_i / (2 pi)
 * rotations over the trained context and ramp = clamp((r_i - beta_slow) / (beta_fast -
 * beta_slow), 0, 1), theta'_i = ramp * theta_i + (1 - ramp) * theta_i / factor, and q and k
 * are both multiplied by 0.1 ln(factor) + 1. */
typedef struct spc_rope {
  float base;            /* rotary base */
  float factor;          /* YaRN context scale; <= 1 gives plain rotary embedding */
  int32_t orig_max_pos;  /* context length the frequencies were trained for (> 0) */
  float beta_fast;       /* ramp end (rotations), > beta_slow */
  float beta_slow;       /* ramp start (rotations) */
} spc_rope;

/* flags of spc_elastic_update */
enum { SPC_PLAN = 1u, SPC_COPY = 2u };

/* row modes of spc_sparse_decode_attn */
enum {
  SPC_ROWS_SLOTS = 0,  /* rows = slot map [B][n_groups][budget]; slot x is attended iff rows[x] >= 0,
                          and its K/V is row x of the store */
  SPC_ROWS_GATHER = 1  /* rows = position lists [B][n_groups][budget], first row_count[b][g] valid;
                          K/V is row rows[i] of the store (e.g. selections into a full cache) */
};

int spc_abi_version(void);
const char* spc_status_string(int status);
const char* spc_last_error(void);

/* Bytes of scratch the call needs for this shape (0 if none). */
size_t spc_workspace_size(int which_call, const spc_shape* s);

/*
 * Retrieval-head front end, upstream of stage 1 (SpeContext blog section 5 "C1":
 * the retrieval head keeps the distilled model's embedding and Query/Key
 * projections; paper summary section 4.1: EAGLE-3's single decoder layer, its 2K
 * context extended with training-free YaRN; section 4.3).  For each sequence b
 * with new token t = tokens[b] at position p = positions[b]:
 *   x = emb[t];  x^ = gamma * x / sqrt(mean(x^2) + eps)       (the layer's input norm)
 *   q = rope_p(W_q x^) -> q_out[b]                            [H_q][head_dim]
 *   k = rope_p(W_k x^) -> dlm_k[b][g][p] for 0 <= p < max_len [H_kv][head_dim]
 * rope_p rotates the pairs (i, i + head_dim/2) by p * theta'_i (see spc_rope).  Results
 * are rounded to s->dtype (bf16: nearest even); accumulation is float32, the rotation
 * angle is reduced in double precision.  The new key becomes a candidate of stage 1
 * once lengths[b] > p (the next step of a growing sequence).
 *   hidden     multiple of 1024, <= 16384          vocab  rows of emb (>= 1)
 *   tokens, positions  device int32 [B]; a token outside [0, vocab) gives zero q and k
 *   emb    device [vocab][hidden]       gamma device [hidden]
 *   wq     device [H_q * head_dim][hidden]   wk device [H_kv * head_dim][hidden]
 *          (row h * head_dim + i produces dimension i of head h); all s->dtype
 *   q_out  device [B][H_q][head_dim] s->dtype        dlm_k device [B][H_kv][max_len][head_dim] (in/out)
 *   ws     spc_workspace_size(SPC_CALL_FRONT, s) bytes (float32 partial sums)
 * Supported: batch <= 16, head_dim 64 or 128, dtype bf16 or f32.
 */
int spc_retrieval_head_qk(const spc_shape* s, int32_t hidden, int64_t vocab, const spc_rope* rope, float eps,
                          const int32_t* tokens, const int32_t* positions, const void* emb, const void* gamma,
                          const void* wq, const void* wk, void* q_out, void* dlm_k, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Stage 1 - retrieval scores.  The retrieval head's attention weights of one
 * new query token over all cached keys, per query head:
 *   probs[b][i][j] = softmax_j( scale * q[b][i] . k[b][i / (H_q/H_kv)][j] ),  j < lengths[b]
 * (SpeContext blog section 2, AttentionWeight formula; blog section 5 and paper
 * summary sections 4.2-4.3: only the Q/K path of the distilled model is kept,
 * head-level weights.)
 *   q        device [B][H_q][head_dim], dtype s->dtype.  MLA shapes (head_dim 576): the float32
 *            absorbed query [B][H_q][576] written by spc_mla_absorb_q, scored on MFMA against
 *            the bf16 latent cache (n_kv_heads 1, H_q a multiple of 16, at most 128)
 *   k        device [B][H_kv][max_len][head_dim], dtype s->dtype
 *   lengths  device [B] int32
 *   probs    device [B][H_q][max_len] float32 out; entries j >= lengths[b] are left untouched
 * Requires head_dim % 8 == 0.  The softmax is exact up to float32 rounding
 * (all positions, no approximation).
 */
int spc_retrieval_scores(const spc_shape* s, const void* q, const void* k, const int32_t* lengths,
                         float* probs, void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 1 in log-domain form, for a caller that only ranks the weights (stage 2):
 * the same softmax as spc_retrieval_scores, kept as the logits plus what
 * normalises them, in one pass over the key cache (the probabilities are never
 * written).
 *   logits[b][i][j]     = scale * q[b][i] . k[b][i / (H_q/H_kv)][j],   j < lengths[b]
 *   tile_stats[b][i][t] = (m, s) with m = max and s = sum of exp(logit - m) over the
 *                         positions j < lengths[b] of tile t = [t T, (t+1) T),
 *                         T = spc_score_tile(s); tiles t >= ceil(lengths[b] / T) are
 *                         left untouched
 * so that probs[b][i][j] = exp(logits[b][i][j] - lse[b][i]) with lse the
 * log-sum-exp of the head's tile pairs (SpeContext blog section 2, AttentionWeight
 * formula; the same inputs and supported shapes as spc_retrieval_scores).
 *   logits      device [B][H_q][max_len] float32 out; entries j >= lengths[b] untouched
 *   tile_stats  device float32 pairs [B][H_q][ceil(max_len / T)] out, 8-byte aligned,
 *               tile_stats_bytes >= spc_tile_stats_size(s) (else SPC_ERR_INVALID_ARG); may be NULL
 *               (tile_stats_bytes ignored) when every query head is its own group
 *               (n_q_heads == n_groups): the Top-K then ranks the logits as they are and needs no
 *               stats, and none are computed; NULL with several heads per group is
 *               SPC_ERR_INVALID_ARG
 */
int spc_retrieval_logits(const spc_shape* s, const void* q, const void* k, const int32_t* lengths,
                         float* logits, float* tile_stats, size_t tile_stats_bytes, void* stream);

/* Positions per tile of the stage-1 statistics, 0 for an invalid shape: 128; MLA shapes 512 when
 * batch x ceil(H_q / 64) x ceil(max_len / 512) >= 512 (two scoring workgroups per CU), else 256. */
int spc_score_tile(const spc_shape* s);
/* Bytes of spc_retrieval_logits' tile_stats for the shape, 0 for an invalid shape. */
size_t spc_tile_stats_size(const spc_shape* s);

/*
 * Stage 2 - group max and Top-K.
 *   v[b][g][j] = max over the query heads i of group g of probs[b][i][j]
 *   S[b][g]    = the first min(K, n) positions j < n = lengths[b] ordered by
 *                (v desc, j asc): the lower index wins a tie (-0.0 and +0.0 are equal values)
 * (blog section 5, GQA element-wise max then per-group Top-K, MQA one group,
 * MHA per head; blog section 2, the KV budget K; paper summary section 4.3.)
 *   probs      device [B][H_q][max_len] float32 (as written by stage 1)
 *   sel_idx    device [B][n_groups][budget] int32 out: S ascending, -1 after sel_count
 *   sel_count  device [B][n_groups] int32 out: min(K, n)
 *   ws         scratch of spc_workspace_size(SPC_CALL_TOPK) bytes (the keys and
 *              first-digit histograms of the radix select)
 * The selection is exact on the float32 values (no approximation).
 */
int spc_group_max_topk(const spc_shape* s, const float* probs, const int32_t* lengths, int32_t* sel_idx,
                       int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 2 on the log-domain form of spc_retrieval_logits: the selection of
 * spc_group_max_topk, ranked by
 *   v[b][g][j] = exp( max over the query heads i of group g of (logits[b][i][j] - lse[b][i]) )
 * which is the group max of the probabilities (exp is increasing, so it commutes
 * with the max); lse[b][i] is the log-sum-exp of the head's tile pairs, formed here.
 * With one query head per group (MHA, MLA) the logits themselves are ranked (the
 * same order as the head's probabilities, without exp rounding) and tile_stats
 * may be NULL; otherwise it is required.
 *   logits, tile_stats  as written by spc_retrieval_logits for the same shape; tile_stats_bytes
 *               is the size of the tile_stats buffer, at least spc_tile_stats_size(s) when the
 *               stats are required (else SPC_ERR_INVALID_ARG), ignored when they are not
 *   sel_idx, sel_count, ws  as for spc_group_max_topk (same workspace size)
 * At most 64 query heads per group.  The selection is exact on the float32 values v
 * (as in the probability form, values below float32's range tie at zero).
 */
int spc_group_max_topk_logits(const spc_shape* s, const float* logits, const float* tile_stats,
                              size_t tile_stats_bytes, const int32_t* lengths, int32_t* sel_idx,
                              int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/*
 * Stage 2 and the plan of stage 3 in one call, as the step runs them: the selection of
 * spc_group_max_topk_logits, then the SPC_PLAN half of spc_elastic_update on it (blog section 4: the
 * retrieval head's Top-K, then to_load = selected - resident).  Where the selection, the plan's two
 * lists and a bitmap of the selection fit 64 KB of LDS (budget + max(4096, 2 budget + ceil(max_len/32))
 * words) and the two-phase select applies, the plan runs at the end of the Top-K's last kernel while
 * the selection is still in LDS; otherwise the plan is its own launch.  The outputs are exactly those
 * of the two calls.
 *   logits, tile_stats, tile_stats_bytes, lengths, sel_idx, sel_count, ws, ws_bytes
 *              as for spc_group_max_topk_logits (same workspace size)
 *   slot_pos, resident_bm, load_pos, load_slot, load_count
 *              as for spc_elastic_update (state in/out, plan out); budget <= 8192
 */
int spc_group_max_topk_plan_logits(const spc_shape* s, const float* logits, const float* tile_stats,
                                   size_t tile_stats_bytes, const int32_t* lengths, int32_t* sel_idx,
                                   int32_t* sel_count, int32_t* slot_pos, uint32_t* resident_bm,
                                   int32_t* load_pos, int32_t* load_slot, int32_t* load_count, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * Stage 3 - elastic loading (blog section 4 pseudocode: the positions to load
 * are the new selection minus the resident ones, fetched asynchronously; blog
 * section 6 worked example {1,8,21,35} -> {1,8,21,50} loads only 50, in place
 * of 35; paper summary section 5.4: fixed budget, in place).
 *
 * State, per (b, g), owned by the caller and initialised by spc_elastic_reset:
 *   slot_pos     device [B][n_groups][budget] int32: position held by slot x, or -1
 *   resident_bm  device [B][n_groups][ceil(max_len/32)] uint32: bit j set iff some
 *                slot holds position j
 * SPC_PLAN (on plan_stream):
 *   to_load = sorted(S - R) where R = {slot_pos[x] != -1}
 *   freed   = sorted slots that are empty or hold a position not in S
 *   load_pos[i] = to_load[i], load_slot[i] = freed[i], load_count = |to_load|;
 *   slot_pos[freed[i]] = to_load[i]; freed slots left over become -1; resident_bm
 *   follows.  Kept positions never move.  Entries after load_count are -1.
 *   load_pos, load_slot: device [B][n_groups][budget] int32; load_count [B][n_groups].
 * SPC_COPY (on copy_stream, reading the load lists): for every layer l in
 *   [layer_begin, layer_end), KV head h and i < load_count[b][g], g = h / (n_kv_heads / n_groups):
 *     dev_kv  K,V row load_slot[b][g][i] of (b, l, h)  <-  host_kv K,V row load_pos[b][g][i] of (b, l, h)
 *   (GQA: g = h.  n_groups must divide n_kv_heads: the device store has one slot row per
 *   (KV head, slot), and every KV head of a group holds the group's selection.)
 *   host_kv must be pinned host memory mapped for the device (hipHostMalloc,
 *   torch pin_memory=True); the device reads it directly over the host link.
 * With both flags, the plan runs on plan_stream and the copy on copy_stream;
 * the caller orders copy_stream after plan_stream (e.g. with an event) when they
 * differ.  Run SPC_PLAN exactly once per step: a repeated plan is empty.
 */
int spc_elastic_update(const spc_shape* s, const int32_t* sel_idx, const int32_t* sel_count, int32_t* slot_pos,
                       uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                       const void* host_kv, const spc_kv_layout* host_l, void* dev_kv,
                       const spc_kv_layout* dev_l, int32_t layer_begin, int32_t layer_end, unsigned flags,
                       void* plan_stream, void* copy_stream);

/* Empty every slot of sequence `batch_index` (or of all sequences if -1):
 * slot_pos = -1, resident_bm = 0.  The next plan loads its whole selection. */
int spc_elastic_reset(const spc_shape* s, int32_t batch_index, int32_t* slot_pos, uint32_t* resident_bm,
                      void* stream);

/*
 * Stage 3 for the pipelined loop of the SpeContext blog's section 4 (while the
 * target model attends over the sparse KV loaded in the previous iteration,
 * the retrieval head already selects the positions for the following one;
 * paper summary section 5.4: three sets, the previous selection, the current one
 * and the resident one).  Per (b, group):
 *   keep       = slots whose position is in cur or next (cur is being attended
 *                in this step, next will be);
 *   to_load    = next - resident, ascending, into the ascending remaining slots;
 *                leftover remaining slots become empty (-1);
 *   attend_rows = the ascending slots that hold cur after the update, followed by -1;
 *                attend_count = |cur| (the row list of spc_sparse_decode_attn in
 *                SPC_ROWS_GATHER mode over the pool).
 *   s        shape whose budget is the pool size P (>= 2 * sel_budget, <= 8192)
 *   sel_cur, cur_count, sel_next, next_count  device int32 [B][G][sel_budget], [B][G]
 *   slot_pos device int32 [B][G][P], resident_bm [B][G][ceil(max_len/32)]: state, in/out
 *   load_pos, load_slot [B][G][P], load_count [B][G]: out (input of spc_elastic_update SPC_COPY
 *            with the same pool shape)
 *   attend_rows [B][G][sel_budget], attend_count [B][G]: out
 * The copy that follows may run concurrently with this step's attention over
 * attend_rows (they touch different slots); it must follow the previous step's
 * attention, whose rows it may reuse.
 */
int spc_elastic_plan_lag1(const spc_shape* s, int32_t sel_budget, const int32_t* sel_cur, const int32_t* cur_count,
                          const int32_t* sel_next, const int32_t* next_count, int32_t* slot_pos,
                          uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                          int32_t* attend_rows, int32_t* attend_count, void* stream);

/*
 * Adaptive memory management (SpeContext blog section 7 "C3"; paper summary
 * sections 6.1-6.2.1): layers are offloaded to host memory one at a time, the
 * last layer still on the GPU first, as the sequence grows; an offloaded layer
 * keeps only its budget-sized working set (the slots of stage 3) on the GPU.
 * The memory model, with c layers offloaded at sequence length L:
 *   bytes(L, c) = fixed_bytes + L * token_bytes
 *               + (n_layers - c) * L * layer_token + c * budget * layer_token,
 *   layer_token = batch * n_kv_heads * (head_dim + v_dim) * elem_bytes.
 * spc_offload_thresholds writes threshold[c], c = 0..n_layers: the first length at
 * which c offloaded layers no longer fit in gpu_bytes (0 if not even an empty
 * cache fits, INT32_MAX if every int32 length fits).  The runtime rule is the
 * pages' loop: while seq_len >= threshold[c] and c < n_layers, offload one more.
 * Host-only arithmetic (no GPU); all sizes >= 0, n_layers, batch, heads >= 1.
 */
typedef struct spc_mem_model {
  int64_t gpu_bytes;    /* GPU memory the model may use */
  int64_t fixed_bytes;  /* everything independent of the length: weights, workspaces */
  int64_t token_bytes;  /* per cached position outside the target K/V (DLM keys, probabilities, ...) */
  int32_t n_layers, batch, n_kv_heads, head_dim, v_dim, budget, elem_bytes;
} spc_mem_model;

int spc_offload_thresholds(const spc_mem_model* m, int32_t* threshold /* [n_layers + 1] */);

/*
 * Stage 4 - sparse decode attention over the resident sparse KV only
 * (blog section 4 pseudocode, llm.forward(..., sparse_kv=resident_kv); the
 * AttentionWeight formula of blog section 2):
 *   out[b][l][i] = sum_r softmax_r(scale * q_l[b][i] . K[r]) V[r]
 * over the rows r of group i / (H_q/n_groups) (see row modes above), for every
 * layer l in [layer_begin, layer_end).
 *   q, q_l   device queries, dtype s->dtype, strides q_l (elements).  MLA shapes (head_dim 576):
 *            the float32 absorbed query, strides in float32 elements; kv is the latent
 *            cache with s_kv = 0 (V = the first 512 elements of each latent row)
 *   kv, kv_l device K/V store, dtype s->dtype (slots, or a full cache for GATHER).  The row
 *            stride s_row must be at least head_dim and v_dim, and the rows of one (sequence,
 *            layer, head) -- budget rows for SLOTS, max_len for GATHER -- must span under
 *            2 GiB (they are read through 32-bit ranges); otherwise SPC_ERR_UNSUPPORTED
 *   rows, row_count  see SPC_ROWS_*; row_count is ignored for SLOTS
 *   out      device [B][n_layers][H_q][v_dim] float32; only layers in range are written
 * A group with no rows writes zeros.  Accumulation is float32.
 */
int spc_sparse_decode_attn(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                           const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count,
                           int rows_mode, int32_t layer_begin, int32_t layer_end, float* out, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * spc_sparse_decode_attn without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, checks, kernels and output as spc_sparse_decode_attn, with the split-K
 * partials kept in a scratch array of 64 MiB that the library holds on each GPU it runs on until
 * the process ends.  The call allocates and frees nothing.
 *   - A layer range whose partials, batch x layers x H_q x splits x (v_dim + 2) x 4 bytes (splits =
 *     ceil(budget / 128), or / 64 with 8 query heads per workgroup), exceed 64 MiB is rejected with
 *     SPC_ERR_WORKSPACE before anything launches: split the layer range.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (on different
 *     streams, or from different threads) race and corrupt each other's outputs; order them.
 *   - The array keeps the last call's partials; no part of it needs to start at zero (every split
 *     writes all of its partials before the merge reads them).
 *   - The first call on a device resolves the array's device address (SPC_ERR_HIP if that fails).
 */
int spc_sparse_decode_attn_noalloc(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                                   const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count,
                                   int rows_mode, int32_t layer_begin, int32_t layer_end, float* out,
                                   void* stream);

/*
 * The two halves of spc_sparse_decode_attn (split-K), for a caller that runs them
 * apart (the merge on another stream, or later) or times them:
 *   spc_attn_partial  attends every split of the rows and leaves, in ws, each split's
 *                     unnormalised output and (max, sum of exp) per head, in the
 *                     library's own layout; same arguments as spc_sparse_decode_attn
 *                     without `out`
 *   spc_attn_merge    combines those splits with their log-sum-exp weights into `out`
 *                     for the same shape and layer range; ws is only read
 * spc_attn_partial followed by spc_attn_merge on one stream (or ordered by an event)
 * gives exactly the output of spc_sparse_decode_attn.
 */
int spc_attn_partial(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                     const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count, int rows_mode,
                     int32_t layer_begin, int32_t layer_end, void* ws, size_t ws_bytes, void* stream);
int spc_attn_merge(const spc_shape* s, int32_t layer_begin, int32_t layer_end, const void* ws, size_t ws_bytes,
                   float* out, void* stream);

/*
 * MLA helpers (SpeContext blog section 5, last paragraph; paper summary section
 * 4.3: MLA keeps a low-dimensional latent per position, retrieval stays
 * head-level, and only the selected latent rows are expanded).  The per-head
 * up-projections are absorbed into the query and the output, which equals
 * expanding the selected rows in real arithmetic:
 *   q_h . (W_UK[h] c_j || r_j) = (W_UK[h]^T q_nope_h || q_rope_h) . (c_j || r_j)
 *   sum_j w_j W_UV[h] c_j      = W_UV[h] (sum_j w_j c_j)
 * Shapes: head_dim 576 (latent 512 + rope 64), v_dim 512, n_kv_heads 1,
 * n_groups = n_q_heads, dtype bf16, batch <= 16.
 *
 * spc_mla_absorb_q: q_abs[b][h][0:512) = W_UK[h]^T q_nope[b][h], q_abs[b][h][512:576) = q_rope[b][h].
 *   w_uk   device bf16 [H][nope_dim][512]     q_nope device bf16 [B][H][nope_dim]
 *   q_rope device bf16 [B][H][64]             q_abs  device float32 [B][H][576] out
 */
int spc_mla_absorb_q(const spc_shape* s, int32_t nope_dim, const void* w_uk, const void* q_nope,
                     const void* q_rope, float* q_abs, void* stream);

/* spc_mla_out_proj: out[b][h][0:dv) = W_UV[h] o_lat[b][layer][h] (float32).
 *   w_uv   device bf16 [H][dv][512]
 *   o_lat  device float32 [B][n_layers][H][512], as written by spc_sparse_decode_attn
 *   out    device float32 [B][H][dv] out */
int spc_mla_out_proj(const spc_shape* s, int32_t dv, const void* w_uv, const float* o_lat, int32_t layer,
                     float* out, void* stream);

/* spc_mla_attn_out_proj: stage 4 of one MLA layer and the output projection in one call,
 *   out[b][h][0:dv) = W_UV[h] o[b][h],  o = the latent attention of spc_sparse_decode_attn
 * over the layer range [layer, layer + 1) with the same q, kv, rows and workspace arguments
 * (the absorbed form of the per-head output up-projection, SpeContext blog section 5 and paper
 * summary section 4.3, MLA bullet, as for spc_mla_out_proj).  Where each head's budget fits one
 * attention split (budget <= 2048 rows, batch x n_layers x n_q_heads >= 512) it is one launch, each
 * workgroup attending one head and projecting its output, and o_lat is not written; otherwise
 * spc_sparse_decode_attn writes o into o_lat and spc_mla_out_proj projects it, on the same stream.
 *   s, q, q_l, kv, kv_l, rows, row_count, rows_mode, ws, ws_bytes  as spc_sparse_decode_attn
 *          (an MLA shape: head_dim 576, v_dim 512, n_kv_heads 1, n_groups = n_q_heads, bf16)
 *   layer  the layer, in [0, n_layers)
 *   dv     output rows per head, in [1, 4096];  w_uv  device bf16 [H][dv][512]
 *   o_lat  device float32 [B][n_layers][H][512] (the second path's attention output)
 *   out    device float32 [B][H][dv] out
 * Errors: those of spc_sparse_decode_attn and spc_mla_out_proj, checked before any launch. */
int spc_mla_attn_out_proj(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                          const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count, int rows_mode,
                          int32_t layer, int32_t dv, const void* w_uv, float* o_lat, float* out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * MLA in the literal form (SpeContext blog section 5, last paragraph; paper summary
 * section 4.3, MLA bullet: only the selected latent rows are expanded, 512 ->
 * 128 x 128 K/V up-projection, before sparse attention): each head keeps its own
 * K/V slots, and a step expands only the rows the head newly loads (the load
 * lists of spc_elastic_update's plan for this shape), the rows it keeps stay
 * expanded from earlier steps:
 *   kv_exp[b][h][slot][0:128)   = bf16( W_UK[h] c_pos )      (nope part of the key)
 *   kv_exp[b][h][slot][128:192) = r_pos                      (rotary dims, copied)
 *   kv_exp[b][h][slot][192:320) = bf16( W_UV[h] c_pos )      (value)
 * for every (pos, slot) = (load_pos[b][h][i], load_slot[b][h][i]), i < load_count[b][h];
 * float32 accumulation on MFMA, rounded to nearest even.  With q_exp given,
 * q_exp[b][h] = q_nope[b][h] || q_rope[b][h] (bf16, [B][H][192]) as well: the head's
 * query against these keys.  Attention then runs with spc_sparse_decode_attn on
 * the shape (n_kv_heads = n_groups = H, head_dim 192, v_dim 128) over kv_exp as
 * slots (row stride 320 elements, V at offset 192); its output is the head's output
 * directly (no output projection).
 *   s          the MLA shape (head_dim 576, v_dim 512, n_kv_heads 1, n_groups = H, bf16,
 *              batch <= 16); budget = slots per head
 *   nope_dim, v_head_dim  128 each (the supported per-head dims)
 *   latent     device bf16 [B][max_len][576];  w_uk, w_uv device bf16 [H][128][512]
 *   load_pos, load_slot, load_count  device int32 [B][H][budget], [B][H] (plan output)
 *   kv_exp     device bf16 [B][H][budget][320]: only the listed slots are written
 *   q_nope, q_rope, q_exp  device bf16 [B][H][128], [B][H][64], [B][H][192], or all NULL
 */
int spc_mla_expand(const spc_shape* s, int32_t nope_dim, int32_t v_head_dim, const void* latent, const void* w_uk,
                   const void* w_uv, const void* q_nope, const void* q_rope, const int32_t* load_pos,
                   const int32_t* load_slot, const int32_t* load_count, void* kv_exp, void* q_exp, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPC_H */
