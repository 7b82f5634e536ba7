// Internal launchers of libspc: validated arguments in, kernels enqueued on a stream.
// Each returns hipSuccess or the launch error; the C-ABI layer (spc_api.cpp)
// validates every argument before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spc.h"

namespace spc {

// ---- stage 1: scores
constexpr int kScoreTile = 128;        // positions per workgroup of the logits kernel
constexpr int kMlaScoreTile = 256;     // positions per workgroup of the MLA scoring kernel
constexpr int kMlaScoreTileLarge = 512;   // the same when the grid still gives every CU two workgroups
constexpr int kNormChunk = 2048;       // positions per workgroup of the normalize kernel
size_t scores_ws_bytes(const spc_shape& s);
bool scores_supported(const spc_shape& s);
hipError_t launch_scores(const spc_shape& s, const void* q, const void* k, const int32_t* lengths, float* probs,
                         void* ws, hipStream_t st);
// one pass: logits and their per-tile (max, sum exp) stats [B*Hq][ceil(max_len/score_tile)]
hipError_t launch_logits(const spc_shape& s, const void* q, const void* k, const int32_t* lengths, float* logits,
                         float2* stats, hipStream_t st);
// rewrites logits as probabilities from per-tile (max, sum exp) partials [B*Hq][ntiles]
int mla_score_tile(const spc_shape& s);   // kMlaScoreTile or kMlaScoreTileLarge
int score_tile(const spc_shape& s);    // positions per (max, sum) partial of the scores workspace
hipError_t launch_scores_normalize(const spc_shape& s, float* probs, const float2* part, const int32_t* lengths,
                                   int ntiles, hipStream_t st);

// ---- MLA (latent 512 + rope 64, one shared latent KV head)
constexpr int kMlaLatent = 512;
constexpr int kMlaRope = 64;
constexpr int kMlaMaxBatch = 16;
bool mla_shape(const spc_shape& s);   // head_dim 576: the MLA layout
hipError_t launch_mla_absorb(int B, int H, int dn, const void* w_uk, const void* q_nope, const void* q_rope,
                             float* q_abs, hipStream_t st);
hipError_t launch_mla_logits(const spc_shape& s, const float* q_abs, const void* latent, const int32_t* lengths,
                             float* logits, float2* stats, hipStream_t st);
constexpr int kMlaExpandDims = 128;   // per-head nope / value dims of the literal expansion
hipError_t launch_mla_expand(const spc_shape& s, const void* latent, const void* w_uk, const void* w_uv,
                             const void* q_nope, const void* q_rope, const int32_t* load_pos,
                             const int32_t* load_slot, const int32_t* load_count, void* kv_exp, void* q_exp,
                             hipStream_t st);
hipError_t launch_mla_out_proj(int B, int H, int dv, const void* w_uv, const float* o_lat, int64_t lat_b_stride,
                               float* out, hipStream_t st);

// ---- stage 2: group max + Top-K
constexpr int kTopkLdsKeys = 32768;    // lengths up to this keep their keys in LDS
constexpr int kKeyChunk = 1024;        // positions per workgroup of the key / first-digit kernel
constexpr int kMaxGroupHeads = 64;     // query heads per group of the log-domain ranking
size_t topk_ws_bytes(const spc_shape& s);
// scores: probabilities (stats NULL) or logits with per-tile (max, sum exp) stats of
// stat_tile positions [B*Hq][ceil(max_len/stat_tile)] (NULL allowed with one head per group)
hipError_t launch_topk(const spc_shape& s, const float* scores, const float2* stats, int stat_tile,
                       const int32_t* lengths, int32_t* sel_idx, int32_t* sel_count, void* ws, hipStream_t st);
// stage 2 and the elastic plan in one launch sequence (the plan inside the Top-K's last kernel) where
// select_plan_fused(s); same workspace as launch_topk
bool select_plan_fused(const spc_shape& s);
hipError_t launch_select_plan(const spc_shape& s, const float* scores, const float2* stats, int stat_tile,
                              const int32_t* lengths, int32_t* sel_idx, int32_t* sel_count, int32_t* slot_pos,
                              uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                              void* ws, hipStream_t st);

// ---- stage 3: elastic plan / copy / reset
constexpr int kPlanMaxBudget = 8192;
constexpr size_t kPlanBmLdsBytes = 65536;  // the bitmap plan: two K-lists + the bitmap of S in LDS
constexpr int kPlanLag1MaxWords = 16384;   // 3 selections' + 2 pools' int32 in 64 KB of LDS
constexpr int kCopyMaxInstances = 4096;
constexpr int kCopyBlocksDefault = 48;   // workgroups of the gather (override: SPC_COPY_BLOCKS)
hipError_t launch_plan(const spc_shape& s, const int32_t* sel_idx, const int32_t* sel_count, int32_t* slot_pos,
                       uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                       hipStream_t st);
hipError_t launch_plan_lag1(const spc_shape& s, int sel_budget, const int32_t* sel_cur, const int32_t* cur_count,
                            const int32_t* sel_next, const int32_t* next_count, int32_t* slot_pos,
                            uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                            int32_t* attend_rows, int32_t* attend_count, hipStream_t st);
hipError_t launch_copy(const spc_shape& s, const int32_t* load_pos, const int32_t* load_slot,
                       const int32_t* load_count, const void* host_dev_ptr, const spc_kv_layout& hl, void* dev_kv,
                       const spc_kv_layout& dl, int layer_begin, int layer_end, hipStream_t st);
hipError_t launch_reset(const spc_shape& s, int batch_begin, int batch_end, int32_t* slot_pos,
                        uint32_t* resident_bm, hipStream_t st);

// ---- retrieval-head front end (token -> stage-1 query, DLM key append)
constexpr int kFrontSlice = 1024;      // hidden elements per GEMV workgroup slice
constexpr int kFrontMaxSlices = 16;    // hidden <= 16384
constexpr int kFrontMaxBatch = 16;
constexpr int kFrontMaxHeadDim = 128;
size_t front_ws_bytes(const spc_shape& s);
hipError_t launch_front(const spc_shape& s, int hidden, int64_t vocab, const spc_rope& rope, float eps,
                        const int32_t* tokens, const int32_t* positions, const void* emb, const void* gamma,
                        const void* wq, const void* wk, void* q_out, void* dlm_k, void* ws, hipStream_t st);

// ---- stage 4: sparse decode attention
constexpr int kCombineMaxSplits = 1024;  // splits per head the combine merges
size_t attn_ws_bytes(const spc_shape& s);
bool attn_supported(const spc_shape& s);
int attn_splits(const spc_shape& s);     // row splits per (instance, head)
hipError_t launch_attn(const spc_shape& s, const void* q, const spc_q_layout& ql, const void* kv,
                       const spc_kv_layout& kl, const int32_t* rows, const int32_t* row_count, int mode,
                       int layer_begin, int layer_end, float* out, void* ws, hipStream_t st);
// the two halves of launch_attn: the split kernel (partials into ws) and the merge
hipError_t launch_attn_partial(const spc_shape& s, const void* q, const spc_q_layout& ql, const void* kv,
                               const spc_kv_layout& kl, const int32_t* rows, const int32_t* row_count, int mode,
                               int layer_begin, int layer_end, void* ws, hipStream_t st);
size_t attn_ws_bytes_layers(const spc_shape& s, int n_lay);   // the partials of n_lay layers of one call
hipError_t launch_attn_merge(const spc_shape& s, int layer_begin, int layer_end, const void* ws, float* out,
                             hipStream_t st);
// MLA: the latent attention of one layer and its output projection W_UV[h] o[h] -> out [B][H][dv]; one
// launch where each head's budget fits one split (o_lat not written), else the attention into o_lat
// and launch_mla_out_proj
bool latent_one_split(const spc_shape& s);
hipError_t launch_mla_attn_out_proj(const spc_shape& s, const void* q, const spc_q_layout& ql, const void* kv,
                                    const spc_kv_layout& kl, const int32_t* rows, const int32_t* row_count,
                                    int mode, int layer, int dv, const void* w_uv, float* o_lat, float* out, void* ws,
                                    hipStream_t st);

}  // namespace spc
