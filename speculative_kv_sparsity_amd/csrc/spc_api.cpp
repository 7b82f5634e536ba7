// C ABI of libspc: argument validation, workspace sizes, error reporting and
// dispatch to the HIP launchers.  Nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/spc.h"
#include "spc_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SPC_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SPC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_bytes(const spc_shape* s) { return s->dtype == SPC_BF16 ? 2 : 4; }

constexpr int kMaxGridY = 65535;      // workgroups in the second and third grid dimensions

int check_shape(const spc_shape* s) {
  if (!s) return fail(SPC_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_groups < 1)
    return fail(SPC_ERR_INVALID_ARG, "batch and head counts must be >= 1");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(SPC_ERR_INVALID_ARG, "n_q_heads (%d) %% n_kv_heads (%d) != 0", s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads % s->n_groups != 0)
    return fail(SPC_ERR_INVALID_ARG, "n_q_heads (%d) %% n_groups (%d) != 0", s->n_q_heads, s->n_groups);
  // each group lies within one KV head (GQA, MHA, MLA), or each KV head within one group (one
  // selection shared by the heads of several KV heads, e.g. all of them)
  if (s->n_groups % s->n_kv_heads != 0 && s->n_kv_heads % s->n_groups != 0)
    return fail(SPC_ERR_INVALID_ARG, "n_groups (%d) and n_kv_heads (%d): neither divides the other", s->n_groups,
                s->n_kv_heads);
  if (s->max_len < 1) return fail(SPC_ERR_INVALID_ARG, "max_len must be >= 1");
  if (s->budget < 1 || s->budget > s->max_len)
    return fail(SPC_ERR_INVALID_ARG, "budget (%d) must be in [1, max_len=%d]", s->budget, s->max_len);
  if (s->n_layers < 1) return fail(SPC_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (s->dtype != SPC_F32 && s->dtype != SPC_BF16) return fail(SPC_ERR_UNSUPPORTED, "dtype %d", s->dtype);
  if (s->head_dim < 1 || s->v_dim < 1) return fail(SPC_ERR_INVALID_ARG, "head_dim and v_dim must be >= 1");
  if (!(s->scale > 0.f)) return fail(SPC_ERR_INVALID_ARG, "scale must be > 0");
  // (sequence, query head) and (sequence, group) instances index the second grid dimension
  if ((long long)s->batch * s->n_q_heads > kMaxGridY)
    return fail(SPC_ERR_UNSUPPORTED, "batch * n_q_heads = %lld exceeds %d", (long long)s->batch * s->n_q_heads,
                kMaxGridY);
  return SPC_OK;
}

hipStream_t as_stream(void* p) { return static_cast<hipStream_t>(p); }

}  // namespace

// Scratch of spc_sparse_decode_attn_noalloc: the split-K partials of one call live in this array,
// which the HIP runtime places in each GPU's memory when it loads the library's code there and
// keeps until the process ends.  Host code never passes its name to a kernel (in host code the name
// is a stand-in, not a device address): scratch_address() resolves the device address, once per
// device, and every launch uses that.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];       // device address of `scratch` per device, resolved on first use

// The device address of `scratch` on the current device (hipGetSymbolAddress with that device current,
// checked, kept per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SPC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPC_OK;
}

}  // namespace

extern "C" {

int spc_abi_version(void) { return SPC_ABI_VERSION; }

const char* spc_status_string(int status) {
  switch (status) {
    case SPC_OK: return "ok";
    case SPC_ERR_INVALID_ARG: return "invalid argument";
    case SPC_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SPC_ERR_WORKSPACE: return "workspace too small";
    case SPC_ERR_NOT_MAPPED: return "host pointer is not pinned device-mapped memory";
    case SPC_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* spc_last_error(void) { return g_last_error.c_str(); }

size_t spc_workspace_size(int which_call, const spc_shape* s) {
  if (check_shape(s) != SPC_OK) return 0;
  switch (which_call) {
    case SPC_CALL_SCORES: return spc::scores_ws_bytes(*s);
    case SPC_CALL_TOPK: return spc::topk_ws_bytes(*s);
    case SPC_CALL_ATTN: return spc::attn_ws_bytes(*s);
    case SPC_CALL_FRONT: return spc::front_ws_bytes(*s);
    default: return 0;
  }
}

int spc_score_tile(const spc_shape* s) { return check_shape(s) == SPC_OK ? spc::score_tile(*s) : 0; }

size_t spc_tile_stats_size(const spc_shape* s) { return check_shape(s) == SPC_OK ? spc::scores_ws_bytes(*s) : 0; }

int spc_retrieval_scores(const spc_shape* s, const void* q, const void* k, const int32_t* lengths, float* probs,
                         void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_shape(s)) return e;
  if (!q || !k || !lengths || !probs) return fail(SPC_ERR_INVALID_ARG, "NULL q, k, lengths or probs");
  if (!spc::scores_supported(*s))
    return fail(SPC_ERR_UNSUPPORTED, "retrieval scores: head_dim %d with dtype %d", s->head_dim, s->dtype);
  if (!aligned16(q) || !aligned16(k)) return fail(SPC_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (!aligned4(probs) || !aligned4(lengths)) return fail(SPC_ERR_INVALID_ARG, "probs/lengths misaligned");
  const size_t need = spc::scores_ws_bytes(*s);
  if (ws_bytes < need || (need && !ws))
    return fail(SPC_ERR_WORKSPACE, "retrieval scores need %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(SPC_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const hipError_t e = spc::launch_scores(*s, q, k, lengths, probs, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "retrieval scores launch");
}

int spc_retrieval_logits(const spc_shape* s, const void* q, const void* k, const int32_t* lengths, float* logits,
                         float* tile_stats, size_t tile_stats_bytes, void* stream) {
  if (int e = check_shape(s)) return e;
  if (!q || !k || !lengths || !logits)
    return fail(SPC_ERR_INVALID_ARG, "NULL q, k, lengths or logits");
  if (!tile_stats && s->n_q_heads != s->n_groups)
    return fail(SPC_ERR_INVALID_ARG, "tile_stats are needed with %d query heads per group",
                s->n_q_heads / s->n_groups);
  if (!spc::scores_supported(*s))
    return fail(SPC_ERR_UNSUPPORTED, "retrieval logits: head_dim %d with dtype %d", s->head_dim, s->dtype);
  if (!aligned16(q) || !aligned16(k)) return fail(SPC_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (!aligned4(logits) || !aligned4(lengths)) return fail(SPC_ERR_INVALID_ARG, "logits/lengths misaligned");
  if ((reinterpret_cast<uintptr_t>(tile_stats) & 7u) != 0)
    return fail(SPC_ERR_INVALID_ARG, "tile_stats must be 8-byte aligned");
  if (tile_stats && tile_stats_bytes < spc::scores_ws_bytes(*s))
    return fail(SPC_ERR_INVALID_ARG, "tile_stats holds %zu bytes, the shape needs %zu", tile_stats_bytes,
                spc::scores_ws_bytes(*s));
  const hipError_t e = spc::launch_logits(*s, q, k, lengths, logits, reinterpret_cast<float2*>(tile_stats),
                                          as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "retrieval logits launch");
}

namespace {
// Arguments of stage 2 on the log-domain form (spc_group_max_topk_logits and the fused call).
int check_topk_logits(const spc_shape* s, const float* logits, const float* tile_stats, size_t tile_stats_bytes,
                      const int32_t* lengths, int32_t* sel_idx, int32_t* sel_count, void* ws, size_t ws_bytes) {
  if (int e = check_shape(s)) return e;
  if (!logits || !lengths || !sel_idx || !sel_count)
    return fail(SPC_ERR_INVALID_ARG, "NULL logits, lengths, sel_idx or sel_count");
  const int gq = s->n_q_heads / s->n_groups;
  if (gq > 1 && !tile_stats)
    return fail(SPC_ERR_INVALID_ARG, "tile_stats are needed with %d query heads per group", gq);
  if (gq > spc::kMaxGroupHeads)
    return fail(SPC_ERR_UNSUPPORTED, "%d query heads per group exceed %d", gq, spc::kMaxGroupHeads);
  if (!aligned4(logits) || !aligned4(sel_idx) || !aligned4(sel_count) || !aligned4(lengths))
    return fail(SPC_ERR_INVALID_ARG, "misaligned int32/float buffer");
  if ((reinterpret_cast<uintptr_t>(tile_stats) & 7u) != 0)
    return fail(SPC_ERR_INVALID_ARG, "tile_stats must be 8-byte aligned");
  if (gq > 1 && tile_stats_bytes < spc::scores_ws_bytes(*s))
    return fail(SPC_ERR_INVALID_ARG, "tile_stats holds %zu bytes, the shape needs %zu", tile_stats_bytes,
                spc::scores_ws_bytes(*s));
  const size_t need = spc::topk_ws_bytes(*s);
  if (ws_bytes < need || !ws)
    return fail(SPC_ERR_WORKSPACE, "group max / top-k needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(SPC_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return SPC_OK;
}
}  // namespace

int spc_group_max_topk_logits(const spc_shape* s, const float* logits, const float* tile_stats,
                              size_t tile_stats_bytes, const int32_t* lengths, int32_t* sel_idx, int32_t* sel_count,
                              void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_topk_logits(s, logits, tile_stats, tile_stats_bytes, lengths, sel_idx, sel_count, ws, ws_bytes))
    return e;
  const int gq = s->n_q_heads / s->n_groups;
  const float2* st = gq > 1 ? reinterpret_cast<const float2*>(tile_stats) : nullptr;
  const hipError_t e = spc::launch_topk(*s, logits, st, spc::score_tile(*s), lengths, sel_idx, sel_count, ws,
                                        as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "group max / top-k (logits) launch");
}

int spc_group_max_topk_plan_logits(const spc_shape* s, const float* logits, const float* tile_stats,
                                   size_t tile_stats_bytes, const int32_t* lengths, int32_t* sel_idx,
                                   int32_t* sel_count, int32_t* slot_pos, uint32_t* resident_bm, int32_t* load_pos,
                                   int32_t* load_slot, int32_t* load_count, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (int e = check_topk_logits(s, logits, tile_stats, tile_stats_bytes, lengths, sel_idx, sel_count, ws, ws_bytes))
    return e;
  if (!slot_pos || !resident_bm || !load_pos || !load_slot || !load_count)
    return fail(SPC_ERR_INVALID_ARG, "the plan needs slot_pos, resident_bm, load_pos, load_slot and load_count");
  if (!aligned4(slot_pos) || !aligned4(resident_bm) || !aligned4(load_pos) || !aligned4(load_slot) ||
      !aligned4(load_count))
    return fail(SPC_ERR_INVALID_ARG, "misaligned plan buffer");
  if (s->budget > spc::kPlanMaxBudget)
    return fail(SPC_ERR_UNSUPPORTED, "budget %d exceeds the plan kernel's %d", s->budget, spc::kPlanMaxBudget);
  const int gq = s->n_q_heads / s->n_groups;
  const float2* st = gq > 1 ? reinterpret_cast<const float2*>(tile_stats) : nullptr;
  hipError_t e;
  if (spc::select_plan_fused(*s)) {
    e = spc::launch_select_plan(*s, logits, st, spc::score_tile(*s), lengths, sel_idx, sel_count, slot_pos,
                                resident_bm, load_pos, load_slot, load_count, ws, as_stream(stream));
  } else {
    e = spc::launch_topk(*s, logits, st, spc::score_tile(*s), lengths, sel_idx, sel_count, ws, as_stream(stream));
    if (e == hipSuccess)
      e = spc::launch_plan(*s, sel_idx, sel_count, slot_pos, resident_bm, load_pos, load_slot, load_count,
                           as_stream(stream));
  }
  return e == hipSuccess ? ok() : hip_fail(e, "group max / top-k + plan launch");
}

int spc_group_max_topk(const spc_shape* s, const float* probs, const int32_t* lengths, int32_t* sel_idx,
                       int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_shape(s)) return e;
  if (!probs || !lengths || !sel_idx || !sel_count)
    return fail(SPC_ERR_INVALID_ARG, "NULL probs, lengths, sel_idx or sel_count");
  if (!aligned4(probs) || !aligned4(sel_idx) || !aligned4(sel_count) || !aligned4(lengths))
    return fail(SPC_ERR_INVALID_ARG, "misaligned int32/float buffer");
  const size_t need = spc::topk_ws_bytes(*s);
  if (ws_bytes < need || !ws)
    return fail(SPC_ERR_WORKSPACE, "group max / top-k needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(SPC_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const hipError_t e = spc::launch_topk(*s, probs, nullptr, 0, lengths, sel_idx, sel_count, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "group max / top-k launch");
}

int spc_elastic_update(const spc_shape* s, const int32_t* sel_idx, const int32_t* sel_count, int32_t* slot_pos,
                       uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                       const void* host_kv, const spc_kv_layout* host_l, void* dev_kv, const spc_kv_layout* dev_l,
                       int32_t layer_begin, int32_t layer_end, unsigned flags, void* plan_stream,
                       void* copy_stream) {
  if (int e = check_shape(s)) return e;
  if ((flags & ~(unsigned)(SPC_PLAN | SPC_COPY)) != 0 || flags == 0)
    return fail(SPC_ERR_INVALID_ARG, "flags must be a non-empty combination of SPC_PLAN and SPC_COPY");
  if (!load_pos || !load_slot || !load_count) return fail(SPC_ERR_INVALID_ARG, "NULL load lists");
  if (flags & SPC_PLAN) {
    if (!sel_idx || !sel_count || !slot_pos || !resident_bm)
      return fail(SPC_ERR_INVALID_ARG, "plan needs sel_idx, sel_count, slot_pos and resident_bm");
    if (s->budget > spc::kPlanMaxBudget)
      return fail(SPC_ERR_UNSUPPORTED, "budget %d exceeds the plan kernel's %d", s->budget, spc::kPlanMaxBudget);
  }
  const void* host_dev = nullptr;
  if (flags & SPC_COPY) {
    if (!host_kv || !host_l || !dev_kv || !dev_l)
      return fail(SPC_ERR_INVALID_ARG, "copy needs host_kv, host layout, dev_kv and device layout");
    if (s->n_kv_heads % s->n_groups != 0)
      return fail(SPC_ERR_UNSUPPORTED, "copy needs every KV head inside one selection group (n_kv_heads %% n_groups "
                  "== 0; %d KV heads, %d groups)", s->n_kv_heads, s->n_groups);
    if ((long long)s->batch * s->n_groups > spc::kCopyMaxInstances)
      return fail(SPC_ERR_UNSUPPORTED, "batch * n_groups exceeds %d", spc::kCopyMaxInstances);
    if (layer_begin < 0 || layer_end > s->n_layers || layer_begin >= layer_end)
      return fail(SPC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end,
                  s->n_layers);
    const int eb = elem_bytes(s);
    const double vecs = (double)s->batch * s->n_kv_heads * s->budget * (layer_end - layer_begin) *
                        ((double)(s->head_dim + s->v_dim) * eb / 16.0);
    if (vecs >= 4294967296.0)
      return fail(SPC_ERR_UNSUPPORTED, "copy of %.0f 16-byte vectors exceeds one launch; split the layer range",
                  vecs);
    if ((s->head_dim * eb) % 16 || (s->v_dim * eb) % 16)
      return fail(SPC_ERR_UNSUPPORTED, "K and V rows must be whole 16-byte vectors");
    const spc_kv_layout* ls[2] = {host_l, dev_l};
    for (const spc_kv_layout* l : ls) {
      if ((l->s_b * eb) % 16 || (l->s_layer * eb) % 16 || (l->s_head * eb) % 16 || (l->s_row * eb) % 16 ||
          (l->s_kv * eb) % 16)
        return fail(SPC_ERR_INVALID_ARG, "K/V layout strides must be multiples of 16 bytes");
    }
    if (!aligned16(host_kv) || !aligned16(dev_kv)) return fail(SPC_ERR_INVALID_ARG, "KV stores must be 16-byte aligned");
    hipPointerAttribute_t attr;
    hipError_t he = hipPointerGetAttributes(&attr, host_kv);
    if (he != hipSuccess || attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) {
      (void)hipGetLastError();
      return fail(SPC_ERR_NOT_MAPPED, "host_kv %p is not pinned, device-mapped host memory", host_kv);
    }
    host_dev = attr.devicePointer;
  }
  if (flags & SPC_PLAN) {
    const hipError_t e = spc::launch_plan(*s, sel_idx, sel_count, slot_pos, resident_bm, load_pos, load_slot,
                                          load_count, as_stream(plan_stream));
    if (e != hipSuccess) return hip_fail(e, "elastic plan launch");
  }
  if (flags & SPC_COPY) {
    const hipError_t e = spc::launch_copy(*s, load_pos, load_slot, load_count, host_dev, *host_l, dev_kv, *dev_l,
                                          layer_begin, layer_end, as_stream(copy_stream));
    if (e != hipSuccess) return hip_fail(e, "elastic copy launch");
  }
  return ok();
}

int spc_elastic_reset(const spc_shape* s, int32_t batch_index, int32_t* slot_pos, uint32_t* resident_bm,
                      void* stream) {
  if (int e = check_shape(s)) return e;
  if (!slot_pos || !resident_bm) return fail(SPC_ERR_INVALID_ARG, "NULL slot_pos or resident_bm");
  if (batch_index < -1 || batch_index >= s->batch)
    return fail(SPC_ERR_INVALID_ARG, "batch_index %d outside [-1, %d)", batch_index, s->batch);
  const int b0 = batch_index < 0 ? 0 : batch_index;
  const int b1 = batch_index < 0 ? s->batch : batch_index + 1;
  const hipError_t e = spc::launch_reset(*s, b0, b1, slot_pos, resident_bm, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "elastic reset launch");
}

}  // extern "C"

namespace {
// Arguments of the partial half (and of the whole call, which adds `out`).
int check_attn(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv, const spc_kv_layout* kv_l,
               const int32_t* rows, const int32_t* row_count, int rows_mode, int32_t layer_begin, int32_t layer_end,
               void* ws, size_t ws_bytes, size_t need) {
  if (int e = check_shape(s)) return e;
  if (!q || !q_l || !kv || !kv_l || !rows) return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (rows_mode != SPC_ROWS_SLOTS && rows_mode != SPC_ROWS_GATHER)
    return fail(SPC_ERR_INVALID_ARG, "rows_mode %d", rows_mode);
  if (rows_mode == SPC_ROWS_GATHER && !row_count) return fail(SPC_ERR_INVALID_ARG, "GATHER needs row_count");
  if (layer_begin < 0 || layer_end > s->n_layers || layer_begin >= layer_end)
    return fail(SPC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end, s->n_layers);
  if (!spc::attn_supported(*s))
    return fail(SPC_ERR_UNSUPPORTED, "attention: head_dim %d / v_dim %d with dtype %d", s->head_dim, s->v_dim,
                s->dtype);
  if (spc::attn_splits(*s) > spc::kCombineMaxSplits)
    return fail(SPC_ERR_UNSUPPORTED, "attention: budget %d needs more than %d row splits", s->budget,
                spc::kCombineMaxSplits);
  if ((long long)s->batch * (layer_end - layer_begin) * s->n_groups > kMaxGridY)
    return fail(SPC_ERR_UNSUPPORTED, "attention: batch * layers * n_groups exceeds %d (split the layer range)",
                kMaxGridY);
  if (s->head_dim == 576 && kv_l->s_kv != 0)
    return fail(SPC_ERR_UNSUPPORTED, "head_dim 576 reads V from the latent row itself (s_kv must be 0)");
  const int eb = elem_bytes(s);
  {                                         // one head's rows are read through 32-bit buffer ranges
    const long long span = (long long)(rows_mode == SPC_ROWS_SLOTS ? s->budget : s->max_len) * kv_l->s_row * eb;
    if (kv_l->s_row < s->head_dim || kv_l->s_row < s->v_dim || span >= (1LL << 31))
      return fail(SPC_ERR_UNSUPPORTED, "attention: the rows of one head span %lld bytes with row stride %lld "
                  "(the stride must cover a key and a value row; limit 2 GiB)", span, (long long)kv_l->s_row);
  }
  const int qeb = spc::mla_shape(*s) ? 4 : eb;   // MLA: float32 absorbed query
  if (!aligned16(q) || !aligned16(kv)) return fail(SPC_ERR_INVALID_ARG, "q and kv must be 16-byte aligned");
  if ((q_l->s_b * qeb) % 16 || (q_l->s_layer * qeb) % 16 || (q_l->s_head * qeb) % 16)
    return fail(SPC_ERR_INVALID_ARG, "query strides must be multiples of 16 bytes");
  if ((kv_l->s_b * eb) % 16 || (kv_l->s_layer * eb) % 16 || (kv_l->s_head * eb) % 16 || (kv_l->s_row * eb) % 16 ||
      (kv_l->s_kv * eb) % 16)
    return fail(SPC_ERR_INVALID_ARG, "K/V strides must be multiples of 16 bytes");
  if (ws_bytes < need || !ws)
    return fail(SPC_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(SPC_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return SPC_OK;
}
}  // namespace

extern "C" {

int spc_sparse_decode_attn(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                           const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count, int rows_mode,
                           int32_t layer_begin, int32_t layer_end, float* out, void* ws, size_t ws_bytes,
                           void* stream) {
  if (int e = check_attn(s, q, q_l, kv, kv_l, rows, row_count, rows_mode, layer_begin, layer_end, ws, ws_bytes,
                            spc::attn_ws_bytes(*s)))
    return e;
  if (!out || !aligned16(out)) return fail(SPC_ERR_INVALID_ARG, "out must be a 16-byte aligned device pointer");
  const hipError_t e = spc::launch_attn(*s, q, *q_l, kv, *kv_l, rows, row_count, rows_mode, layer_begin, layer_end,
                                        out, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "sparse decode attention launch");
}

int spc_sparse_decode_attn_noalloc(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                                   const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count,
                                   int rows_mode, int32_t layer_begin, int32_t layer_end, float* out, void* stream) {
  if (int e = check_shape(s)) return e;
  if (layer_begin < 0 || layer_end > s->n_layers || layer_begin >= layer_end)
    return fail(SPC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end, s->n_layers);
  if (!spc::attn_supported(*s))
    return fail(SPC_ERR_UNSUPPORTED, "attention: head_dim %d / v_dim %d with dtype %d", s->head_dim, s->v_dim,
                s->dtype);
  const size_t need = spc::attn_ws_bytes_layers(*s, layer_end - layer_begin);
  if (need > kNoAllocScratchBytes)
    return fail(SPC_ERR_WORKSPACE, "the allocation-free attention needs %zu bytes of scratch for %d layers, its "
                "array holds %zu: split the layer range, or call spc_sparse_decode_attn with a workspace", need,
                layer_end - layer_begin, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (int e = scratch_address(&ws)) return e;
  // the partials of this layer range only (the launch lays them out for [layer_begin, layer_end))
  if (int e = check_attn(s, q, q_l, kv, kv_l, rows, row_count, rows_mode, layer_begin, layer_end, ws,
                         kNoAllocScratchBytes, need))
    return e;
  if (!out || !aligned16(out)) return fail(SPC_ERR_INVALID_ARG, "out must be a 16-byte aligned device pointer");
  const hipError_t e = spc::launch_attn(*s, q, *q_l, kv, *kv_l, rows, row_count, rows_mode, layer_begin, layer_end,
                                        out, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "sparse decode attention (allocation-free) launch");
}

int spc_attn_partial(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                     const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count, int rows_mode,
                     int32_t layer_begin, int32_t layer_end, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_attn(s, q, q_l, kv, kv_l, rows, row_count, rows_mode, layer_begin, layer_end, ws, ws_bytes,
                            spc::attn_ws_bytes(*s)))
    return e;
  const hipError_t e = spc::launch_attn_partial(*s, q, *q_l, kv, *kv_l, rows, row_count, rows_mode, layer_begin,
                                                layer_end, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "partial attention launch");
}

int spc_attn_merge(const spc_shape* s, int32_t layer_begin, int32_t layer_end, const void* ws, size_t ws_bytes,
                   float* out, void* stream) {
  if (int e = check_shape(s)) return e;
  if (!ws || !out) return fail(SPC_ERR_INVALID_ARG, "NULL ws or out");
  if (layer_begin < 0 || layer_end > s->n_layers || layer_begin >= layer_end)
    return fail(SPC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end, s->n_layers);
  if (!spc::attn_supported(*s))
    return fail(SPC_ERR_UNSUPPORTED, "attention: head_dim %d / v_dim %d with dtype %d", s->head_dim, s->v_dim,
                s->dtype);
  if (spc::attn_splits(*s) > spc::kCombineMaxSplits)
    return fail(SPC_ERR_UNSUPPORTED, "attention: budget %d needs more than %d row splits", s->budget,
                spc::kCombineMaxSplits);
  if (ws_bytes < spc::attn_ws_bytes(*s))
    return fail(SPC_ERR_WORKSPACE, "attention merge reads %zu workspace bytes, got %zu", spc::attn_ws_bytes(*s),
                ws_bytes);
  if (!aligned16(ws) || !aligned16(out)) return fail(SPC_ERR_INVALID_ARG, "ws and out must be 16-byte aligned");
  const hipError_t e = spc::launch_attn_merge(*s, layer_begin, layer_end, ws, out, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "attention merge launch");
}

}  // extern "C"

namespace {
int check_mla(const spc_shape* s) {
  if (int e = check_shape(s)) return e;
  if (!spc::mla_shape(*s) || s->v_dim != spc::kMlaLatent || s->n_kv_heads != 1 || s->dtype != SPC_BF16)
    return fail(SPC_ERR_UNSUPPORTED, "MLA helpers need head_dim 576, v_dim 512, one latent head, bf16");
  if (s->batch > spc::kMlaMaxBatch) return fail(SPC_ERR_UNSUPPORTED, "MLA helpers support batch <= %d", spc::kMlaMaxBatch);
  return SPC_OK;
}
}  // namespace

extern "C" {

int spc_mla_absorb_q(const spc_shape* s, int32_t nope_dim, const void* w_uk, const void* q_nope,
                     const void* q_rope, float* q_abs, void* stream) {
  if (int e = check_mla(s)) return e;
  if (!w_uk || !q_nope || !q_rope || !q_abs) return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (nope_dim < 1 || nope_dim > 1024) return fail(SPC_ERR_INVALID_ARG, "nope_dim %d outside [1, 1024]", nope_dim);
  if (!aligned16(q_abs)) return fail(SPC_ERR_INVALID_ARG, "q_abs must be 16-byte aligned");
  const hipError_t e = spc::launch_mla_absorb(s->batch, s->n_q_heads, nope_dim, w_uk, q_nope, q_rope, q_abs,
                                              as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "MLA query absorption launch");
}

int spc_mla_out_proj(const spc_shape* s, int32_t dv, const void* w_uv, const float* o_lat, int32_t layer,
                     float* out, void* stream) {
  if (int e = check_mla(s)) return e;
  if (!w_uv || !o_lat || !out) return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (dv < 1 || dv > 4096) return fail(SPC_ERR_INVALID_ARG, "dv %d outside [1, 4096]", dv);
  if (layer < 0 || layer >= s->n_layers) return fail(SPC_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, s->n_layers);
  if (!aligned16(w_uv) || !aligned16(o_lat)) return fail(SPC_ERR_INVALID_ARG, "w_uv and o_lat must be 16-byte aligned");
  const int64_t b_stride = (int64_t)s->n_layers * s->n_q_heads * spc::kMlaLatent;
  const hipError_t e = spc::launch_mla_out_proj(s->batch, s->n_q_heads, dv, w_uv,
                                                o_lat + (size_t)layer * s->n_q_heads * spc::kMlaLatent, b_stride, out,
                                                as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "MLA output projection launch");
}

int spc_mla_attn_out_proj(const spc_shape* s, const void* q, const spc_q_layout* q_l, const void* kv,
                          const spc_kv_layout* kv_l, const int32_t* rows, const int32_t* row_count, int rows_mode,
                          int32_t layer, int32_t dv, const void* w_uv, float* o_lat, float* out, void* ws,
                          size_t ws_bytes, void* stream) {
  if (int e = check_mla(s)) return e;
  if (layer < 0 || layer >= s->n_layers) return fail(SPC_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, s->n_layers);
  if (int e = check_attn(s, q, q_l, kv, kv_l, rows, row_count, rows_mode, layer, layer + 1, ws, ws_bytes,
                         spc::attn_ws_bytes(*s)))
    return e;
  if (!w_uv || !o_lat || !out) return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (dv < 1 || dv > 4096) return fail(SPC_ERR_INVALID_ARG, "dv %d outside [1, 4096]", dv);
  if (!aligned16(w_uv) || !aligned16(o_lat) || !aligned16(out))
    return fail(SPC_ERR_INVALID_ARG, "w_uv, o_lat and out must be 16-byte aligned");
  const hipError_t e = spc::launch_mla_attn_out_proj(*s, q, *q_l, kv, *kv_l, rows, row_count, rows_mode, layer, dv,
                                                     w_uv, o_lat, out, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "MLA attention and output projection launch");
}

int spc_retrieval_head_qk(const spc_shape* s, int32_t hidden, int64_t vocab, const spc_rope* rope, float eps,
                          const int32_t* tokens, const int32_t* positions, const void* emb, const void* gamma,
                          const void* wq, const void* wk, void* q_out, void* dlm_k, void* ws, size_t ws_bytes,
                          void* stream) {
  if (int e = check_shape(s)) return e;
  if (!rope || !tokens || !positions || !emb || !gamma || !wq || !wk || !q_out || !dlm_k)
    return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (s->batch > spc::kFrontMaxBatch)
    return fail(SPC_ERR_UNSUPPORTED, "batch %d > %d for the front end", s->batch, spc::kFrontMaxBatch);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SPC_ERR_UNSUPPORTED, "front end head_dim %d (64 or 128 built)", s->head_dim);
  if (hidden < spc::kFrontSlice || hidden % spc::kFrontSlice != 0 || hidden > spc::kFrontSlice * spc::kFrontMaxSlices)
    return fail(SPC_ERR_INVALID_ARG, "hidden %d must be a multiple of %d, at most %d", hidden, spc::kFrontSlice,
                spc::kFrontSlice * spc::kFrontMaxSlices);
  if (vocab < 1) return fail(SPC_ERR_INVALID_ARG, "vocab must be >= 1");
  if (!(eps >= 0.f)) return fail(SPC_ERR_INVALID_ARG, "eps must be >= 0");
  if (!(rope->base > 1.f) || !(rope->factor > 0.f) || rope->orig_max_pos < 1)
    return fail(SPC_ERR_INVALID_ARG, "rope: base > 1, factor > 0 and orig_max_pos >= 1 required");
  if (rope->factor > 1.f && !(rope->beta_fast > rope->beta_slow))
    return fail(SPC_ERR_INVALID_ARG, "rope: beta_fast must exceed beta_slow");
  if (!aligned16(wq) || !aligned16(wk) || !aligned4(emb) || !aligned4(gamma) || !aligned16(q_out) ||
      !aligned16(dlm_k))
    return fail(SPC_ERR_INVALID_ARG, "wq, wk, q_out and dlm_k must be 16-byte aligned (emb, gamma 4-byte)");
  const size_t need = spc::front_ws_bytes(*s);
  if (ws_bytes < need || !ws)
    return fail(SPC_ERR_WORKSPACE, "front end needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(SPC_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const hipError_t e = spc::launch_front(*s, hidden, vocab, *rope, eps, tokens, positions, emb, gamma, wq, wk, q_out,
                                         dlm_k, ws, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "retrieval head front end launch");
}

int spc_offload_thresholds(const spc_mem_model* m, int32_t* threshold) {
  if (!m || !threshold) return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (m->gpu_bytes < 0 || m->fixed_bytes < 0 || m->token_bytes < 0 || m->n_layers < 1 || m->batch < 1 ||
      m->n_kv_heads < 1 || m->head_dim < 0 || m->v_dim < 0 || m->budget < 0 || m->elem_bytes < 1)
    return fail(SPC_ERR_INVALID_ARG, "memory model sizes must be >= 0 (layers, batch, heads, element bytes >= 1)");
  // exact integer arithmetic in 128 bits: bytes(L, c) = A_c + L * S_c
  const __int128 layer_token = (__int128)m->batch * m->n_kv_heads * (m->head_dim + m->v_dim) * m->elem_bytes;
  const __int128 M = m->gpu_bytes;
  const int64_t kMax = 2147483647;
  for (int c = 0; c <= m->n_layers; ++c) {
    const __int128 A = (__int128)m->fixed_bytes + (__int128)c * m->budget * layer_token;
    const __int128 S = (__int128)m->token_bytes + (__int128)(m->n_layers - c) * layer_token;
    if (A > M) {
      threshold[c] = 0;
    } else if (S == 0) {
      threshold[c] = (int32_t)kMax;
    } else {
      const __int128 last_fit = (M - A) / S;           // the largest L with A + L S <= M
      threshold[c] = last_fit >= kMax - 1 ? (int32_t)kMax : (int32_t)(last_fit + 1);
    }
  }
  return ok();
}

int spc_elastic_plan_lag1(const spc_shape* s, int32_t sel_budget, const int32_t* sel_cur, const int32_t* cur_count,
                          const int32_t* sel_next, const int32_t* next_count, int32_t* slot_pos,
                          uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                          int32_t* attend_rows, int32_t* attend_count, void* stream) {
  if (int e = check_shape(s)) return e;
  if (!sel_cur || !cur_count || !sel_next || !next_count || !slot_pos || !resident_bm || !load_pos || !load_slot ||
      !load_count || !attend_rows || !attend_count)
    return fail(SPC_ERR_INVALID_ARG, "NULL argument");
  if (sel_budget < 1 || (int64_t)s->budget < 2 * (int64_t)sel_budget)
    return fail(SPC_ERR_INVALID_ARG, "pool (shape budget %d) must hold two selections of %d", s->budget, sel_budget);
  if (s->budget > spc::kPlanMaxBudget)
    return fail(SPC_ERR_UNSUPPORTED, "pool %d exceeds the plan kernel's %d", s->budget, spc::kPlanMaxBudget);
  if (3 * sel_budget + 2 * s->budget > spc::kPlanLag1MaxWords)
    return fail(SPC_ERR_UNSUPPORTED, "pool %d and selections of %d exceed the plan kernel's LDS", s->budget,
                sel_budget);
  const hipError_t e = spc::launch_plan_lag1(*s, sel_budget, sel_cur, cur_count, sel_next, next_count, slot_pos,
                                             resident_bm, load_pos, load_slot, load_count, attend_rows, attend_count,
                                             as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "pipelined elastic plan launch");
}

int spc_mla_expand(const spc_shape* s, int32_t nope_dim, int32_t v_head_dim, const void* latent, const void* w_uk,
                   const void* w_uv, const void* q_nope, const void* q_rope, const int32_t* load_pos,
                   const int32_t* load_slot, const int32_t* load_count, void* kv_exp, void* q_exp, void* stream) {
  if (int e = check_mla(s)) return e;
  if (nope_dim != spc::kMlaExpandDims || v_head_dim != spc::kMlaExpandDims)
    return fail(SPC_ERR_UNSUPPORTED, "literal expansion supports nope and value head dims of %d (got %d, %d)",
                spc::kMlaExpandDims, nope_dim, v_head_dim);
  if (s->n_groups != s->n_q_heads)
    return fail(SPC_ERR_INVALID_ARG, "literal expansion needs one selection group per head");
  if (!latent || !w_uk || !w_uv || !load_pos || !load_slot || !load_count || !kv_exp)
    return fail(SPC_ERR_INVALID_ARG, "NULL latent, weights, load lists or kv_exp");
  const bool with_q = q_exp != nullptr;
  if (with_q != (q_nope != nullptr) || with_q != (q_rope != nullptr))
    return fail(SPC_ERR_INVALID_ARG, "q_nope, q_rope and q_exp must be all given or all NULL");
  if (!aligned16(latent) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(kv_exp))
    return fail(SPC_ERR_INVALID_ARG, "latent, weights and kv_exp must be 16-byte aligned");
  if (!aligned4(load_pos) || !aligned4(load_slot) || !aligned4(load_count))
    return fail(SPC_ERR_INVALID_ARG, "misaligned load lists");
  if (with_q && ((reinterpret_cast<uintptr_t>(q_nope) | reinterpret_cast<uintptr_t>(q_rope) |
                  reinterpret_cast<uintptr_t>(q_exp)) & 1u))
    return fail(SPC_ERR_INVALID_ARG, "misaligned bf16 query buffers");
  const hipError_t e = spc::launch_mla_expand(*s, latent, w_uk, w_uv, q_nope, q_rope, load_pos, load_slot,
                                              load_count, kv_exp, q_exp, as_stream(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "MLA literal expansion launch");
}

}  // extern "C"
