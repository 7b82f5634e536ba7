// Stage 3 - elastic loading: plan (set difference, in-place slot reuse) and copy.
//
// The SpeContext blog's section 4 loop takes the positions to load as the new
// selection minus the resident ones and prefetches only those rows; its section 6
// worked example ({1,8,21,35} -> {1,8,21,50}) loads only 50, into the place of
// 35; the paper summary's section 5.4 keeps the budget fixed and loads in place.
//
// plan_kernel  one workgroup (1024 threads) per (b, g).  A slot is kept iff its
//   position is in S (binary search in the ascending S held in LDS); a
//   position of S is loaded iff its bit in the resident bitmap is clear.  Two
//   ordered compactions (block scans over contiguous ranges) give the freed
//   slots and the positions to load, both ascending; the i-th position goes to
//   the i-th freed slot.  Slot map and bitmap are then updated in place.
// plan_bm_kernel  the same where a bitmap of S fits LDS (below): bit tests instead of
//   the binary search, and the resident bitmap rewritten from it.
// plan_lag1_kernel  the same for the pipelined loop (see below).
// copy_kernel  a grid-stride gather over (layer, KV head of the group, instance,
//   entry, 16-byte vector): every KV head of a selection group takes the group's
//   load lists; every lane reads 16 bytes of a K||V row straight from pinned,
//   device-mapped host memory over the host link and writes them into the
//   row's slot in HBM.  Consecutive lanes cover consecutive bytes of a row, so
//   each wave reads whole rows; each lane keeps several reads in flight.
#include <cstdlib>

#include "spc_common.h"
#include "spc_launch.h"
#include "spc_plan.h"

namespace spc {

namespace {

__device__ __forceinline__ bool sorted_contains(const int32_t* a, int n, int32_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo < n && a[lo] == v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ sel_idx,
                                                            const int32_t* __restrict__ sel_count,
                                                            int32_t* __restrict__ slot_pos,
                                                            uint32_t* __restrict__ resident_bm,
                                                            int32_t* __restrict__ load_pos,
                                                            int32_t* __restrict__ load_slot,
                                                            int32_t* __restrict__ load_count, int K, int bm_words) {
  __shared__ int32_t sS[kPlanMaxBudget];   // the new selection, ascending
  __shared__ int32_t sL[kPlanMaxBudget];   // positions to load, ascending
  __shared__ int32_t sF[kPlanMaxBudget];   // freed slots, ascending
  __shared__ int32_t sP[kPlanMaxBudget];   // slot map before the step
  __shared__ uint32_t scan_smem[16];

  const int inst = blockIdx.x;
  const int tid = threadIdx.x;
  int c = sel_count[inst];
  c = c < 0 ? 0 : (c > K ? K : c);
  const int32_t* S = sel_idx + (size_t)inst * K;
  int32_t* sp = slot_pos + (size_t)inst * K;
  uint32_t* bm = resident_bm + (size_t)inst * bm_words;

  for (int i = tid; i < c; i += kPlanThreads) sS[i] = S[i];
  for (int x = tid; x < K; x += kPlanThreads) sP[x] = sp[x];
  __syncthreads();

  // freed slots: empty, or holding a position that left the selection
  const int Cx = (K + kPlanThreads - 1) / kPlanThreads;
  const int x0 = min(tid * Cx, K), x1 = min(x0 + Cx, K);
  uint32_t fmask = 0u, nf_loc = 0u;
  for (int x = x0; x < x1; ++x) {
    const int32_t pos = sP[x];
    const bool keep = pos >= 0 && sorted_contains(sS, c, pos);
    if (!keep) { fmask |= 1u << (x - x0); ++nf_loc; }
  }
  // positions of S not resident
  const int Ci = (c + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(tid * Ci, c), i1 = min(i0 + Ci, c);
  uint32_t lmask = 0u, nl_loc = 0u;
  const int32_t pos_end = bm_words * 32;     // positions outside [0, pos_end) are never loaded
  for (int i = i0; i < i1; ++i) {
    const int32_t j = sS[i];
    if (j < 0 || j >= pos_end) continue;
    const bool resident = (bm[j >> 5] >> (j & 31)) & 1u;
    if (!resident) { lmask |= 1u << (i - i0); ++nl_loc; }
  }
  uint32_t nf, nl;
  uint32_t fo = block_excl_scan(nf_loc, scan_smem, nf);
  uint32_t lo = block_excl_scan(nl_loc, scan_smem, nl);
  for (int x = x0; x < x1; ++x)
    if (fmask >> (x - x0) & 1u) sF[fo++] = x;
  for (int i = i0; i < i1; ++i)
    if (lmask >> (i - i0) & 1u) sL[lo++] = sS[i];
  __syncthreads();

  // apply: the i-th position to load goes to the i-th freed slot; the rest empty
  for (int i = tid; i < (int)nf; i += kPlanThreads) {
    const int x = sF[i];
    const int32_t old = sP[x];
    if (old >= 0 && old < pos_end) atomicAnd(&bm[old >> 5], ~(1u << (old & 31)));
    if (i < (int)nl) {
      const int32_t pos = sL[i];
      sp[x] = pos;
      atomicOr(&bm[pos >> 5], 1u << (pos & 31));
    } else {
      sp[x] = -1;
    }
  }
  int32_t* lp = load_pos + (size_t)inst * K;
  int32_t* ls = load_slot + (size_t)inst * K;
  for (int i = tid; i < K; i += kPlanThreads) {
    const bool v = i < (int)nl;
    lp[i] = v ? sL[i] : -1;
    ls[i] = v ? sF[i] : -1;
  }
  if (tid == 0) load_count[inst] = (int32_t)nl;
}

// The plan when a bitmap of the new selection fits LDS (the common case): a slot is
// kept iff its position's bit is set (one LDS read instead of a binary search), and
// since every position of S is resident after the step, the resident bitmap is
// rewritten whole from that bitmap (coalesced stores, no atomics).  Slot map entries
// and selection entries are read into registers (CPT contiguous ones per thread);
// one block scan of packed 16-bit counts orders both compactions (plan_bitmap).
template <int CPT>
__global__ __launch_bounds__(kPlanThreads) void plan_bm_kernel(const int32_t* __restrict__ sel_idx,
                                                               const int32_t* __restrict__ sel_count,
                                                               int32_t* __restrict__ slot_pos,
                                                               uint32_t* __restrict__ resident_bm,
                                                               int32_t* __restrict__ load_pos,
                                                               int32_t* __restrict__ load_slot,
                                                               int32_t* __restrict__ load_count, int K, int bm_words) {
  extern __shared__ int32_t lds[];
  int32_t* sL = lds;                                       // positions to load, ascending [K]
  int32_t* sF = sL + K;                                    // freed slots, ascending [K]
  uint32_t* sB = reinterpret_cast<uint32_t*>(sF + K);      // bitmap of S [bm_words]
  __shared__ uint32_t scan_smem[16];
  const int inst = blockIdx.x;
  int c = sel_count[inst];
  c = c < 0 ? 0 : (c > K ? K : c);
  plan_bitmap<CPT>(sel_idx + (size_t)inst * K, c, slot_pos + (size_t)inst * K, resident_bm + (size_t)inst * bm_words,
                   load_pos + (size_t)inst * K, load_slot + (size_t)inst * K, load_count + inst, K, bm_words, sL, sF,
                   sB, scan_smem);
}

// The plan of the pipelined loop: the target model attends over the current
// selection C (loaded in the previous step) while the next selection N is loaded, so a
// slot of the pool (P >= 2 K slots) is reusable only if its position is in
// neither; the new positions are N - resident.  Also writes the ascending slots
// that hold C (the rows the attention of this step gathers).  Same block scans
// and in-place update as plan_kernel.
__global__ __launch_bounds__(kPlanThreads) void plan_lag1_kernel(
    const int32_t* __restrict__ sel_cur, const int32_t* __restrict__ cur_count,
    const int32_t* __restrict__ sel_next, const int32_t* __restrict__ next_count, int32_t* __restrict__ slot_pos,
    uint32_t* __restrict__ resident_bm, int32_t* __restrict__ load_pos, int32_t* __restrict__ load_slot,
    int32_t* __restrict__ load_count, int32_t* __restrict__ attend_rows, int32_t* __restrict__ attend_count, int Ks,
    int P, int bm_words) {
  extern __shared__ int32_t lds[];
  int32_t* sN = lds;              // next selection [Ks], ascending
  int32_t* sC = sN + Ks;          // current selection [Ks], ascending
  int32_t* sL = sC + Ks;          // positions to load [Ks]
  int32_t* sF = sL + Ks;          // reusable slots [P]
  int32_t* sP = sF + P;           // the pool's slot map [P]
  __shared__ uint32_t scan_smem[16];

  const int inst = blockIdx.x;
  const int tid = threadIdx.x;
  int cn = next_count[inst], cc = cur_count[inst];
  cn = cn < 0 ? 0 : (cn > Ks ? Ks : cn);
  cc = cc < 0 ? 0 : (cc > Ks ? Ks : cc);
  int32_t* sp = slot_pos + (size_t)inst * P;
  uint32_t* bm = resident_bm + (size_t)inst * bm_words;
  for (int i = tid; i < cn; i += kPlanThreads) sN[i] = sel_next[(size_t)inst * Ks + i];
  for (int i = tid; i < cc; i += kPlanThreads) sC[i] = sel_cur[(size_t)inst * Ks + i];
  for (int x = tid; x < P; x += kPlanThreads) sP[x] = sp[x];
  __syncthreads();

  const int Cx = (P + kPlanThreads - 1) / kPlanThreads;
  const int x0 = min(tid * Cx, P), x1 = min(x0 + Cx, P);
  uint32_t fmask = 0u, nf_loc = 0u;
  for (int x = x0; x < x1; ++x) {
    const int32_t pos = sP[x];
    const bool keep = pos >= 0 && (sorted_contains(sN, cn, pos) || sorted_contains(sC, cc, pos));
    if (!keep) { fmask |= 1u << (x - x0); ++nf_loc; }
  }
  const int Ci = (cn + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(tid * Ci, cn), i1 = min(i0 + Ci, cn);
  uint32_t lmask = 0u, nl_loc = 0u;
  const int32_t pos_end = bm_words * 32;
  for (int i = i0; i < i1; ++i) {
    const int32_t j = sN[i];
    if (j < 0 || j >= pos_end) continue;
    if (!((bm[j >> 5] >> (j & 31)) & 1u)) { lmask |= 1u << (i - i0); ++nl_loc; }
  }
  uint32_t nf, nl;
  uint32_t fo = block_excl_scan(nf_loc, scan_smem, nf);
  uint32_t lo = block_excl_scan(nl_loc, scan_smem, nl);
  for (int x = x0; x < x1; ++x)
    if (fmask >> (x - x0) & 1u) sF[fo++] = x;
  for (int i = i0; i < i1; ++i)
    if (lmask >> (i - i0) & 1u) sL[lo++] = sN[i];
  __syncthreads();
  // the host guarantees P >= 2 Ks, so nl <= nf
  for (int i = tid; i < (int)nf; i += kPlanThreads) {
    const int x = sF[i];
    const int32_t old = sP[x];
    if (old >= 0 && old < pos_end) atomicAnd(&bm[old >> 5], ~(1u << (old & 31)));
    int32_t nw = -1;
    if (i < (int)nl) {
      nw = sL[i];
      atomicOr(&bm[nw >> 5], 1u << (nw & 31));
    }
    sp[x] = nw;
    sP[x] = nw;
  }
  int32_t* lp = load_pos + (size_t)inst * P;
  int32_t* ls = load_slot + (size_t)inst * P;
  for (int i = tid; i < P; i += kPlanThreads) {
    const bool v = i < (int)nl;
    lp[i] = v ? sL[i] : -1;
    ls[i] = v ? sF[i] : -1;
  }
  if (tid == 0) load_count[inst] = (int32_t)nl;
  __syncthreads();
  // the slots holding the current selection, ascending
  uint32_t amask = 0u, na_loc = 0u;
  for (int x = x0; x < x1; ++x) {
    const int32_t pos = sP[x];
    if (pos >= 0 && sorted_contains(sC, cc, pos)) { amask |= 1u << (x - x0); ++na_loc; }
  }
  uint32_t na;
  uint32_t ao = block_excl_scan(na_loc, scan_smem, na);
  int32_t* ar = attend_rows + (size_t)inst * Ks;
  for (int x = x0; x < x1; ++x)
    if ((amask >> (x - x0) & 1u) && ao < (uint32_t)Ks) ar[ao++] = x;
  for (int i = (int)na + tid; i < Ks; i += kPlanThreads) ar[i] = -1;
  if (tid == 0) attend_count[inst] = (int32_t)(na < (uint32_t)Ks ? na : (uint32_t)Ks);
}

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;

struct ByteLayout {
  int64_t b, layer, head, row, kv;
};

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const int32_t* __restrict__ load_pos,
                                                            const int32_t* __restrict__ load_slot,
                                                            const int32_t* __restrict__ load_count,
                                                            const char* __restrict__ host, ByteLayout hl,
                                                            char* __restrict__ dev, ByteLayout dl, int n_inst,
                                                            int n_groups, int hpg, int K, int max_len,
                                                            int layer_begin, int n_lay, int vk, int vrow) {
  __shared__ uint32_t pre[kCopyMaxInstances + 1];
  __shared__ uint32_t scan_smem[16];
  // prefix sums of the load counts over instances
  uint32_t carry = 0u;
  for (int base = 0; base < n_inst; base += kCopyThreads) {
    const int i = base + threadIdx.x;
    uint32_t v = 0u;
    if (i < n_inst) {
      const int32_t cnt = load_count[i];
      v = cnt < 0 ? 0u : (cnt > K ? (uint32_t)K : (uint32_t)cnt);
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan(v, scan_smem, tot);
    if (i < n_inst) pre[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[n_inst] = carry;
  __syncthreads();
  // 32-bit vector ids: the host checks n_inst * hpg * K * n_lay * vrow < 2^32
  const uint32_t total = carry;
  const uint32_t per_layer = total * (uint32_t)hpg;       // (KV head of the group, entry) pairs
  const uint32_t nvec = per_layer * (uint32_t)n_lay * (uint32_t)vrow;
  const uint32_t stride = gridDim.x * kCopyThreads;

  for (uint32_t v0 = blockIdx.x * kCopyThreads + threadIdx.x; v0 < nvec; v0 += stride * kCopyUnroll) {
    Vec16 buf[kCopyUnroll];
    char* dst[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint32_t vid = v0 + (uint32_t)u * stride;
      dst[u] = nullptr;
      if (vid < nvec) {
        const uint32_t item = vid / (uint32_t)vrow;
        const int v = (int)(vid - item * (uint32_t)vrow);
        const int lo_ = (int)(item / per_layer);
        const uint32_t he = item - (uint32_t)lo_ * per_layer;
        const int hh = (int)(he / total);
        const uint32_t e = he - (uint32_t)hh * total;
        // instance holding entry e: last inst with pre[inst] <= e
        int a = 0, z = n_inst;
        while (z - a > 1) {
          const int mid = (a + z) >> 1;
          if (pre[mid] <= e) a = mid; else z = mid;
        }
        const int inst = a;
        const int i = (int)(e - pre[inst]);
        const int b = inst / n_groups, g = (inst - (inst / n_groups) * n_groups) * hpg + hh;   // KV head
        const int layer = layer_begin + lo_;
        const int32_t pos = load_pos[(size_t)inst * K + i];
        const int32_t slot = load_slot[(size_t)inst * K + i];
        if (pos < 0 || pos >= max_len || slot < 0 || slot >= K) continue;   // malformed entry: skipped
        const int64_t off_h = v < vk ? (int64_t)v * 16 : hl.kv + (int64_t)(v - vk) * 16;
        const int64_t off_d = v < vk ? (int64_t)v * 16 : dl.kv + (int64_t)(v - vk) * 16;
        const char* src = host + b * hl.b + layer * hl.layer + g * hl.head + (int64_t)pos * hl.row + off_h;
        dst[u] = dev + b * dl.b + layer * dl.layer + g * dl.head + (int64_t)slot * dl.row + off_d;
        buf[u] = ld16(src);
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (dst[u]) st16(dst[u], buf[u]);
  }
}

__global__ void reset_kernel(int32_t* __restrict__ slot_pos, uint32_t* __restrict__ bm, int64_t n_slot,
                             int64_t n_words) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slot; i += stride) slot_pos[i] = -1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride) bm[i] = 0u;
}

}  // namespace

hipError_t launch_plan(const spc_shape& s, const int32_t* sel_idx, const int32_t* sel_count, int32_t* slot_pos,
                       uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                       hipStream_t st) {
  const int bm_words = (s.max_len + 31) / 32;
  const dim3 grid(s.batch * s.n_groups);
  const size_t lds = (size_t)(2 * s.budget + bm_words) * sizeof(int32_t);
  const int cpt = (s.budget + kPlanThreads - 1) / kPlanThreads;
  if (lds <= kPlanBmLdsBytes) {
    switch (cpt <= 1 ? 1 : cpt <= 2 ? 2 : cpt <= 4 ? 4 : 8) {
#define SPC_CASE(N)                                                                                           \
  case N:                                                                                                     \
    plan_bm_kernel<N><<<grid, kPlanThreads, lds, st>>>(sel_idx, sel_count, slot_pos, resident_bm, load_pos,   \
                                                       load_slot, load_count, s.budget, bm_words);            \
    break;
      SPC_CASE(1)
      SPC_CASE(2)
      SPC_CASE(4)
      SPC_CASE(8)
#undef SPC_CASE
    }
  } else {
    plan_kernel<<<grid, kPlanThreads, 0, st>>>(sel_idx, sel_count, slot_pos, resident_bm, load_pos, load_slot,
                                               load_count, s.budget, bm_words);
  }
  return hipGetLastError();
}

hipError_t launch_plan_lag1(const spc_shape& s, int sel_budget, const int32_t* sel_cur, const int32_t* cur_count,
                            const int32_t* sel_next, const int32_t* next_count, int32_t* slot_pos,
                            uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                            int32_t* attend_rows, int32_t* attend_count, hipStream_t st) {
  const int bm_words = (s.max_len + 31) / 32;
  const size_t lds = (size_t)(3 * sel_budget + 2 * s.budget) * sizeof(int32_t);
  plan_lag1_kernel<<<dim3(s.batch * s.n_groups), kPlanThreads, lds, st>>>(
      sel_cur, cur_count, sel_next, next_count, slot_pos, resident_bm, load_pos, load_slot, load_count, attend_rows,
      attend_count, sel_budget, s.budget, bm_words);
  return hipGetLastError();
}

hipError_t launch_copy(const spc_shape& s, const int32_t* load_pos, const int32_t* load_slot,
                       const int32_t* load_count, const void* host_dev_ptr, const spc_kv_layout& hl, void* dev_kv,
                       const spc_kv_layout& dl, int layer_begin, int layer_end, hipStream_t st) {
  const int eb = s.dtype == SPC_BF16 ? 2 : 4;
  const int vk = s.head_dim * eb / 16;
  const int vrow = vk + s.v_dim * eb / 16;
  const ByteLayout hb{hl.s_b * eb, hl.s_layer * eb, hl.s_head * eb, hl.s_row * eb, hl.s_kv * eb};
  const ByteLayout db{dl.s_b * eb, dl.s_layer * eb, dl.s_head * eb, dl.s_row * eb, dl.s_kv * eb};
  static const int blocks = [] {
    const char* e = getenv("SPC_COPY_BLOCKS");
    const int v = e ? atoi(e) : 0;
    return v > 0 && v <= 65535 ? v : kCopyBlocksDefault;
  }();
  copy_kernel<<<dim3(blocks), kCopyThreads, 0, st>>>(
      load_pos, load_slot, load_count, static_cast<const char*>(host_dev_ptr), hb, static_cast<char*>(dev_kv), db,
      s.batch * s.n_groups, s.n_groups, s.n_kv_heads / s.n_groups, s.budget, s.max_len, layer_begin,
      layer_end - layer_begin, vk, vrow);
  return hipGetLastError();
}

hipError_t launch_reset(const spc_shape& s, int batch_begin, int batch_end, int32_t* slot_pos,
                        uint32_t* resident_bm, hipStream_t st) {
  const int64_t bm_words = (s.max_len + 31) / 32;
  const int64_t per_b_slots = (int64_t)s.n_groups * s.budget;
  const int64_t per_b_words = (int64_t)s.n_groups * bm_words;
  const int64_t nb = batch_end - batch_begin;
  reset_kernel<<<dim3(256), 256, 0, st>>>(slot_pos + batch_begin * per_b_slots,
                                          resident_bm + batch_begin * per_b_words, nb * per_b_slots,
                                          nb * per_b_words);
  return hipGetLastError();
}

}  // namespace spc
