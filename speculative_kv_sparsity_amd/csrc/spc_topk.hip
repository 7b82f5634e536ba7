// Stage 2 - GQA group max and per-group Top-K.
//
//   v[b][g][j] = max over the query heads i of group g of probs[b][i][j]
//     (SpeContext blog section 5 / paper summary section 4.3: element-wise max
//      over a GQA group; MQA is one group; MHA selects per head)
//   S[b][g]    = the first min(K, n) positions by (v desc, j asc), written ascending
//     (blog section 2: at most K positions per head per round; the lower index
//      wins a tie)
//
// Each fp32 value becomes an order-preserving uint32 key (-0 and +0 are one
// value); the K-th largest key T is found by radix select over 8 + 12 + 12 bits,
// or, for raw logits staged in LDS, 12 + 12 + 8 bits (a 12-bit first digit --
// sign, exponent and three mantissa bits -- spreads logits over many bins, so
// the first histogram's LDS atomics rarely collide).
//
// The scores may also arrive in log-domain form (logits plus each head's
// per-tile max and sum of exp): the group max is then taken over
// logit - log-sum-exp and exponentiated, which is the group max of the
// probabilities (exp is increasing), so the probabilities need never be
// written.  With one head per group the logits are ranked as they are.
//
// topk_keys_kernel    many workgroups per (b, g), kKeyChunk positions each:
//   takes the group max while reading the heads' rows once, writes the keys to
//   the workspace and the chunk's histogram of the top 8 key bits.  With one
//   head per group (MHA, MLA) the keys are not written: the select kernel maps
//   the probabilities to keys as it loads them.
// topk_select_kernel  one 1024-thread workgroup per (b, g): sums the chunk
//   histograms (first digit; with one head per group and rows that fit LDS the
//   select counts it from its staged keys and no keys pass runs), runs the two
//   remaining passes with LDS
//   histograms over the keys that still match the prefix, and compacts every j
//   with key > T plus the lowest-index `need` ones with key == T, ascending,
//   with two block scans over per-thread contiguous index ranges.  For
//   n <= 32768 the keys are staged in LDS (one pad word per 32 keys keeps the
//   contiguous-range sweeps free of bank conflicts); longer rows are read from
//   the workspace (L2) in every pass.  The LDS form can end with the elastic
//   plan of its instance (spc_plan.h), so the selection is never re-read.
#include "spc_common.h"
#include "spc_launch.h"
#include "spc_plan.h"

namespace spc {

namespace {

constexpr int kKeyThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kBins1 = 256;                       // first digit: key bits 31..24
static_assert(kSelThreads == kPlanThreads, "the fused plan runs on the select's workgroup");

// Order-preserving map from fp32 bits to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);   // -0 + 0 = +0: the two zeros are one value (a tie)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Keys of 4 loaded words: the words themselves, or (RAW) the keys of 4 fp32 values.
template <bool RAW>
__device__ __forceinline__ uint4 to_keys(uint4 w) {
  if (!RAW) return w;
  return make_uint4(order_key(__uint_as_float(w.x)), order_key(__uint_as_float(w.y)), order_key(__uint_as_float(w.z)),
                    order_key(__uint_as_float(w.w)));
}

// Online merge of two (max, sum exp(x - max)) pairs.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __expf(m - M)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - M));
  m = M;
}

// LOGITS: `scores` are logits and, with several heads per group, `stats` holds
// each head's per-tile (max, sum exp) [B*Hq][ntiles] over tiles of `tile`
// positions.  The group max is then taken over l - lse of every head and keyed
// as exp of it: exp is increasing, so that is the group max of the
// probabilities exp(l - lse), formed here instead of stored.  (Keying the
// log-probabilities themselves would rank the same, but they crowd into one or
// two values of the first radix digit - sign and high exponent bits - and the
// select would then carry the whole row as candidates.)
template <bool LOGITS>
__global__ __launch_bounds__(kKeyThreads) void topk_keys_kernel(const float* __restrict__ scores,
                                                                const float2* __restrict__ stats,
                                                                const int32_t* __restrict__ lengths,
                                                                uint32_t* __restrict__ keys,
                                                                uint32_t* __restrict__ chist, int Hq, int n_groups,
                                                                int max_len, int budget, int nchunk, int ntiles,
                                                                int tile) {
  const int inst = blockIdx.y;
  const int c = blockIdx.x;
  const int b = inst / n_groups;
  const int g = inst - b * n_groups;
  const int n = clamp_len(lengths, b, max_len);
  const int j0 = c * kKeyChunk;
  if (n <= budget || j0 >= n) return;
  const int j1 = min(j0 + kKeyChunk, n);
  const int Gq = Hq / n_groups;
  const float* pb = scores + ((size_t)b * Hq + (size_t)g * Gq) * max_len;
  uint32_t* kout = keys + (size_t)inst * max_len;
  __shared__ uint32_t h[kBins1];
  __shared__ float s_lse[kMaxGroupHeads];
  h[threadIdx.x] = 0u;
  constexpr int kPer = kKeyChunk / kKeyThreads;       // positions per thread
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + threadIdx.x + u * kKeyThreads;
    v[u] = j < j1 ? pb[j] : 0.f;
  }
  // the other heads' rows of up to kMaxPre heads, loaded now so that their latency overlaps the
  // tile-pair loads of the log-sum-exp below
  constexpr int kMaxPre = 8;
  float w[kMaxPre - 1][kPer];
#pragma unroll
  for (int hh = 1; hh < kMaxPre; ++hh)
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = j0 + threadIdx.x + u * kKeyThreads;
      w[hh - 1][u] = hh < Gq && j < j1 ? pb[(size_t)hh * max_len + j] : 0.f;
    }
  const bool lse = LOGITS && Gq > 1;
  if (lse) {
    // log-sum-exp of every head of the group from its tile pairs (one wave per head)
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nt = (n + tile - 1) / tile;
    for (int hh = wid; hh < Gq; hh += kKeyThreads / 64) {
      const float2* st = stats + ((size_t)b * Hq + (size_t)g * Gq + hh) * ntiles;
      float m = -INFINITY, sm = 0.f;
      for (int t0 = 0; t0 < nt; t0 += 4 * 64) {
        float2 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = t0 + lane + 64 * u;
          x[u] = t < nt ? st[t] : make_float2(-INFINITY, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) merge_ms(m, sm, x[u].x, x[u].y);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const float s2 = __shfl_xor(sm, o, kWave);
        merge_ms(m, sm, m2, s2);
      }
      if (lane == 0) s_lse[hh] = m + __logf(sm);
    }
  }
  __syncthreads();
  if (lse) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u] -= s_lse[0];
  }
#pragma unroll
  for (int hh = 1; hh < kMaxPre; ++hh) {
    if (hh >= Gq) break;
    const float off = lse ? s_lse[hh] : 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = j0 + threadIdx.x + u * kKeyThreads;
      if (j < j1) v[u] = fmaxf(v[u], w[hh - 1][u] - off);
    }
  }
  for (int hh = kMaxPre; hh < Gq; ++hh) {             // groups of more than kMaxPre heads
    const float* ph = pb + (size_t)hh * max_len;
    const float off = lse ? s_lse[hh] : 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = j0 + threadIdx.x + u * kKeyThreads;
      if (j < j1) v[u] = fmaxf(v[u], ph[j] - off);
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + threadIdx.x + u * kKeyThreads;
    if (j < j1) {
      const uint32_t key = order_key(lse ? __expf(v[u]) : v[u]);
      if (Gq > 1) kout[j] = key;      // one head per group: the select kernel keys the scores itself
      atomicAdd(&h[key >> 24], 1u);
    }
  }
  __syncthreads();
  chist[((size_t)inst * nchunk + c) * kBins1 + threadIdx.x] = h[threadIdx.x];
}

// Find the bin (counted from the top) holding the need-th largest key.
// hist[0..nb) are the counts; bins are owned top-down by consecutive threads.
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int need, uint32_t* scan_smem,
                                         uint32_t* bcast) {
  const int tid = threadIdx.x;
  const int bpt = nb >= kSelThreads ? nb / kSelThreads : 1;
  const int hi = nb - tid * bpt;
  uint32_t local = 0u;
  if (hi > 0)
    for (int i = 0; i < bpt; ++i) local += hist[hi - 1 - i];
  uint32_t total;
  const uint32_t above = block_excl_scan(local, scan_smem, total);
  if (hi > 0 && (int)above < need && need <= (int)(above + local)) {
    uint32_t cum = above;
    for (int i = 0; i < bpt; ++i) {
      const int bin = hi - 1 - i;
      if ((int)(cum + hist[bin]) >= need) {
        bcast[0] = (uint32_t)bin;
        bcast[1] = cum;
        break;
      }
      cum += hist[bin];
    }
  }
  __syncthreads();
}

// LDS layout of staged keys: 4-key vector v lives in vector slot v ^ ((v >> 3) & 7),
// so 16-byte reads are free of bank conflicts both when lanes take consecutive
// vectors and when each lane walks its own contiguous run of 8 vectors.
__device__ __forceinline__ int vslot(int v) { return v ^ ((v >> 3) & 7); }

// Rows longer than the LDS stage (streamed): radix passes 2 and 3 over the keys
// read from the workspace or the scores (L2) in every pass, plus the ordered
// compaction.  key_vec(v) returns keys 4v..4v+3 (entries >= n are ignored).
template <bool RAW>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const uint32_t* __restrict__ keys,
                                                                  const uint32_t* __restrict__ chist,
                                                                  const int32_t* __restrict__ lengths,
                                                                  int32_t* __restrict__ sel_idx,
                                                                  int32_t* __restrict__ sel_count, int n_groups,
                                                                  int max_len, int budget, int nchunk) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t scan_smem[16];
  __shared__ uint32_t bcast[2];

  const int inst = blockIdx.x;
  const int b = inst / n_groups;
  const int n = clamp_len(lengths, b, max_len);
  const int K = budget;
  const int tid = threadIdx.x;
  int32_t* out = sel_idx + (size_t)inst * K;
  if (n <= K) {
    for (int i = tid; i < K; i += kSelThreads) out[i] = i < n ? i : -1;
    if (tid == 0) sel_count[inst] = n;
    return;
  }
  const uint32_t* kin = keys + (size_t)inst * max_len;
  const int nv = (n + 3) / 4;                          // key vectors (the last may be partial)
  const bool aligned = (max_len % 4) == 0;             // rows of the key buffer start 16-byte aligned
  auto key_vec = [&](int v) -> uint4 {
    const int j = 4 * v;
    if (aligned && j + 3 < n) return to_keys<RAW>(reinterpret_cast<const uint4*>(kin)[v]);
    return to_keys<RAW>(
        make_uint4(kin[j], j + 1 < n ? kin[j + 1] : 0u, j + 2 < n ? kin[j + 2] : 0u, j + 3 < n ? kin[j + 3] : 0u));
  };

  // first digit from the chunk histograms: thread t sums bin t % 256 over the
  // chunks c = t / 256 (mod 4), eight independent loads at a time
  const int nch = (n + kKeyChunk - 1) / kKeyChunk;
  if (tid < kBins1) hist[tid] = 0u;
  __syncthreads();
  {
    const int bin = tid & (kBins1 - 1), c0 = tid >> 8;
    const uint32_t* ch = chist + (size_t)inst * nchunk * kBins1 + bin;
    uint32_t s = 0u;
    for (int cb = c0; cb < nch; cb += 32) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = cb + 4 * u;
        v[u] = c < nch ? ch[(size_t)c * kBins1] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    atomicAdd(&hist[bin], s);
  }
  __syncthreads();

  int need = K;
  find_bin(hist, kBins1, need, scan_smem, bcast);
  uint32_t prefix = bcast[0] << 24;
  uint32_t pmask = 0xFF000000u;
  need -= (int)bcast[1];
  bool whole = (int)hist[bcast[0]] == need;       // every key of the bin is taken: T is resolved
  __syncthreads();
#pragma unroll 1
  for (int pass = 0; pass < 2 && !whole; ++pass) {
    const int shift = pass == 0 ? 12 : 0;
    for (int i = tid; i < 4096; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int v = tid; v < nv; v += kSelThreads) {
      const uint4 kv = key_vec(v);
      const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * v + e < n && (k4[e] & pmask) == prefix) atomicAdd(&hist[(k4[e] >> shift) & 4095u], 1u);
    }
    __syncthreads();
    find_bin(hist, 4096, need, scan_smem, bcast);
    prefix |= bcast[0] << shift;
    pmask |= 4095u << shift;
    need -= (int)bcast[1];
    whole = (int)hist[bcast[0]] == need;
    __syncthreads();
  }
  // Selected: masked key > prefix, plus the first `need` (in index order) with
  // masked key == prefix.  When all 32 bits are resolved those keys are equal
  // and the lower indices win; otherwise every one of them is taken.
  // Thread t owns the contiguous vectors [t*C4, t*C4 + C4); flags are kept as
  // bit masks of 32 keys so the keys are swept once.
  const int C4 = (nv + kSelThreads - 1) / kSelThreads;
  const int v0 = min(tid * C4, nv), v1 = min(v0 + C4, nv);
  uint32_t gt = 0u, eq = 0u;
  int ee = 0, eq_before = 0, gt_before = 0, take_eq = 0;
  uint32_t tot;
  if (C4 <= 8) {
    uint32_t gtm = 0u, eqm = 0u;
    for (int v = v0; v < v1; ++v) {
      const uint4 kv = key_vec(v);
      const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bit = 4 * (v - v0) + e;
        const uint32_t mk = k4[e] & pmask;
        const bool valid = 4 * v + e < n;
        gtm |= (uint32_t)(valid && mk > prefix) << bit;
        eqm |= (uint32_t)(valid && mk == prefix) << bit;
      }
    }
    gt = __popc(gtm);
    eq = __popc(eqm);
    if (n < 65536) {
      const uint32_t before = block_excl_scan((eq << 16) | gt, scan_smem, tot);
      eq_before = (int)(before >> 16);
      gt_before = (int)(before & 0xFFFFu);
    } else {
      eq_before = (int)block_excl_scan(eq, scan_smem, tot);
      gt_before = (int)block_excl_scan(gt, scan_smem, tot);
    }
    take_eq = max(0, min((int)eq, need - eq_before));
    // drop the equal keys beyond take_eq, then write the set bits in index order
    uint32_t keep_eq = eqm;
    for (int drop = (int)eq - take_eq; drop > 0; --drop) keep_eq &= ~(0x80000000u >> __clz(keep_eq));
    uint32_t m = gtm | keep_eq;
    int o = gt_before + min(eq_before, need);
    const int jbase = 4 * v0;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (o < K) out[o++] = jbase + bit;
    }
  } else {
    for (int v = v0; v < v1; ++v) {
      const uint4 kv = key_vec(v);
      const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t mk = k4[e] & pmask;
        const bool valid = 4 * v + e < n;
        gt += valid && mk > prefix;
        eq += valid && mk == prefix;
      }
    }
    eq_before = (int)block_excl_scan(eq, scan_smem, tot);
    gt_before = (int)block_excl_scan(gt, scan_smem, tot);
    take_eq = max(0, min((int)eq, need - eq_before));
    int o = gt_before + min(eq_before, need);
    for (int v = v0; v < v1; ++v) {
      const uint4 kv = key_vec(v);
      const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * v + e;
        if (j >= n) continue;
        const uint32_t mk = k4[e] & pmask;
        bool take = mk > prefix;
        if (mk == prefix) {
          take = ee < take_eq;
          ++ee;
        }
        if (take && o < K) out[o++] = j;
      }
    }
  }
  if (tid == 0) sel_count[inst] = K;
}

// Rows of at most 32768 keys (staged in LDS, 32 keys per thread).  The kernel's cost is the vector
// instructions its one workgroup issues, so every step past the first sweep touches only the
// candidates (the keys in the threshold's first-digit bin):
//   - the keys are loaded with buffer loads (past the row: zeros, no branch) in strided, coalesced
//     order, keyed, and staged in LDS; thread t then reads its contiguous positions [32t, 32t+32);
//   - one sweep marks, as bit masks, the keys above the threshold's first digit (selected) and
//     those in its bin (candidates), and appends the candidates' positions to an LDS list (one
//     counter add per wave), whose length the first-digit histogram gives in advance;
//   - the second and third digit passes and the final compare run over that list, one entry per
//     thread, and mark the candidates above the threshold and those equal to it (ties) in two LDS
//     bitmaps of the row, word t of which belongs to thread t;
//   - two block scans order the selected keys and the ties (the lowest positions win), and the
//     selection is staged in LDS and written out in coalesced order.
// When the bin holds more candidates than the list, the passes run over each thread's own keys.
//
// With CPT > 0 the kernel also makes the instance's elastic plan: the selection mask of thread t is
// word t of the selection's bitmap, and the plan (plan_words) runs on those words with the keys'
// LDS, no longer read, holding its lists.
struct PlanBufs {
  int32_t* slot_pos;
  uint32_t* resident_bm;
  int32_t* load_pos;
  int32_t* load_slot;
  int32_t* load_count;
  int bm_words;
};

constexpr int kCandList = 3072;      // candidate positions the LDS list holds

// Exclusive scan over the NT-thread block; `smem` holds NT / 64 words, 16-byte aligned.
// Ends with a barrier.
template <int NT = kSelThreads>
__device__ __forceinline__ uint32_t scan_block(uint32_t v, uint32_t* smem, uint32_t& total) {
  constexpr int kWaves = NT / kWave;
  static_assert(kWaves % 4 == 0 && kWaves <= 16, "16-byte reads of wave totals");
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) smem[wid] = incl;
  __syncthreads();
  const uint4* s4 = reinterpret_cast<const uint4*>(smem);
  uint32_t base = 0u, tot = 0u;
#pragma unroll
  for (int q = 0; q < kWaves / 4; ++q) {
    const uint4 x = s4[q];
    const uint32_t a[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      base += 4 * q + e < wid ? a[e] : 0u;
      tot += a[e];
    }
  }
  total = tot;
  __syncthreads();
  return base + incl - v;
}

// find_bin over NB bins with the bin counts held in registers between the scan and the search
// (NT threads).
template <int NB, int NT = kSelThreads>
__device__ __forceinline__ void find_bin_fixed(const uint32_t* hist, int need, uint32_t* scan_smem, uint32_t* bcast) {
  constexpr int BPT = NB >= NT ? NB / NT : 1;
  const int hi = NB - (int)threadIdx.x * BPT;          // this thread's bins: hi-1, hi-2, ... (top down)
  uint32_t h[BPT];
  uint32_t local = 0u;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = hi - 1 - i >= 0 ? hist[hi - 1 - i] : 0u;
    local += h[i];
  }
  uint32_t total;
  const uint32_t above = scan_block<NT>(local, scan_smem, total);
  if ((int)above < need && need <= (int)(above + local)) {   // exactly one thread
    uint32_t cum = above;
    bool found = false;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (!found && (int)(cum + h[i]) >= need) {
        bcast[0] = (uint32_t)(hi - 1 - i);
        bcast[1] = cum;
        found = true;
      }
      cum += h[i];
    }
  }
  __syncthreads();
}

template <bool RAW, int CPT>
__global__ __launch_bounds__(kSelThreads) void topk_select_lds_kernel(const uint32_t* __restrict__ keys,
                                                                      const uint32_t* __restrict__ chist,
                                                                      const int32_t* __restrict__ lengths,
                                                                      int32_t* __restrict__ sel_idx,
                                                                      int32_t* __restrict__ sel_count,
                                                                      int n_groups, int max_len, int budget,
                                                                      int nchunk, PlanBufs pb) {
  __shared__ uint4 skeys[kTopkLdsKeys / 4];
  __shared__ uint32_t hist[4096];
  __shared__ int32_t clist[kCandList];
  __shared__ __align__(16) uint32_t scan_smem[16];
  __shared__ uint32_t bcast[2];
  __shared__ uint32_t ccount;
  constexpr int kVecPerThread = kTopkLdsKeys / 4 / kSelThreads;   // 8 vectors = 32 keys
  constexpr int kKeysPerThread = 4 * kVecPerThread;
  constexpr int kListPerThread = kCandList / kSelThreads;
  static_assert(kCandList % kSelThreads == 0 && 2 * kSelThreads <= 4096, "list passes; bitmaps in the histogram");
  // digits of the order key: raw float32 keys take 12 + 12 + 8 bits (the top 12 bits -- sign,
  // exponent and 3 mantissa bits -- spread logits over many bins, so the first histogram's LDS
  // atomics rarely collide); keys of the keys pass take 8 (its chunk histograms) + 12 + 12
  constexpr int S1 = RAW ? 20 : 24;                // first digit: bits 31..S1
  constexpr int S2 = S1 - 12;                      // second digit: 12 bits S1-1..S2; third: S2-1..0

  const int inst = blockIdx.x;
  const int b = inst / n_groups;
  const int n = clamp_len(lengths, b, max_len);
  const int K = budget;
  const int tid = threadIdx.x;
  int32_t* out = sel_idx + (size_t)inst * K;
  constexpr bool kPlan = CPT > 0;
  constexpr int kP = kPlan ? CPT : 1;
  // the plan's inputs, loaded first so that their latency hides behind the select
  uint32_t oldw[1] = {0u};
  int32_t pos[kP];
  int32_t* sp = pb.slot_pos + (size_t)inst * K;
  uint32_t* bm = pb.resident_bm + (size_t)inst * pb.bm_words;
  if (kPlan) {
    const int Cx = (K + kSelThreads - 1) / kSelThreads;
    const int x0 = min(tid * Cx, K), x1 = min(x0 + Cx, K);
#pragma unroll
    for (int u = 0; u < kP; ++u) pos[u] = x0 + u < x1 ? sp[x0 + u] : -1;
    if (tid < pb.bm_words) oldw[0] = bm[tid];
  }
  auto plan = [&](uint32_t selw) {
    int32_t* sL = reinterpret_cast<int32_t*>(skeys);
    const uint32_t sw[1] = {selw};
    plan_words<kP, 1>(sw, oldw, pos, sp, bm, pb.load_pos + (size_t)inst * K, pb.load_slot + (size_t)inst * K,
                      pb.load_count + inst, K, pb.bm_words, sL + K, sL + 2 * K,
                      reinterpret_cast<uint32_t*>(sL + 3 * K), scan_smem);
  };
  if (n <= K) {
    for (int i = tid; i < K; i += kSelThreads) out[i] = i < n ? i : -1;
    if (tid == 0) sel_count[inst] = n;
    if (kPlan) {
      const int r = n - 32 * tid;                  // this thread's word: positions [32 tid, 32 tid + 32)
      plan(r >= 32 ? 0xFFFFFFFFu : r > 0 ? (1u << r) - 1u : 0u);
    }
    return;
  }
  const uint32_t* kin = keys + (size_t)inst * max_len;
  const int nv = (n + 3) / 4;

  // key loads (strided, coalesced) and the chunk-histogram loads, issued together
  uint4 v[kVecPerThread];
  if ((max_len & 3) == 0) {                        // rows start 16-byte aligned: 16-byte loads
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kin), (short)0,
                                                                       nv * 16, kBufferRsrcWord3);
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const Vec16 x = ld16_buffer(r, (uint32_t)(tid + u * kSelThreads) * 16u);
      v[u] = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
    }
  } else {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kin), (short)0, n * 4,
                                                                       kBufferRsrcWord3);
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int o = (tid + u * kSelThreads) * 16;
      v[u] = make_uint4((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0),
                        (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, o + 4, 0, 0),
                        (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, o + 8, 0, 0),
                        (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, o + 12, 0, 0));
    }
  }
  const int hbin = tid & (kBins1 - 1), c0 = tid >> 8;
  uint32_t hs = 0u;
  if (!RAW) {                                       // first digit: the chunk histograms of the keys kernel
    const int nch = (n + kKeyChunk - 1) / kKeyChunk;   // <= 32 = 4 x 8 loads per bin
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(chist + (size_t)inst * nchunk * kBins1), (short)0, nch * kBins1 * 4, kBufferRsrcWord3);
    uint32_t hv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      hv[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, ((c0 + 4 * u) * kBins1 + hbin) * 4, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) hs += hv[u];
  }
#pragma unroll
  for (int i = 0; i < 4096 / kSelThreads; ++i) hist[tid + i * kSelThreads] = 0u;
  if (tid == 0) ccount = 0u;
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int i4 = tid + u * kSelThreads;
    v[u] = to_keys<RAW>(v[u]);
    if (i4 < nv) skeys[vslot(i4)] = v[u];
  }
  __syncthreads();
  if (RAW) {
    // one head per group: no keys pass ran; the first digit is counted here from the loaded keys
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int j = 4 * (tid + u * kSelThreads);
      if (j + 3 < n) {
        atomicAdd(&hist[v[u].x >> S1], 1u);
        atomicAdd(&hist[v[u].y >> S1], 1u);
        atomicAdd(&hist[v[u].z >> S1], 1u);
        atomicAdd(&hist[v[u].w >> S1], 1u);
      } else if (j < n) {
        atomicAdd(&hist[v[u].x >> S1], 1u);
        if (j + 1 < n) atomicAdd(&hist[v[u].y >> S1], 1u);
        if (j + 2 < n) atomicAdd(&hist[v[u].z >> S1], 1u);
      }
    }
  } else {
    atomicAdd(&hist[hbin], hs);
  }
  __syncthreads();

  int need = K;
  find_bin_fixed<(1 << (32 - S1))>(hist, need, scan_smem, bcast);
  const uint32_t d1 = bcast[0];
  need -= (int)bcast[1];
  const int ncand = (int)hist[d1];                  // keys in the threshold's first-digit bin
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4096 / kSelThreads; ++i) hist[tid + i * kSelThreads] = 0u;

  // the sweep over the thread's contiguous keys (kept in registers for the long-bin path)
  const int v0 = tid * kVecPerThread;
  const uint32_t* skw = reinterpret_cast<const uint32_t*>(skeys);
  auto key_at = [&](int j) { return skw[vslot(j >> 2) * 4 + (j & 3)]; };
  uint4 kv[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) kv[u] = skeys[vslot(v0 + u)];
  const int nvalid = min(max(n - 4 * v0, 0), kKeysPerThread);
  const uint32_t vmask = nvalid >= 32 ? 0xFFFFFFFFu : (1u << nvalid) - 1u;
  uint32_t gtm = 0u, cm = 0u;
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t top = k4[e] >> S1;
      gtm |= (uint32_t)(top > d1) << (4 * u + e);
      cm |= (uint32_t)(top == d1) << (4 * u + e);
    }
  }
  gtm &= vmask;
  cm &= vmask;
  const bool use_list = ncand <= kCandList;         // uniform over the workgroup
  if (use_list) {
    // append the candidates' positions, in any order: one LDS counter add per wave
    const uint32_t c = __popc(cm);
    const uint32_t incl = wave_incl_scan(c);
    uint32_t wbase = 0u;
    if ((tid & (kWave - 1)) == kWave - 1 && incl) wbase = atomicAdd(&ccount, incl);
    uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)wbase, kWave - 1) + incl - c;
    for (uint32_t m = cm; m; m &= m - 1)
      if (at < (uint32_t)kCandList) clist[at++] = 32 * tid + __ffs(m) - 1;
  }
  __syncthreads();
  if (use_list) {
#pragma unroll
    for (int q = 0; q < kListPerThread; ++q) {
      const int i = tid + q * kSelThreads;
      if (i < ncand) atomicAdd(&hist[(key_at(clist[i]) >> S2) & 4095u], 1u);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((cm >> (4 * u + e)) & 1u) atomicAdd(&hist[(k4[e] >> S2) & 4095u], 1u);
    }
  }
  __syncthreads();
  find_bin_fixed<4096>(hist, need, scan_smem, bcast);
  uint32_t prefix = (d1 << S1) | (bcast[0] << S2);
  uint32_t pmask = ~((1u << S2) - 1u);
  need -= (int)bcast[1];
  const bool whole = (int)hist[bcast[0]] == need;   // every key of the bin is taken: T is resolved
  __syncthreads();
  if (!whole) {
#pragma unroll
    for (int i = 0; i < 4096 / kSelThreads; ++i) hist[tid + i * kSelThreads] = 0u;
    __syncthreads();
    if (use_list) {
#pragma unroll
      for (int q = 0; q < kListPerThread; ++q) {
        const int i = tid + q * kSelThreads;
        if (i < ncand) {
          const uint32_t k = key_at(clist[i]);
          if ((k & pmask) == prefix) atomicAdd(&hist[k & ((1u << S2) - 1u)], 1u);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kVecPerThread; ++u) {
        const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (((cm >> (4 * u + e)) & 1u) && (k4[e] & pmask) == prefix) atomicAdd(&hist[k4[e] & ((1u << S2) - 1u)], 1u);
      }
    }
    __syncthreads();
    find_bin_fixed<(1 << S2)>(hist, need, scan_smem, bcast);
    prefix |= bcast[0];
    pmask = 0xFFFFFFFFu;
    need -= (int)bcast[1];
  }
  // resolve the candidates: masked key > prefix -> selected; == prefix -> tie at T
  uint32_t eqm = 0u;
  if (use_list) {
    uint32_t* selbm = hist;                         // the histogram is read no more (find_bin's barrier)
    uint32_t* tiebm = hist + kSelThreads;
    selbm[tid] = 0u;
    tiebm[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kListPerThread; ++q) {
      const int i = tid + q * kSelThreads;
      if (i < ncand) {
        const int j = clist[i];
        const uint32_t mk = key_at(j) & pmask;
        if (mk > prefix) atomicOr(&selbm[j >> 5], 1u << (j & 31));
        else if (mk == prefix) atomicOr(&tiebm[j >> 5], 1u << (j & 31));
      }
    }
    __syncthreads();
    gtm |= selbm[tid];
    eqm = tiebm[tid];
  } else {
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t mk = k4[e] & pmask;
        const bool c = (cm >> (4 * u + e)) & 1u;
        gtm |= (uint32_t)(c && mk > prefix) << (4 * u + e);
        eqm |= (uint32_t)(c && mk == prefix) << (4 * u + e);
      }
    }
  }
  // when all 32 bits are resolved the tied keys are equal and the lower positions win; otherwise
  // every one of them is taken (need equals their count)
  const uint32_t gt = __popc(gtm), eq = __popc(eqm);
  uint32_t tot;
  const uint32_t before = scan_block((eq << 16) | gt, scan_smem, tot);   // n <= 32768 < 2^16
  const int eq_before = (int)(before >> 16), gt_before = (int)(before & 0xFFFFu);
  const int take_eq = max(0, min((int)eq, need - eq_before));
  uint32_t keep_eq = eqm;
  for (int drop = (int)eq - take_eq; drop > 0; --drop) keep_eq &= ~(0x80000000u >> __clz(keep_eq));
  const uint32_t selw = gtm | keep_eq;
  // stage the selection in LDS (the keys are read no more: the scan's barriers passed), then write
  // it out coalesced
  int32_t* sOut = reinterpret_cast<int32_t*>(skeys);
  int o = gt_before + min(eq_before, need);
  for (uint32_t m = selw; m; m &= m - 1)
    if (o < K) sOut[o++] = 32 * tid + __ffs(m) - 1;
  __syncthreads();
  for (int i = tid; i < K; i += kSelThreads) out[i] = sOut[i];
  if (tid == 0) sel_count[inst] = K;
  if (kPlan) plan(selw);
}

// The register-resident select: the keys of a row stay in registers, 64 per thread in strided
// (coalesced) vectors v = tid + NT u, and never in LDS.  NT = 1024 takes rows of 32 769 .. 65 536
// keys with a budget of at most kRegList; NT = 512 takes rows of up to 32 768 keys for many instances
// of one head each (see below).  With one head per group
// the first digit (12 bits) is counted here from the loaded keys, each vector as it lands, and no
// keys pass runs; otherwise it comes from the chunk histograms (8 bits).  The sweep marks keys above
// the threshold's first-digit bin in an LDS bitmap of the row (a 4-key vector is 4 bits of one word;
// the 8 lanes of a word OR their pieces by DPP and one of them stores it) and
// lists the candidates' positions; their keys are fetched once more from the row (L2) into the list,
// so the later digit passes and the final compare run over the list alone.  Thread t then owns bitmap
// words 2t and 2t + 1 (positions [64t, 64t + 64)) for the ordered output.
// NT = 512 (a list of 4096, ~60 KB of LDS, at most 128 registers): two workgroups share a CU, so that
// many instances of one head each (MLA: 4 x 128) run as one round, where the LDS-staged select runs
// one workgroup per CU.
constexpr int kRegKeys = 65536;
constexpr int kRegList = 8192;
constexpr int kRegThreadsHalf = 512;

template <bool RAW, int CPT, int NT = kSelThreads>
__global__ __launch_bounds__(NT, 4) void topk_select_reg_kernel(const uint32_t* __restrict__ keys,
                                                                      const uint32_t* __restrict__ chist,
                                                                      const int32_t* __restrict__ lengths,
                                                                      int32_t* __restrict__ sel_idx,
                                                                      int32_t* __restrict__ sel_count,
                                                                      int n_groups, int max_len, int budget,
                                                                      int nchunk, PlanBufs pb) {
  constexpr int kKeys = 64 * NT;                   // keys of a row at most
  constexpr int kList = 8 * NT;                    // candidate list entries
  constexpr int kWords = kKeys / 32;               // bitmap words of a row: 2 per thread
  constexpr int kVec = kKeys / 4 / NT;             // 16 vectors = 64 keys per thread
  constexpr int S1 = RAW ? 20 : 24;
  constexpr int S2 = S1 - 12;
  static_assert(kWords == 2 * NT && kList % NT == 0 && 4096 % NT == 0, "row and list layout");
  __shared__ uint32_t hist[4096];
  __shared__ int32_t cpos[kList];                  // candidate positions; later the staged selection
  __shared__ uint32_t ckey[kList];
  __shared__ uint32_t gtbm[kWords], selbm[kWords], tiebm[kWords];
  __shared__ __align__(16) uint32_t scan_smem[16];
  __shared__ uint32_t bcast[2];
  __shared__ uint32_t ccount;

  const int inst = blockIdx.x;
  const int b = inst / n_groups;
  const int n = clamp_len(lengths, b, max_len);
  const int K = budget;
  const int tid = threadIdx.x;
  int32_t* out = sel_idx + (size_t)inst * K;
  // with CPT > 0 the instance's plan follows (2 K <= kList: its lists take the key list's LDS)
  constexpr bool kPlan = CPT > 0;
  constexpr int kP = kPlan ? CPT : 1;
  uint32_t oldw[2] = {0u, 0u};
  int32_t pos[kP];
  int32_t* sp = pb.slot_pos + (size_t)inst * K;
  uint32_t* bm = pb.resident_bm + (size_t)inst * pb.bm_words;
  if (kPlan) {
    const int Cx = (K + NT - 1) / NT;
    const int x0 = min(tid * Cx, K), x1 = min(x0 + Cx, K);
#pragma unroll
    for (int u = 0; u < kP; ++u) pos[u] = x0 + u < x1 ? sp[x0 + u] : -1;
#pragma unroll
    for (int w = 0; w < 2; ++w)
      if (2 * tid + w < pb.bm_words) oldw[w] = bm[2 * tid + w];
  }
  auto plan = [&](uint64_t sel64) {
    const uint32_t sw[2] = {(uint32_t)sel64, (uint32_t)(sel64 >> 32)};
    plan_words<kP, 2, NT>(sw, oldw, pos, sp, bm, pb.load_pos + (size_t)inst * K, pb.load_slot + (size_t)inst * K,
                      pb.load_count + inst, K, pb.bm_words, reinterpret_cast<int32_t*>(ckey),
                      reinterpret_cast<int32_t*>(ckey) + K, gtbm, scan_smem);
  };
  if (n <= K) {
    for (int i = tid; i < K; i += NT) out[i] = i < n ? i : -1;
    if (tid == 0) sel_count[inst] = n;
    if (kPlan) {
      const int r = n - 64 * tid;                  // this thread's positions [64 tid, 64 tid + 64)
      plan(r >= 64 ? ~0ull : r > 0 ? (1ull << r) - 1ull : 0ull);
    }
    return;
  }
  const uint32_t* kin = keys + (size_t)inst * max_len;
  const int nv = (n + 3) / 4;
  const bool aligned = (max_len & 3) == 0;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kin), (short)0,
                                                                      aligned ? nv * 16 : n * 4, kBufferRsrcWord3);
  auto load_vec = [&](int u) -> uint4 {             // keys 4v .. 4v + 3, v = tid + NT u (zeros past the row)
    const int o = (tid + u * NT) * 16;
    if (aligned) {
      const Vec16 x = ld16_buffer(kr, (uint32_t)o);
      return make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
    }
    return make_uint4((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(kr, o, 0, 0),
                      (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(kr, o + 4, 0, 0),
                      (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(kr, o + 8, 0, 0),
                      (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(kr, o + 12, 0, 0));
  };
  // one branch around all the loads (not one per vector), so that the waits before each vector's
  // first use count only the loads issued after it
  uint4 v[kVec];
  if (aligned) {
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const Vec16 x = ld16_buffer(kr, (uint32_t)(tid + u * NT) * 16u);
      v[u] = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kVec; ++u) v[u] = load_vec(u);
  }
  // first digit from the chunk histograms (<= kKeys / kKeyChunk chunks): bin tid % 256 of chunks
  // c0, c0 + NT / 256, ...
  constexpr int kChunkGroups = NT / kBins1;
  constexpr int kChunkLoads = kKeys / kKeyChunk / kChunkGroups;
  const int hbin = tid & (kBins1 - 1), c0 = tid / kBins1;
  uint32_t hs = 0u;
  if (!RAW) {
    const int nch = (n + kKeyChunk - 1) / kKeyChunk;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(chist + (size_t)inst * nchunk * kBins1), (short)0, nch * kBins1 * 4, kBufferRsrcWord3);
    uint32_t hv[kChunkLoads];
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u)
      hv[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, ((c0 + kChunkGroups * u) * kBins1 + hbin) * 4, 0, 0);
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u) hs += hv[u];
  }
#pragma unroll
  for (int i = 0; i < 4096 / NT; ++i) hist[tid + i * NT] = 0u;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    selbm[tid + i * NT] = 0u;
    tiebm[tid + i * NT] = 0u;
  }
  if (tid == 0) ccount = 0u;
  // the cleared histogram is visible to every thread; the key loads are still in flight, and each
  // vector is keyed and counted as it lands
  __syncthreads();
  if (RAW) {
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      v[u] = to_keys<RAW>(v[u]);
      const int j = 4 * (tid + u * NT);
      if (j + 3 < n) {
        atomicAdd(&hist[v[u].x >> S1], 1u);
        atomicAdd(&hist[v[u].y >> S1], 1u);
        atomicAdd(&hist[v[u].z >> S1], 1u);
        atomicAdd(&hist[v[u].w >> S1], 1u);
      } else if (j < n) {
        atomicAdd(&hist[v[u].x >> S1], 1u);
        if (j + 1 < n) atomicAdd(&hist[v[u].y >> S1], 1u);
        if (j + 2 < n) atomicAdd(&hist[v[u].z >> S1], 1u);
      }
    }
  } else {
    atomicAdd(&hist[hbin], hs);
  }
  __syncthreads();

  int need = K;
  find_bin_fixed<(1 << (32 - S1)), NT>(hist, need, scan_smem, bcast);
  const uint32_t d1 = bcast[0];
  need -= (int)bcast[1];
  const int ncand = (int)hist[d1];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4096 / NT; ++i) hist[tid + i * NT] = 0u;

  // the sweep: above the bin -> the gt bitmap; in the bin -> a candidate (bit 4u + e of cm)
  uint64_t cm = 0u;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int i4 = tid + u * NT;
    const uint32_t k4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t g4 = 0u, c4 = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = 4 * i4 + e < n;
      const uint32_t top = k4[e] >> S1;
      g4 |= (uint32_t)(valid && top > d1) << e;
      c4 |= (uint32_t)(valid && top == d1) << e;
    }
    // the 8 lanes tid & ~7 .. tid | 7 hold the 32 positions of bitmap word i4 >> 3: their 4-bit
    // pieces are OR-ed by DPP and one lane stores the word (every word is written once, no clear)
    uint32_t gw = g4 << (4 * (i4 & 7));
    gw |= dpp_u<kDppQuadXor1>(gw);
    gw |= dpp_u<kDppQuadXor2>(gw);
    gw |= dpp_u<kDppHalfMirror>(gw);
    if ((tid & 7) == 0) gtbm[i4 >> 3] = gw;
    cm |= (uint64_t)c4 << (4 * u);
  }
  const bool use_list = ncand <= kList;            // uniform over the workgroup
  if (use_list) {
    const uint32_t c = (uint32_t)__popcll(cm);
    const uint32_t incl = wave_incl_scan(c);
    uint32_t wbase = 0u;
    if ((tid & (kWave - 1)) == kWave - 1 && incl) wbase = atomicAdd(&ccount, incl);
    uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)wbase, kWave - 1) + incl - c;
    for (uint64_t m = cm; m; m &= m - 1) {
      const int bit = __builtin_ctzll(m);
      if (at < (uint32_t)kList) cpos[at++] = 4 * (tid + (bit >> 2) * NT) + (bit & 3);
    }
  }
  __syncthreads();
  constexpr int kListPerThread = kList / NT;
  if (use_list) {
    // the candidates' keys, fetched once more from the row (L2), all loads in flight together
    uint32_t kk[kListPerThread];
#pragma unroll
    for (int q = 0; q < kListPerThread; ++q) {
      const int i = tid + q * NT;
      kk[q] = i < ncand ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(kr, cpos[i] * 4, 0, 0) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kListPerThread; ++q) {
      const int i = tid + q * NT;
      if (i < ncand) {
        const uint32_t k = RAW ? order_key(__uint_as_float(kk[q])) : kk[q];
        ckey[i] = k;                                // read back only by this thread
        atomicAdd(&hist[(k >> S2) & 4095u], 1u);
      }
    }
  } else {                                          // a bin past the list: the keys read again (L2)
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const uint4 w = to_keys<RAW>(load_vec(u));
      const uint32_t k4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((cm >> (4 * u + e)) & 1u) atomicAdd(&hist[(k4[e] >> S2) & 4095u], 1u);
    }
  }
  __syncthreads();
  find_bin_fixed<4096, NT>(hist, need, scan_smem, bcast);
  uint32_t prefix = (d1 << S1) | (bcast[0] << S2);
  uint32_t pmask = ~((1u << S2) - 1u);
  need -= (int)bcast[1];
  const bool whole = (int)hist[bcast[0]] == need;
  __syncthreads();
  if (!whole) {
#pragma unroll
    for (int i = 0; i < 4096 / NT; ++i) hist[tid + i * NT] = 0u;
    __syncthreads();
    if (use_list) {
#pragma unroll
      for (int q = 0; q < kListPerThread; ++q) {
        const int i = tid + q * NT;
        if (i < ncand) {
          const uint32_t k = ckey[i];
          if ((k & pmask) == prefix) atomicAdd(&hist[k & ((1u << S2) - 1u)], 1u);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kVec; ++u) {
        const uint4 w = to_keys<RAW>(load_vec(u));
        const uint32_t k4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (((cm >> (4 * u + e)) & 1u) && (k4[e] & pmask) == prefix) atomicAdd(&hist[k4[e] & ((1u << S2) - 1u)], 1u);
      }
    }
    __syncthreads();
    find_bin_fixed<(1 << S2), NT>(hist, need, scan_smem, bcast);
    prefix |= bcast[0];
    pmask = 0xFFFFFFFFu;
    need -= (int)bcast[1];
  }
  // resolve the candidates into the selected and tied bitmaps
  if (use_list) {
#pragma unroll
    for (int q = 0; q < kListPerThread; ++q) {
      const int i = tid + q * NT;
      if (i < ncand) {
        const int j = cpos[i];
        const uint32_t mk = ckey[i] & pmask;
        if (mk > prefix) atomicOr(&selbm[j >> 5], 1u << (j & 31));
        else if (mk == prefix) atomicOr(&tiebm[j >> 5], 1u << (j & 31));
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int i4 = tid + u * NT;
      const uint4 w = to_keys<RAW>(load_vec(u));
      const uint32_t k4[4] = {w.x, w.y, w.z, w.w};
      uint32_t s4 = 0u, t4 = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool c = (cm >> (4 * u + e)) & 1u;
        const uint32_t mk = k4[e] & pmask;
        s4 |= (uint32_t)(c && mk > prefix) << e;
        t4 |= (uint32_t)(c && mk == prefix) << e;
      }
      if (s4) atomicOr(&selbm[i4 >> 3], s4 << (4 * (i4 & 7)));
      if (t4) atomicOr(&tiebm[i4 >> 3], t4 << (4 * (i4 & 7)));
    }
  }
  __syncthreads();
  // thread t: positions [64t, 64t + 64) = words 2t, 2t + 1
  const uint64_t selm = ((uint64_t)(gtbm[2 * tid + 1] | selbm[2 * tid + 1]) << 32) | (gtbm[2 * tid] | selbm[2 * tid]);
  const uint64_t eqm = ((uint64_t)tiebm[2 * tid + 1] << 32) | tiebm[2 * tid];
  const uint32_t gt = (uint32_t)__popcll(selm), eq = (uint32_t)__popcll(eqm);
  uint32_t tot;
  // gt totals at most K <= kList < 2^14; eq totals at most 65536 < 2^18
  const uint32_t before = scan_block<NT>((eq << 14) | gt, scan_smem, tot);
  const int eq_before = (int)(before >> 14), gt_before = (int)(before & 0x3FFFu);
  const int take_eq = max(0, min((int)eq, need - eq_before));
  uint64_t keep_eq = eqm;
  for (int drop = (int)eq - take_eq; drop > 0; --drop) keep_eq &= ~(1ull << (63 - __clzll(keep_eq)));
  // stage the selection in LDS (the candidate list is read no more: the scan's barriers passed)
  int o = gt_before + min(eq_before, need);
  for (uint64_t m = selm | keep_eq; m; m &= m - 1)
    if (o < K) cpos[o++] = 64 * tid + __builtin_ctzll(m);
  __syncthreads();
  for (int i = tid; i < K; i += NT) out[i] = cpos[i];
  if (tid == 0) sel_count[inst] = K;
  if (kPlan) plan(selm | keep_eq);                  // its LDS (key list, gt bitmap) is read no more
}

}  // namespace

size_t topk_ws_bytes(const spc_shape& s) {
  const size_t inst = (size_t)s.batch * s.n_groups;
  const size_t nchunk = (size_t)(s.max_len + kKeyChunk - 1) / kKeyChunk;
  return inst * (size_t)s.max_len * sizeof(uint32_t) + inst * nchunk * kBins1 * sizeof(uint32_t);
}

namespace {

// Rows past the LDS stage that the register-resident select takes.
bool reg_select(const spc_shape& s) {
  return s.max_len > kTopkLdsKeys && s.max_len <= kRegKeys && s.budget <= kRegList;
}

// Many instances of one head each with rows that fit the LDS stage: the LDS-staged select runs one
// workgroup per CU (more than 256 instances: several rounds), the 512-thread register select two per
// CU.  Budgets of up to 2048 (its plan's two lists take the 4096-entry key list).
bool half_select(const spc_shape& s) {
  return s.n_q_heads == s.n_groups && s.max_len <= kTopkLdsKeys && s.batch * s.n_groups > 256 &&
         s.budget <= 8 * kRegThreadsHalf / 2;
}

// The keys pass (group max, first-digit histograms), unless one head per group with rows that fit
// LDS lets the select key the scores and count the first digit itself.  *kin: the keys the select
// reads (with one head per group, the scores' own words, keyed on load).
hipError_t launch_keys(const spc_shape& s, const float* scores, const float2* stats, int stat_tile,
                       const int32_t* lengths, void* ws, hipStream_t st, const uint32_t** kin, uint32_t** chist) {
  const int inst = s.batch * s.n_groups;
  const int nchunk = (s.max_len + kKeyChunk - 1) / kKeyChunk;
  const int ntiles = stat_tile > 0 ? (s.max_len + stat_tile - 1) / stat_tile : 0;
  uint32_t* keys = static_cast<uint32_t*>(ws);
  *chist = keys + (size_t)inst * s.max_len;
  const bool raw = s.n_q_heads == s.n_groups;
  *kin = raw ? reinterpret_cast<const uint32_t*>(scores) : keys;
  if (raw && (s.max_len <= kTopkLdsKeys || reg_select(s))) return hipSuccess;
  const dim3 kg(nchunk, inst);
  if (stats)
    topk_keys_kernel<true><<<kg, kKeyThreads, 0, st>>>(scores, stats, lengths, keys, *chist, s.n_q_heads,
                                                       s.n_groups, s.max_len, s.budget, nchunk, ntiles, stat_tile);
  else
    topk_keys_kernel<false><<<kg, kKeyThreads, 0, st>>>(scores, nullptr, lengths, keys, *chist, s.n_q_heads,
                                                        s.n_groups, s.max_len, s.budget, nchunk, 0, 1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const spc_shape& s, const float* scores, const float2* stats, int stat_tile,
                       const int32_t* lengths, int32_t* sel_idx, int32_t* sel_count, void* ws, hipStream_t st) {
  const int inst = s.batch * s.n_groups;
  const int nchunk = (s.max_len + kKeyChunk - 1) / kKeyChunk;
  const uint32_t* kin;
  uint32_t* chist;
  const hipError_t e = launch_keys(s, scores, stats, stat_tile, lengths, ws, st, &kin, &chist);
  if (e != hipSuccess) return e;
  const bool raw = s.n_q_heads == s.n_groups;
  const PlanBufs none{};
  if (half_select(s)) {
    topk_select_reg_kernel<true, 0, kRegThreadsHalf><<<dim3(inst), kRegThreadsHalf, 0, st>>>(
        kin, chist, lengths, sel_idx, sel_count, s.n_groups, s.max_len, s.budget, nchunk, none);
  } else if (s.max_len <= kTopkLdsKeys) {
    if (raw)
      topk_select_lds_kernel<true, 0><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx, sel_count,
                                                                          s.n_groups, s.max_len, s.budget, nchunk,
                                                                          none);
    else
      topk_select_lds_kernel<false, 0><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx,
                                                                           sel_count, s.n_groups, s.max_len,
                                                                           s.budget, nchunk, none);
  } else if (reg_select(s)) {
    if (raw)
      topk_select_reg_kernel<true, 0><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx, sel_count,
                                                                          s.n_groups, s.max_len, s.budget, nchunk,
                                                                          none);
    else
      topk_select_reg_kernel<false, 0><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx,
                                                                           sel_count, s.n_groups, s.max_len,
                                                                           s.budget, nchunk, none);
  } else {
    if (raw)
      topk_select_kernel<true><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx, sel_count,
                                                                   s.n_groups, s.max_len, s.budget, nchunk);
    else
      topk_select_kernel<false><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx, sel_count,
                                                                    s.n_groups, s.max_len, s.budget, nchunk);
  }
  return hipGetLastError();
}

bool select_plan_fused(const spc_shape& s) {
  // LDS select: the staged selection and the plan's lists (3 K words) and bitmap (<= 1024 words) fit
  // the keys' LDS; register select: the plan's two lists fit the key list
  if (s.max_len <= kTopkLdsKeys)
    return s.budget <= kPlanMaxBudget && 3 * s.budget + 1024 <= kTopkLdsKeys;
  return reg_select(s) && 2 * s.budget <= kRegList;
}

hipError_t launch_select_plan(const spc_shape& s, const float* scores, const float2* stats, int stat_tile,
                              const int32_t* lengths, int32_t* sel_idx, int32_t* sel_count, int32_t* slot_pos,
                              uint32_t* resident_bm, int32_t* load_pos, int32_t* load_slot, int32_t* load_count,
                              void* ws, hipStream_t st) {
  if (!select_plan_fused(s)) return hipErrorInvalidValue;
  const int inst = s.batch * s.n_groups;
  const int nchunk = (s.max_len + kKeyChunk - 1) / kKeyChunk;
  const uint32_t* kin;
  uint32_t* chist;
  const hipError_t e = launch_keys(s, scores, stats, stat_tile, lengths, ws, st, &kin, &chist);
  if (e != hipSuccess) return e;
  const bool raw = s.n_q_heads == s.n_groups;
  const PlanBufs pb{slot_pos, resident_bm, load_pos, load_slot, load_count, (s.max_len + 31) / 32};
  if (half_select(s)) {                            // 512 threads, budget <= 2048: cpt <= 4
    const int hc = (s.budget + kRegThreadsHalf - 1) / kRegThreadsHalf;
    switch (hc <= 1 ? 1 : hc <= 2 ? 2 : 4) {
#define SPC_CASE(N)                                                                                           \
  case N:                                                                                                     \
    topk_select_reg_kernel<true, N, kRegThreadsHalf><<<dim3(inst), kRegThreadsHalf, 0, st>>>(                 \
        kin, chist, lengths, sel_idx, sel_count, s.n_groups, s.max_len, s.budget, nchunk, pb);                 \
    break;
      SPC_CASE(1)
      SPC_CASE(2)
      SPC_CASE(4)
#undef SPC_CASE
    }
    return hipGetLastError();
  }
  const int cpt = (s.budget + kSelThreads - 1) / kSelThreads;
  if (s.max_len > kTopkLdsKeys) {                  // register select (budget <= kRegList / 2: cpt <= 4)
    switch ((cpt <= 1 ? 1 : cpt <= 2 ? 2 : 4) * (raw ? -1 : 1)) {
#define SPC_CASE(N)                                                                                           \
  case N:                                                                                                     \
    topk_select_reg_kernel<false, N><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx,        \
                                                                         sel_count, s.n_groups, s.max_len,    \
                                                                         s.budget, nchunk, pb);               \
    break;                                                                                                    \
  case -N:                                                                                                    \
    topk_select_reg_kernel<true, N><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx,         \
                                                                        sel_count, s.n_groups, s.max_len,     \
                                                                        s.budget, nchunk, pb);                \
    break;
      SPC_CASE(1)
      SPC_CASE(2)
      SPC_CASE(4)
#undef SPC_CASE
    }
    return hipGetLastError();
  }
  switch ((cpt <= 1 ? 1 : cpt <= 2 ? 2 : cpt <= 4 ? 4 : 8) * (raw ? -1 : 1)) {
#define SPC_CASE(N)                                                                                           \
  case N:                                                                                                     \
    topk_select_lds_kernel<false, N><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx,        \
                                                                         sel_count, s.n_groups, s.max_len,    \
                                                                         s.budget, nchunk, pb);               \
    break;                                                                                                    \
  case -N:                                                                                                    \
    topk_select_lds_kernel<true, N><<<dim3(inst), kSelThreads, 0, st>>>(kin, chist, lengths, sel_idx,         \
                                                                        sel_count, s.n_groups, s.max_len,     \
                                                                        s.budget, nchunk, pb);                \
    break;
    SPC_CASE(1)
    SPC_CASE(2)
    SPC_CASE(4)
    SPC_CASE(8)
#undef SPC_CASE
  }
  return hipGetLastError();
}

}  // namespace spc
