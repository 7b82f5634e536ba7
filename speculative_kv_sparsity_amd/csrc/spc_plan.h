// The elastic plan of one (sequence, group) instance with a bitmap of the new selection in LDS,
// shared by the plan kernel (selection given as a list) and the Top-K select that ends with the
// plan (selection given as bitmap words, one per thread).
//
// The SpeContext blog's section 4 loop loads the positions of the new selection that are not
// resident (the set difference); its section 6 worked example ({1,8,21,35} -> {1,8,21,50})
// writes the one new position into the place of the one that left; the paper summary's section
// 5.4 keeps the budget fixed and loads in place.  Here: a slot is kept iff its position is in S
// (a bit test), a position of S is loaded iff its bit in the old resident bitmap is clear; the
// i-th ascending new position goes to the i-th ascending freed slot, freed slots left over become
// empty, and the resident bitmap becomes the bitmap of S.
#pragma once

#include "spc_common.h"

namespace spc {

constexpr int kPlanThreads = 1024;

// Called by all kPlanThreads threads of the workgroup (it has barriers).  S: the selection, c
// entries, ascending (global or LDS); sp, bm: the instance's slot map [K] and resident bitmap
// [bm_words] (in/out); lp, ls: its load lists [K] (out); lcount: its load count (out).  sL, sF:
// K words of LDS each, sB: bm_words words of LDS, scan_smem: 16 words.  CPT >= ceil(K / 1024).
template <int CPT>
__device__ __forceinline__ void plan_bitmap(const int32_t* S, int c, int32_t* __restrict__ sp,
                                            uint32_t* __restrict__ bm, int32_t* __restrict__ lp,
                                            int32_t* __restrict__ ls, int32_t* __restrict__ lcount, int K,
                                            int bm_words, int32_t* sL, int32_t* sF, uint32_t* sB,
                                            uint32_t* scan_smem) {
  const int tid = threadIdx.x;
  const int32_t pos_end = bm_words * 32;                   // positions outside [0, pos_end) are never loaded
  const int Cx = (K + kPlanThreads - 1) / kPlanThreads;   // <= CPT
  const int x0 = min(tid * Cx, K), x1 = min(x0 + Cx, K);
  const int Ci = (c + kPlanThreads - 1) / kPlanThreads;   // <= Cx
  const int i0 = min(tid * Ci, c), i1 = min(i0 + Ci, c);
  int32_t pos[CPT], sel[CPT];
  uint32_t oldw[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    pos[u] = x0 + u < x1 ? sp[x0 + u] : -1;
    sel[u] = i0 + u < i1 ? S[i0 + u] : -1;
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {                          // resident before the step (outside: never loaded)
    const int32_t j = sel[u];
    oldw[u] = j >= 0 && j < pos_end ? bm[j >> 5] : 0xFFFFFFFFu;
  }
  for (int w = tid; w < bm_words; w += kPlanThreads) sB[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int32_t j = sel[u];
    if (j >= 0 && j < pos_end) atomicOr(&sB[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t fmask = 0u, lmask = 0u, nf_loc = 0u, nl_loc = 0u;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int32_t q = pos[u];
    const bool keep = q >= 0 && q < pos_end && ((sB[q >> 5] >> (q & 31)) & 1u);
    if (x0 + u < x1 && !keep) { fmask |= 1u << u; ++nf_loc; }
    const int32_t j = sel[u];
    if (i0 + u < i1 && !((oldw[u] >> (j & 31)) & 1u)) { lmask |= 1u << u; ++nl_loc; }
  }
  uint32_t tot;
  const uint32_t before = block_excl_scan(nf_loc | (nl_loc << 16), scan_smem, tot);   // counts <= K < 2^16
  uint32_t fo = before & 0xFFFFu, lo = before >> 16;
  const int nf = (int)(tot & 0xFFFFu), nl = (int)(tot >> 16);
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    if ((fmask >> u) & 1u) sF[fo++] = x0 + u;
    if ((lmask >> u) & 1u) sL[lo++] = sel[u];
  }
  __syncthreads();
  // apply: the i-th position to load goes to the i-th freed slot, the rest empty; the resident set
  // becomes S
  for (int i = tid; i < nf; i += kPlanThreads) sp[sF[i]] = i < nl ? sL[i] : -1;
  for (int w = tid; w < bm_words; w += kPlanThreads) bm[w] = sB[w];
  for (int i = tid; i < K; i += kPlanThreads) {
    const bool v = i < nl;
    lp[i] = v ? sL[i] : -1;
    ls[i] = v ? sF[i] : -1;
  }
  if (tid == 0) *lcount = nl;
}

// The same plan with the selection given as bitmap words: thread t holds WPT consecutive words,
// selw[w] = word t WPT + w of the selection's bitmap (bit i set iff position 32 (t WPT + w) + i is
// selected, so S is the set bits in ascending order), oldw[w], the same words of the resident bitmap
// before the step, and pos[u], the slot map entries of its slots [t*Cx, t*Cx + Cx) (Cx = ceil(K /
// NT) <= CPT; -1 beyond K), for a workgroup of NT threads.  Requires bm_words <= WPT * NT.  sL, sF: K
// words of LDS each, sB: bm_words words.  The results are those of plan_bitmap on the same selection,
// entry for entry.
template <int CPT, int WPT = 1, int NT = kPlanThreads>
__device__ __forceinline__ void plan_words(const uint32_t (&selw)[WPT], const uint32_t (&oldw)[WPT],
                                           const int32_t (&pos)[CPT], int32_t* __restrict__ sp,
                                           uint32_t* __restrict__ bm, int32_t* __restrict__ lp,
                                           int32_t* __restrict__ ls, int32_t* __restrict__ lcount, int K,
                                           int bm_words, int32_t* sL, int32_t* sF, uint32_t* sB,
                                           uint32_t* scan_smem) {
  const int tid = threadIdx.x;
  const int32_t pos_end = bm_words * 32;
  const int Cx = (K + NT - 1) / NT;
  const int x0 = min(tid * Cx, K), x1 = min(x0 + Cx, K);
#pragma unroll
  for (int w = 0; w < WPT; ++w)
    if (tid * WPT + w < bm_words) sB[tid * WPT + w] = selw[w];
  __syncthreads();
  uint32_t fmask = 0u, nf_loc = 0u;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int32_t q = pos[u];
    const bool keep = q >= 0 && q < pos_end && ((sB[q >> 5] >> (q & 31)) & 1u);
    if (x0 + u < x1 && !keep) { fmask |= 1u << u; ++nf_loc; }
  }
  uint32_t lmask[WPT], nl_loc = 0u;
#pragma unroll
  for (int w = 0; w < WPT; ++w) {                          // selected and not resident: loaded
    lmask[w] = tid * WPT + w < bm_words ? selw[w] & ~oldw[w] : 0u;
    nl_loc += __popc(lmask[w]);
  }
  uint32_t tot;
  const uint32_t before = block_excl_scan(nf_loc | (nl_loc << 16), scan_smem, tot);   // counts <= K < 2^16
  uint32_t fo = before & 0xFFFFu, lo = before >> 16;
  const int nf = (int)(tot & 0xFFFFu), nl = (int)(tot >> 16);
#pragma unroll
  for (int u = 0; u < CPT; ++u)
    if ((fmask >> u) & 1u) sF[fo++] = x0 + u;
#pragma unroll
  for (int w = 0; w < WPT; ++w)
    for (uint32_t m = lmask[w]; m; m &= m - 1) sL[lo++] = 32 * (tid * WPT + w) + __ffs(m) - 1;
  __syncthreads();
  for (int i = tid; i < nf; i += NT) sp[sF[i]] = i < nl ? sL[i] : -1;
#pragma unroll
  for (int w = 0; w < WPT; ++w)
    if (tid * WPT + w < bm_words) bm[tid * WPT + w] = selw[w];
  for (int i = tid; i < K; i += NT) {
    const bool v = i < nl;
    lp[i] = v ? sL[i] : -1;
    ls[i] = v ? sF[i] : -1;
  }
  if (tid == 0) *lcount = nl;
}

}  // namespace spc
