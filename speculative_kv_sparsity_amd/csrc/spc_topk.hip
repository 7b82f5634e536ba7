// Stage 2 - GQA group max and per-group Top-K.
//
//   v[b][g][j] = max over the query heads i of group g of probs[b][i][j]
//     (SpeContext blog section 5 / paper summary section 4.3: element-wise max
//      over a GQA group; MQA is one group; MHA selects per head)
//   S[b][g]    = the first min(K, n) positions by (v desc, j asc), written ascending
//     (blog section 2: at most K positions per head per round; the lower index
//      wins a tie)
//
// One workgroup of 1024 threads per (b, g).  The group max is taken while the
// keys are loaded.  Each fp32 value becomes an order-preserving uint32 key and
// the K-th largest key T is found by a 3-pass radix select (12 + 12 + 8 bits)
// with LDS histograms: every pass narrows the prefix of T and the number of
// elements still needed from inside it.  A final ordered compaction (two block
// scans over per-thread contiguous index ranges) writes every j with key > T
// and the lowest-index `need` ones with key == T, ascending.  For n <= 32768
// the keys stay in LDS (one pad word per 32 keys keeps the contiguous-range
// sweeps free of bank conflicts); longer rows recompute keys from global
// memory in every pass.
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

constexpr int kThreads = 1024;
constexpr int kPadded = kTopkLdsKeys + kTopkLdsKeys / 32;

__device__ __forceinline__ int pidx(int j) { return j + (j >> 5); }

// Order-preserving map from fp32 bits to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ probs,
                                                        const int32_t* __restrict__ lengths,
                                                        int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
                                                        int Hq, int n_groups, int max_len, int budget) {
  __shared__ uint32_t keys[IN_LDS ? kPadded : 1];
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t scan_smem[16];
  __shared__ uint32_t bcast[2];

  const int inst = blockIdx.x;
  const int b = inst / n_groups;
  const int g = inst - b * n_groups;
  const int Gq = Hq / n_groups;
  const int n = clamp_len(lengths, b, max_len);
  const int K = budget;
  const int tid = threadIdx.x;
  int32_t* out = sel_idx + (size_t)inst * K;

  if (n <= K) {
    for (int i = tid; i < K; i += kThreads) out[i] = i < n ? i : -1;
    if (tid == 0) sel_count[inst] = n;
    return;
  }

  const float* pb = probs + ((size_t)b * Hq + (size_t)g * Gq) * max_len;
  auto key_of = [&](int j) -> uint32_t {
    float v = pb[j];
    for (int h = 1; h < Gq; ++h) v = fmaxf(v, pb[(size_t)h * max_len + j]);
    return order_key(v);
  };

  if (IN_LDS) {
    for (int j = tid; j < n; j += kThreads) keys[pidx(j)] = key_of(j);
  }
  __syncthreads();
  auto key_at = [&](int j) -> uint32_t { return IN_LDS ? keys[pidx(j)] : key_of(j); };

  uint32_t prefix = 0u, pmask = 0u;
  int need = K;   // elements still to take from among the keys matching `prefix`
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nb = pass == 2 ? 256 : 4096;
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += kThreads) {
      const uint32_t key = key_at(j);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns the bins [hi - bpt, hi) counted from the top, hi = nb - t*bpt
    const int bpt = nb >= kThreads ? nb / kThreads : 1;
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
    const uint32_t bin = bcast[0];
    need -= (int)bcast[1];
    prefix |= bin << shift;
    pmask |= dmask << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;   // the K-th largest key; `need` copies of it are taken

  const int C = (n + kThreads - 1) / kThreads;
  const int j0 = min(tid * C, n), j1 = min(j0 + C, n);
  uint32_t gt = 0u, eq = 0u;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = key_at(j);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_excl_scan(eq, scan_smem, tot);
  const int take_eq = max(0, min((int)eq, need - (int)eq_before));
  const uint32_t base = block_excl_scan(gt + (uint32_t)take_eq, scan_smem, tot);
  int o = (int)base, e = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = key_at(j);
    bool take = key > T;
    if (key == T) {
      take = e < take_eq;
      ++e;
    }
    if (take && o < K) out[o++] = j;
  }
  if (tid == 0) sel_count[inst] = K;
}

}  // namespace

hipError_t launch_topk(const spc_shape& s, const float* probs, const int32_t* lengths, int32_t* sel_idx,
                       int32_t* sel_count, hipStream_t st) {
  const dim3 grid(s.batch * s.n_groups);
  if (s.max_len <= kTopkLdsKeys)
    topk_kernel<true><<<grid, kThreads, 0, st>>>(probs, lengths, sel_idx, sel_count, s.n_q_heads, s.n_groups,
                                                 s.max_len, s.budget);
  else
    topk_kernel<false><<<grid, kThreads, 0, st>>>(probs, lengths, sel_idx, sel_count, s.n_q_heads, s.n_groups,
                                                  s.max_len, s.budget);
  return hipGetLastError();
}

}  // namespace spc
