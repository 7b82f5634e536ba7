// Stage 2 - GQA group max and per-group Top-K.
//
//   v[b][g][j] = max over the query heads i of group g of probs[b][i][j]
//     (SpeContext blog section 5 / paper summary section 4.3: element-wise max
//      over a GQA group; MQA is one group; MHA selects per head)
//   S[b][g]    = the first min(K, n) positions by (v desc, j asc), written ascending
//     (blog section 2: at most K positions per head per round; the lower index
//      wins a tie)
//
// Each fp32 value becomes an order-preserving uint32 key; the K-th largest key
// T is found by radix select over 8 + 12 + 12 bits.
//
// topk_keys_kernel    many workgroups per (b, g), kKeyChunk positions each:
//   takes the group max while reading the heads' rows once, writes the keys to
//   the workspace and the chunk's histogram of the top 8 key bits.
// topk_select_kernel  one 1024-thread workgroup per (b, g): sums the chunk
//   histograms (first digit), runs the two remaining 12-bit passes with LDS
//   histograms over the keys that still match the prefix, and compacts every j
//   with key > T plus the lowest-index `need` ones with key == T, ascending,
//   with two block scans over per-thread contiguous index ranges.  For
//   n <= 32768 the keys are staged in LDS (one pad word per 32 keys keeps the
//   contiguous-range sweeps free of bank conflicts); longer rows are read from
//   the workspace (L2) in every pass.
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

constexpr int kKeyThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kBins1 = 256;                       // first digit: key bits 31..24
constexpr int kPadded = kTopkLdsKeys + kTopkLdsKeys / 32;

__device__ __forceinline__ int pidx(int j) { return j + (j >> 5); }

// Order-preserving map from fp32 bits to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kKeyThreads) void topk_keys_kernel(const float* __restrict__ probs,
                                                                const int32_t* __restrict__ lengths,
                                                                uint32_t* __restrict__ keys,
                                                                uint32_t* __restrict__ chist, int Hq, int n_groups,
                                                                int max_len, int budget, int nchunk) {
  const int inst = blockIdx.y;
  const int c = blockIdx.x;
  const int b = inst / n_groups;
  const int g = inst - b * n_groups;
  const int n = clamp_len(lengths, b, max_len);
  const int j0 = c * kKeyChunk;
  if (n <= budget || j0 >= n) return;
  const int j1 = min(j0 + kKeyChunk, n);
  const int Gq = Hq / n_groups;
  const float* pb = probs + ((size_t)b * Hq + (size_t)g * Gq) * max_len;
  uint32_t* kout = keys + (size_t)inst * max_len;
  __shared__ uint32_t h[kBins1];
  h[threadIdx.x] = 0u;
  __syncthreads();
  constexpr int kPer = kKeyChunk / kKeyThreads;       // positions per thread
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + threadIdx.x + u * kKeyThreads;
    v[u] = j < j1 ? pb[j] : 0.f;
  }
  for (int hh = 1; hh < Gq; ++hh) {
    const float* ph = pb + (size_t)hh * max_len;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = j0 + threadIdx.x + u * kKeyThreads;
      if (j < j1) v[u] = fmaxf(v[u], ph[j]);
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + threadIdx.x + u * kKeyThreads;
    if (j < j1) {
      const uint32_t key = order_key(v[u]);
      kout[j] = key;
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

template <bool IN_LDS>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const uint32_t* __restrict__ keys,
                                                                  const uint32_t* __restrict__ chist,
                                                                  const int32_t* __restrict__ lengths,
                                                                  int32_t* __restrict__ sel_idx,
                                                                  int32_t* __restrict__ sel_count, int n_groups,
                                                                  int max_len, int budget, int nchunk) {
  __shared__ uint32_t skeys[IN_LDS ? kPadded : 1];
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
  if (IN_LDS) {
    // 16-byte loads, all of a thread's issued before its LDS stores (max_len % 4 == 0 keeps rows aligned)
    constexpr int kVecPerThread = kTopkLdsKeys / 4 / kSelThreads;
    const int n4 = (max_len % 4 == 0) ? n / 4 : 0;
    uint4 v[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int i4 = tid + u * kSelThreads;
      if (i4 < n4) v[u] = reinterpret_cast<const uint4*>(kin)[i4];
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int i4 = tid + u * kSelThreads;
      if (i4 < n4) {
        const int j = 4 * i4;
        skeys[pidx(j)] = v[u].x;
        skeys[pidx(j + 1)] = v[u].y;
        skeys[pidx(j + 2)] = v[u].z;
        skeys[pidx(j + 3)] = v[u].w;
      }
    }
    for (int j = 4 * n4 + tid; j < n; j += kSelThreads) skeys[pidx(j)] = kin[j];
  }
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
  auto key_at = [&](int j) -> uint32_t { return IN_LDS ? skeys[pidx(j)] : kin[j]; };

  int need = K;
  find_bin(hist, kBins1, need, scan_smem, bcast);
  uint32_t prefix = bcast[0] << 24;
  uint32_t pmask = 0xFF000000u;
  need -= (int)bcast[1];
  __syncthreads();
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 12 : 0;
    for (int i = tid; i < 4096; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += kSelThreads) {
      const uint32_t key = key_at(j);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 4095u], 1u);
    }
    __syncthreads();
    find_bin(hist, 4096, need, scan_smem, bcast);
    prefix |= bcast[0] << shift;
    pmask |= 4095u << shift;
    need -= (int)bcast[1];
    __syncthreads();
  }
  const uint32_t T = prefix;   // the K-th largest key; `need` copies of it are taken

  const int C = (n + kSelThreads - 1) / kSelThreads;
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

size_t topk_ws_bytes(const spc_shape& s) {
  const size_t inst = (size_t)s.batch * s.n_groups;
  const size_t nchunk = (size_t)(s.max_len + kKeyChunk - 1) / kKeyChunk;
  return inst * (size_t)s.max_len * sizeof(uint32_t) + inst * nchunk * kBins1 * sizeof(uint32_t);
}

hipError_t launch_topk(const spc_shape& s, const float* probs, const int32_t* lengths, int32_t* sel_idx,
                       int32_t* sel_count, void* ws, hipStream_t st) {
  const int inst = s.batch * s.n_groups;
  const int nchunk = (s.max_len + kKeyChunk - 1) / kKeyChunk;
  uint32_t* keys = static_cast<uint32_t*>(ws);
  uint32_t* chist = keys + (size_t)inst * s.max_len;
  topk_keys_kernel<<<dim3(nchunk, inst), kKeyThreads, 0, st>>>(probs, lengths, keys, chist, s.n_q_heads,
                                                               s.n_groups, s.max_len, s.budget, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.max_len <= kTopkLdsKeys)
    topk_select_kernel<true><<<dim3(inst), kSelThreads, 0, st>>>(keys, chist, lengths, sel_idx, sel_count,
                                                                 s.n_groups, s.max_len, s.budget, nchunk);
  else
    topk_select_kernel<false><<<dim3(inst), kSelThreads, 0, st>>>(keys, chist, lengths, sel_idx, sel_count,
                                                                  s.n_groups, s.max_len, s.budget, nchunk);
  return hipGetLastError();
}

}  // namespace spc
