// Stage 1 - retrieval scores: probs[b][i][j] = softmax_j(scale * q_i . k_{g(i), j}) over j < n_b.
//
// The AttentionWeight formula (SpeContext blog, section 2) evaluated by the
// retrieval head for every cached key, per query head (blog section 5, paper
// summary sections 4.2-4.3: only the Q/K path of the distilled model remains).
//
// Two kernels:
//   scores_logits_kernel    one pass over the key cache.  A workgroup owns one
//       (sequence, KV head, chunk of <= HC query heads) and kScoreTile positions.
//       Each key row is read ONCE for all HC heads that share it (GQA reuse).
//       8 lanes cooperate on a row: lane p holds the 16-byte chunks p, p+8, ...
//       so one wave load instruction covers 8 rows x 128 contiguous bytes (full
//       cache lines).  bf16 dot products use v_dot2_f32_bf16 on packed pairs
//       (no widening), the 8-lane sum uses DPP.  The tile's logits are
//       gathered per head in LDS and written as whole 16-byte vectors; the
//       tile's per-head (max, sum exp) go to the tile stats.
//   scores_normalize_kernel combines the tile partials of a head into
//       (max, sum) and rewrites its logits in place as exp(l - max) / sum.
// The log-domain form (logits + tile stats, no normalize pass) is what the
// ranking of stage 2 needs; the probabilities are the second kernel's work.
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kRowsPerIter = 32;              // 4 waves x 8 rows
constexpr int kIters = kScoreTile / kRowsPerIter;
constexpr int kUnroll = 4;                    // iterations whose loads are issued together

template <int DT, int D, int HC>
__global__ __launch_bounds__(kThreads) void scores_logits_kernel(
    const char* __restrict__ q, const char* __restrict__ k, const int32_t* __restrict__ lengths,
    float* __restrict__ probs, float2* __restrict__ part, int Hq, int Hkv, int max_len, int nchunk, int ntiles,
    float scale) {
  constexpr int EB = DT == SPC_BF16 ? 2 : 4;
  constexpr int RB = D * EB;                  // row bytes
  constexpr int CPL = RB / 16 / 8;            // 16-byte chunks per lane
  static_assert(RB % 128 == 0, "row must be a whole number of 8 x 16-byte chunks");

  const int per_kv = Hq / Hkv;
  const int inst = blockIdx.y;
  const int b = inst / (Hkv * nchunk);
  const int rem = inst - b * Hkv * nchunk;
  const int g = rem / nchunk;
  const int hc = rem - g * nchunk;
  const int h0 = g * per_kv + hc * HC;
  const int nh = min(HC, per_kv - hc * HC);
  const int n = clamp_len(lengths, b, max_len);
  const int row0 = blockIdx.x * kScoreTile;
  if (row0 >= n) return;

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int p = lane & 7, rr = lane >> 3;

  Vec16 qv[HC][CPL];
  const char* qb = q + ((size_t)b * Hq + h0) * RB;
#pragma unroll
  for (int h = 0; h < HC; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (h < nh) {
        qv[h][c] = ld16(qb + (size_t)h * RB + (p + 8 * c) * 16);
      } else {
        qv[h][c].w[0] = qv[h][c].w[1] = qv[h][c].w[2] = qv[h][c].w[3] = 0u;
      }
    }

  const char* kb = k + ((size_t)b * Hkv + g) * (size_t)max_len * RB;
  // the sequence's n key rows through a buffer resource (under 2 GiB, checked on the host): rows
  // past the length read zeros with no branch; the loads are marked nontemporal (each key row is
  // read once per step, so it need not stay in the caches)
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), (short)0, n * RB, kBufferRsrcWord3);
  __shared__ __align__(16) float slg[HC][kScoreTile];   // the tile's logits per head, for coalesced writes
  float lg[kIters];

#pragma unroll
  for (int u0 = 0; u0 < kIters; u0 += kUnroll) {
    Vec16 kv[kUnroll][CPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = row0 + (u0 + u) * kRowsPerIter + wid * 8 + rr;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        kv[u][c] = ld16_buffer<kLoadNontemporal>(krs, (uint32_t)(row * RB + (p + 8 * c) * 16));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = row0 + (u0 + u) * kRowsPerIter + wid * 8 + rr;
      float acc[HC];
#pragma unroll
      for (int h = 0; h < HC; ++h) acc[h] = 0.f;
      if (row < n) {
#pragma unroll
        for (int h = 0; h < HC; ++h)
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[h] = dot16<DT>(kv[u][c], qv[h][c], acc[h]);
      }
      float mine = 0.f;
#pragma unroll
      for (int h = 0; h < HC; ++h) {
        const float t = sum8(acc[h]);
        if (p == h) mine = t;
      }
      mine *= scale;
      const bool ok = row < n && p < nh;
      lg[u0 + u] = ok ? mine : -INFINITY;
      if (p < HC) slg[p][row - row0] = mine;
    }
  }

  // tile (max, sum exp) of head p over this workgroup's rows (not wanted: part is NULL, uniform)
  __shared__ float s_m[4][8];
  __shared__ float s_s[4][8];
  float m = -INFINITY;
  if (part) {
#pragma unroll
    for (int i = 0; i < kIters; ++i) m = fmaxf(m, lg[i]);
    m = max_across_rows8(m);
    if (rr == 0) s_m[wid][p] = m;
  }
  __syncthreads();                                 // also publishes the logits in slg
  // logits of the valid rows: 16-byte stores where four rows are valid and the row start is aligned
  {
    const int nrow = min(kScoreTile, n - row0);
    const bool vec = (max_len & 3) == 0;
    for (int i = threadIdx.x; i < nh * (kScoreTile / 4); i += kThreads) {
      const int h = i / (kScoreTile / 4), r4 = 4 * (i - h * (kScoreTile / 4));
      float* dst = probs + ((size_t)b * Hq + h0 + h) * (size_t)max_len + row0 + r4;
      if (vec && r4 + 3 < nrow) {
        *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(&slg[h][r4]);
      } else {
        for (int e = 0; e < 4 && r4 + e < nrow; ++e) dst[e] = slg[h][r4 + e];
      }
    }
  }
  if (!part) return;
  const float M = fmaxf(fmaxf(s_m[0][p], s_m[1][p]), fmaxf(s_m[2][p], s_m[3][p]));
  float sum = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kIters; ++i) sum += lg[i] == -INFINITY ? 0.f : __expf(lg[i] - M);
  }
  sum = sum_across_rows8(sum);
  if (rr == 0) s_s[wid][p] = sum;
  __syncthreads();
  if ((int)threadIdx.x < nh) {
    const float S = s_s[0][p] + s_s[1][p] + s_s[2][p] + s_s[3][p];
    part[((size_t)b * Hq + h0 + p) * ntiles + blockIdx.x] = make_float2(M, S);
  }
}

__device__ __forceinline__ void combine_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __expf(m - M)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - M));
  m = M;
}

__global__ __launch_bounds__(kThreads) void scores_normalize_kernel(float* __restrict__ probs,
                                                                    const float2* __restrict__ part,
                                                                    const int32_t* __restrict__ lengths, int Hq,
                                                                    int max_len, int ntiles, int tile) {
  const int bh = blockIdx.y;
  const int b = bh / Hq;
  const int n = clamp_len(lengths, b, max_len);
  const int j0 = blockIdx.x * kNormChunk;
  if (j0 >= n) return;
  const int nt = (n + tile - 1) / tile;
  // this workgroup's logits are loaded first: they do not depend on the head's (max, sum), so
  // both round trips overlap
  float* pr = probs + (size_t)bh * max_len;
  const int j1 = min(j0 + kNormChunk, n);
  constexpr int kPer = kNormChunk / kThreads;
  float x[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + threadIdx.x + u * kThreads;
    x[u] = j < j1 ? pr[j] : 0.f;
  }
  float m = -INFINITY, s = 0.f;
  for (int t = threadIdx.x; t < nt; t += kThreads) {
    const float2 v = part[(size_t)bh * ntiles + t];
    combine_ms(m, s, v.x, v.y);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave);
    const float s2 = __shfl_xor(s, o, kWave);
    combine_ms(m, s, m2, s2);
  }
  __shared__ float sm[4], ss[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sm[wid] = m; ss[wid] = s; }
  __syncthreads();
  m = sm[0]; s = ss[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) combine_ms(m, s, sm[w], ss[w]);
  const float inv = 1.f / s;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + threadIdx.x + u * kThreads;
    if (j < j1) pr[j] = __expf(x[u] - m) * inv;
  }
}

template <int DT, int D>
hipError_t launch_logits_hc(int HC, dim3 grid, hipStream_t st, const char* q, const char* k, const int32_t* lengths,
                            float* probs, float2* part, int Hq, int Hkv, int max_len, int nchunk, int ntiles,
                            float scale) {
  switch (HC) {
#define SPC_CASE(N)                                                                                       \
  case N:                                                                                                 \
    scores_logits_kernel<DT, D, N><<<grid, kThreads, 0, st>>>(q, k, lengths, probs, part, Hq, Hkv, max_len, \
                                                             nchunk, ntiles, scale);                     \
    break;
    SPC_CASE(1)
    SPC_CASE(2)
    SPC_CASE(4)
    SPC_CASE(8)
#undef SPC_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int heads_per_chunk(const spc_shape& s) {
  const int per_kv = s.n_q_heads / s.n_kv_heads;
  const int cap = 8;                          // register budget for the query chunks
  int hc = 1;
  while (hc < per_kv && hc < cap) hc <<= 1;
  return hc;
}

}  // namespace

bool mla_shape(const spc_shape& s) { return s.head_dim == kMlaLatent + kMlaRope; }

bool scores_supported(const spc_shape& s) {
  if (mla_shape(s))   // MFMA path: one latent head shared by 16..128 query heads, bf16 latent
    return s.dtype == SPC_BF16 && s.n_kv_heads == 1 && s.n_q_heads % 16 == 0 && s.n_q_heads <= 128;
  // one KV head's keys of a sequence are read through a 32-bit buffer range: under 2 GiB
  const long long span = (long long)s.max_len * s.head_dim * (s.dtype == SPC_F32 ? 4 : 2);
  if (span >= (1LL << 31)) return false;
  if (s.dtype == SPC_F32) return s.head_dim == 128 || s.head_dim == 64;
  return s.head_dim == 64 || s.head_dim == 128 || s.head_dim == 256;
}

int score_tile(const spc_shape& s) { return mla_shape(s) ? mla_score_tile(s) : kScoreTile; }

hipError_t launch_scores_normalize(const spc_shape& s, float* probs, const float2* part, const int32_t* lengths,
                                   int ntiles, hipStream_t st) {
  const dim3 g2((s.max_len + kNormChunk - 1) / kNormChunk, s.batch * s.n_q_heads);
  scores_normalize_kernel<<<g2, kThreads, 0, st>>>(probs, part, lengths, s.n_q_heads, s.max_len, ntiles,
                                                   score_tile(s));
  return hipGetLastError();
}

size_t scores_ws_bytes(const spc_shape& s) {
  const size_t ntiles = (size_t)(s.max_len + score_tile(s) - 1) / score_tile(s);
  return (size_t)s.batch * s.n_q_heads * ntiles * sizeof(float2);
}

hipError_t launch_logits(const spc_shape& s, const void* q, const void* k, const int32_t* lengths, float* logits,
                         float2* part, hipStream_t st) {
  if (mla_shape(s)) return launch_mla_logits(s, static_cast<const float*>(q), k, lengths, logits, part, st);
  const int per_kv = s.n_q_heads / s.n_kv_heads;
  const int HC = heads_per_chunk(s);
  const int nchunk = (per_kv + HC - 1) / HC;
  const int ntiles = (s.max_len + kScoreTile - 1) / kScoreTile;
  const dim3 g1(ntiles, s.batch * s.n_kv_heads * nchunk);
  const char* qc = static_cast<const char*>(q);
  const char* kc = static_cast<const char*>(k);
  hipError_t e = hipErrorInvalidValue;
  if (s.dtype == SPC_F32) {
    if (s.head_dim == 128)
      e = launch_logits_hc<SPC_F32, 128>(HC, g1, st, qc, kc, lengths, logits, part, s.n_q_heads, s.n_kv_heads,
                                         s.max_len, nchunk, ntiles, s.scale);
    else if (s.head_dim == 64)
      e = launch_logits_hc<SPC_F32, 64>(HC, g1, st, qc, kc, lengths, logits, part, s.n_q_heads, s.n_kv_heads,
                                        s.max_len, nchunk, ntiles, s.scale);
  } else {
    switch (s.head_dim) {
#define SPC_D(DIM)                                                                                             \
  case DIM:                                                                                                    \
    e = launch_logits_hc<SPC_BF16, DIM>(HC, g1, st, qc, kc, lengths, logits, part, s.n_q_heads, s.n_kv_heads, \
                                        s.max_len, nchunk, ntiles, s.scale);                                   \
    break;
      SPC_D(64)
      SPC_D(128)
      SPC_D(256)
#undef SPC_D
      default:
        break;
    }
  }
  return e;
}

hipError_t launch_scores(const spc_shape& s, const void* q, const void* k, const int32_t* lengths, float* probs,
                         void* ws, hipStream_t st) {
  float2* part = static_cast<float2*>(ws);
  const hipError_t e = launch_logits(s, q, k, lengths, probs, part, st);
  if (e != hipSuccess) return e;
  const int ntiles = (s.max_len + score_tile(s) - 1) / score_tile(s);
  return launch_scores_normalize(s, probs, part, lengths, ntiles, st);
}

}  // namespace spc
