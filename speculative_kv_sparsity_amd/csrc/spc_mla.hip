// MLA (multi-head latent attention) pieces of the path.
//
// The KV cache holds one low-dimensional latent row per position, c_j (512) || r_j
// (64 rotary dims), shared by all heads.  Head-level retrieval scores the latent
// cache per head, Top-K selects per head, and only the selected latent rows
// enter attention (SpeContext blog section 5, last paragraph; paper summary
// section 4.3, MLA bullet).  Here the per-head up-projections are absorbed into
// the query and the output, which is exact in real arithmetic:
//   q_h . (W_UK^h c_j || r_j) = (W_UK^h^T q_nope_h || q_rope_h) . (c_j || r_j)
//   sum_j w_j W_UV^h c_j      = W_UV^h (sum_j w_j c_j)
//
// mla_absorb_kernel    q_abs[b][h] = (W_UK^h^T q_nope[b][h]) || q_rope[b][h], float32.
// mla_scores_kernel    logits[b][h][j] = scale * q_abs[b][h] . latent[b][j] for all 128
//   heads at once: a dense [heads x 576] x [576 x positions] contraction on MFMA
//   (v_mfma_f32_16x16x32_bf16).  Each of 8 waves owns 16 heads; a tile of latent
//   rows is staged in LDS and shared by the waves.  The float32 query is split
//   into bf16 hi + lo parts (two MFMA passes), which keeps ~16 mantissa bits of
//   the query while the latent rows are bf16 already.  Per-tile (max, sum exp)
//   partials feed the shared normalize kernel of the scores stage.
// mla_out_proj_kernel  out[b][h] = W_UV^h o_lat[b][h] (float32 result).
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMlaD = kMlaLatent + kMlaRope;      // 576 scored dims
constexpr int kKSteps = kMlaD / 32;                // MFMA k-steps of 32
constexpr int kSub = 64;                           // latent rows staged in LDS at a time
constexpr int kLdsRow = kMlaD + 8;                 // padded row (elements): spreads rows over banks
constexpr int kScoreThreads = 512;                 // 8 waves x 16 heads
static_assert(kMlaD % 32 == 0, "k-steps of 32");

__global__ __launch_bounds__(256) void mla_absorb_kernel(const uint16_t* __restrict__ w_uk,
                                                         const uint16_t* __restrict__ q_nope,
                                                         const uint16_t* __restrict__ q_rope,
                                                         float* __restrict__ q_abs, int B, int H, int dn) {
  const int h = blockIdx.x;
  extern __shared__ float sq[];                    // [B][dn] query of this head, widened
  for (int i = threadIdx.x; i < B * dn; i += blockDim.x) {
    const int b = i / dn, n = i - (i / dn) * dn;
    sq[i] = __uint_as_float((uint32_t)q_nope[((size_t)b * H + h) * dn + n] << 16);
  }
  __syncthreads();
  const uint16_t* w = w_uk + (size_t)h * dn * kMlaLatent;
  for (int k = threadIdx.x; k < kMlaLatent; k += blockDim.x) {
    float acc[kMlaMaxBatch];
#pragma unroll
    for (int b = 0; b < kMlaMaxBatch; ++b) acc[b] = 0.f;
    for (int n = 0; n < dn; ++n) {
      const float wv = __uint_as_float((uint32_t)w[(size_t)n * kMlaLatent + k] << 16);
#pragma unroll
      for (int b = 0; b < kMlaMaxBatch; ++b)
        if (b < B) acc[b] = fmaf(wv, sq[b * dn + n], acc[b]);
    }
#pragma unroll
    for (int b = 0; b < kMlaMaxBatch; ++b)
      if (b < B) q_abs[((size_t)b * H + h) * kMlaD + k] = acc[b];
  }
  for (int i = threadIdx.x; i < B * kMlaRope; i += blockDim.x) {
    const int b = i / kMlaRope, r = i - (i / kMlaRope) * kMlaRope;
    q_abs[((size_t)b * H + h) * kMlaD + kMlaLatent + r] =
        __uint_as_float((uint32_t)q_rope[((size_t)b * H + h) * kMlaRope + r] << 16);
  }
}

__device__ __forceinline__ void online_ms(float& m, float& s, float x) {
  const float mn = fmaxf(m, x);
  s = s * __expf(m - mn) + __expf(x - mn);
  m = mn;
}

__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = (m == -INFINITY ? 0.f : s * __expf(m - M)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - M));
  m = M;
}

__global__ __launch_bounds__(kScoreThreads) void mla_scores_kernel(const float* __restrict__ q_abs,
                                                                   const uint16_t* __restrict__ lat,
                                                                   const int32_t* __restrict__ lengths,
                                                                   float* __restrict__ probs,
                                                                   float2* __restrict__ part, int H, int max_len,
                                                                   int ntiles, float scale) {
  __shared__ uint16_t sl[kSub * kLdsRow];
  const int b = blockIdx.y, tile = blockIdx.x;
  const int n = clamp_len(lengths, b, max_len);
  const int row0 = tile * kScoreTile;
  if (row0 >= n) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nw = H / 16;                           // waves that own heads
  const int kc = lane >> 4, col = lane & 15;

  // this lane's query fragments (head 16*wid + col, k-chunk kc of every k-step), hi and lo parts
  bf16x8_t ahi[kKSteps], alo[kKSteps];
  if (wid < nw) {
    const float* qa = q_abs + ((size_t)b * H + 16 * wid + col) * kMlaD;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const float4 x0 = *reinterpret_cast<const float4*>(qa + 32 * s + 8 * kc);
      const float4 x1 = *reinterpret_cast<const float4*>(qa + 32 * s + 8 * kc + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hi = (__bf16)x[e];
        ahi[s][e] = hi;
        alo[s][e] = (__bf16)(x[e] - (float)hi);
      }
    }
  }
  float m_run[4], s_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }

  constexpr int kChunks = kMlaD * 2 / 16;          // 16-byte chunks per latent row
  const uint16_t* lb = lat + (size_t)b * max_len * kMlaD;
#pragma unroll 1
  for (int sub = 0; sub < kScoreTile / kSub; ++sub) {
    const int p_sub = row0 + sub * kSub;
    if (p_sub >= n) break;
    __syncthreads();                               // previous sub-tile fully consumed
    constexpr int kPer = kSub * kChunks / kScoreThreads;
    uint4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + u * kScoreThreads;
      const int r = c / kChunks, ch = c - (c / kChunks) * kChunks;
      v[u] = p_sub + r < n ? *reinterpret_cast<const uint4*>(lb + (size_t)(p_sub + r) * kMlaD + 8 * ch)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + u * kScoreThreads;
      const int r = c / kChunks, ch = c - (c / kChunks) * kChunks;
      *reinterpret_cast<uint4*>(&sl[r * kLdsRow + 8 * ch]) = v[u];
    }
    __syncthreads();
    if (wid < nw) {
#pragma unroll 1
      for (int blk = 0; blk < kSub / 16; ++blk) {
        const int p0 = p_sub + 16 * blk;
        if (p0 >= n) break;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* srow = &sl[(16 * blk + col) * kLdsRow + 8 * kc];
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          const bf16x8_t bfrag = *reinterpret_cast<const bf16x8_t*>(srow + 32 * s);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[s], bfrag, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[s], bfrag, acc, 0, 0, 0);
        }
        const int pos = p0 + col;
        if (pos < n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = 16 * wid + 4 * kc + i;
            const float l = acc[i] * scale;
            probs[((size_t)b * H + h) * max_len + pos] = l;
            online_ms(m_run[i], s_run[i], l);
          }
        }
      }
    }
  }
  if (wid < nw) {
    // merge (max, sum) over the 16 lanes of each row group (the tile's positions)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float m2 = __shfl_xor(m_run[i], o, kWave);
        const float s2 = __shfl_xor(s_run[i], o, kWave);
        merge_ms(m_run[i], s_run[i], m2, s2);
      }
      if (col == 0) part[((size_t)b * H + 16 * wid + 4 * kc + i) * ntiles + tile] = make_float2(m_run[i], s_run[i]);
    }
  }
}

// One workgroup per head; wave w handles output rows w, w+4, ...; a lane holds 8
// contiguous latent dims of the row.
__global__ __launch_bounds__(256) void mla_out_proj_kernel(const uint16_t* __restrict__ w_uv,
                                                           const float* __restrict__ o_lat, int64_t lat_b_stride,
                                                           float* __restrict__ out, int B, int H, int dv) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  static_assert(kMlaLatent == 8 * kWave, "one 16-byte chunk of the latent per lane");
  float ol[kMlaMaxBatch][8];
#pragma unroll
  for (int b = 0; b < kMlaMaxBatch; ++b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ol[b][e] = 0.f;
    if (b < B) {
      const float* src = o_lat + (size_t)b * lat_b_stride + (size_t)h * kMlaLatent + 8 * lane;
#pragma unroll
      for (int e = 0; e < 8; ++e) ol[b][e] = src[e];
    }
  }
  for (int r = wid; r < dv; r += 4) {
    const Vec16 wv = ld16(w_uv + ((size_t)h * dv + r) * kMlaLatent + 8 * lane);
    float x[8];
    widen16<SPC_BF16>(wv, x);
    for (int b = 0; b < B; ++b) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(x[e], ol[b][e], a);
      a = wave_sum(a);
      if (lane == 0) out[((size_t)b * H + h) * dv + r] = a;
    }
  }
}

}  // namespace

hipError_t launch_mla_absorb(int B, int H, int dn, const void* w_uk, const void* q_nope, const void* q_rope,
                             float* q_abs, hipStream_t st) {
  mla_absorb_kernel<<<dim3(H), 256, (size_t)B * dn * sizeof(float), st>>>(
      static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
      q_abs, B, H, dn);
  return hipGetLastError();
}

hipError_t launch_mla_scores(const spc_shape& s, const float* q_abs, const void* latent, const int32_t* lengths,
                             float* probs, void* ws, hipStream_t st) {
  const int ntiles = (s.max_len + kScoreTile - 1) / kScoreTile;
  float2* part = static_cast<float2*>(ws);
  mla_scores_kernel<<<dim3(ntiles, s.batch), kScoreThreads, 0, st>>>(
      q_abs, static_cast<const uint16_t*>(latent), lengths, probs, part, s.n_q_heads, s.max_len, ntiles, s.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_scores_normalize(s, probs, part, lengths, ntiles, st);
}

hipError_t launch_mla_out_proj(int B, int H, int dv, const void* w_uv, const float* o_lat, int64_t lat_b_stride,
                               float* out, hipStream_t st) {
  mla_out_proj_kernel<<<dim3(H), 256, 0, st>>>(static_cast<const uint16_t*>(w_uv), o_lat, lat_b_stride, out, B, H,
                                                dv);
  return hipGetLastError();
}

}  // namespace spc
