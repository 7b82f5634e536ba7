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
//   (v_mfma_f32_16x16x32_bf16).  Each of 4 waves owns 16 heads; a tile of latent
//   rows is staged in LDS (double-buffered) and shared by the waves.  The float32 query is split
//   into bf16 hi + lo parts (two MFMA passes), which keeps ~16 mantissa bits of
//   the query while the latent rows are bf16 already.  Per-tile (max, sum exp)
//   partials feed the shared normalize kernel of the scores stage.
// mla_out_proj_kernel  out[b][h] = W_UV^h o_lat[b][h] (float32 result).
// mla_expand_kernel    the literal form instead of the absorbed one: the rows a
//   head newly loads are expanded into that head's K/V slots, K = W_UK^h c || r
//   and V = W_UV^h c in bf16 (dense [128 x 512] x [512 x rows] on MFMA), and the
//   head's query is joined as q_nope || q_rope; attention then runs over the
//   slots like any other head.
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMlaD = kMlaLatent + kMlaRope;      // 576 scored dims
constexpr int kKSteps = kMlaD / 32;                // MFMA k-steps of 32
constexpr int kSub = 64;                           // latent rows per LDS buffer: four 16-row blocks
// padded row (elements): two 16-byte pad chunks, so that the 16 rows of a B-fragment read fall on
// distinct banks (with one pad chunk the reads conflicted: 38% of the LDS's busy cycles)
constexpr int kLdsRow = kMlaD + 16;
constexpr int kScoreThreads = 512;                 // 8 waves x 16 heads
constexpr int kScoreHeads = 8 * 16;                // heads per workgroup
constexpr int kScoreRowChunks = kLdsRow / 8;       // 16-byte chunks per padded LDS row (two pad chunks)
constexpr int kScoreChunks = kSub * kScoreRowChunks;
constexpr int kScoreLoads = (kScoreChunks + kWave - 1) / kWave;   // wave loads of 64 chunks per sub-tile
constexpr int kScoreBuf = kScoreLoads * kWave * 8;   // LDS elements of a sub-tile buffer
static_assert(kMlaD % 32 == 0 && kSub == 64, "k-steps of 32; two pairs of 16-row blocks per sub-tile");
static_assert(kMlaScoreTile % kSub == 0 && kMlaScoreTileLarge % kSub == 0, "tiles of whole sub-tiles");

// Workgroup = (quarter of the 512 latent dims, head), so a head's 128 KB of W_UK
// is read by four workgroups.  Lane (g, c) of 16 row groups x 16 chunks holds the
// 16-byte chunk c of the quarter in rows g, g + 16, ...; a lane issues all its row
// loads of a pass (eight rows, every row of a 128-row W_UK) together, and each wave
// load covers 4 rows x 256 contiguous bytes.  Sequences go four at a time; the row
// groups' partial sums meet in LDS.
constexpr int kAbsorbParts = 4;
constexpr int kAbsorbDims = kMlaLatent / kAbsorbParts;   // latent dims per workgroup
constexpr int kAbsorbGroups = 16;                        // row groups (256 threads / 16 chunks)
constexpr int kAbsorbRows = 8;                           // rows per lane per pass
static_assert(kAbsorbDims == 8 * 16, "16 chunks of 8 dims per quarter");

__global__ __launch_bounds__(256) void mla_absorb_kernel(const uint16_t* __restrict__ w_uk,
                                                         const uint16_t* __restrict__ q_nope,
                                                         const uint16_t* __restrict__ q_rope,
                                                         float* __restrict__ q_abs, int B, int H, int dn) {
  const int part = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, c = tid & 15, g = tid >> 4;
  extern __shared__ float smem[];
  float* sq = smem;                                 // [B][dn] query of this head, widened
  float* red = smem + B * dn;                       // [16 row groups][4 sequences][128 dims]
  for (int i = tid; i < B * dn; i += blockDim.x) {
    const int b = i / dn, n = i - (i / dn) * dn;
    sq[i] = __uint_as_float((uint32_t)q_nope[((size_t)b * H + h) * dn + n] << 16);
  }
  __syncthreads();
  const uint16_t* w = w_uk + (size_t)h * dn * kMlaLatent + part * kAbsorbDims + 8 * c;
  for (int b0 = 0; b0 < B; b0 += 4) {
    float acc[4][8];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[bb][e] = 0.f;
    for (int n0 = g; n0 < dn; n0 += kAbsorbGroups * kAbsorbRows) {
      Vec16 wv[kAbsorbRows];
#pragma unroll
      for (int u = 0; u < kAbsorbRows; ++u)
        if (n0 + kAbsorbGroups * u < dn) wv[u] = ld16(w + (size_t)(n0 + kAbsorbGroups * u) * kMlaLatent);
#pragma unroll
      for (int u = 0; u < kAbsorbRows; ++u) {
        const int n = n0 + kAbsorbGroups * u;
        if (n >= dn) break;
        float x[8];
        widen16<SPC_BF16>(wv[u], x);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const float qv = b0 + bb < B ? sq[(b0 + bb) * dn + n] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[bb][e] = fmaf(x[e], qv, acc[bb][e]);
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(g * 4 + bb) * kAbsorbDims + 8 * c + e] = acc[bb][e];
    __syncthreads();
    for (int i = tid; i < 4 * kAbsorbDims; i += blockDim.x) {
      const int bb = i / kAbsorbDims, k = i - bb * kAbsorbDims;
      if (b0 + bb < B) {
        float v = 0.f;
#pragma unroll
        for (int gg = 0; gg < kAbsorbGroups; ++gg) v += red[(gg * 4 + bb) * kAbsorbDims + k];
        q_abs[((size_t)(b0 + bb) * H + h) * kMlaD + part * kAbsorbDims + k] = v;
      }
    }
    __syncthreads();
  }
  if (part == 0) {
    for (int i = tid; i < B * kMlaRope; i += blockDim.x) {
      const int b = i / kMlaRope, r = i - (i / kMlaRope) * kMlaRope;
      q_abs[((size_t)b * H + h) * kMlaD + kMlaLatent + r] =
          __uint_as_float((uint32_t)q_rope[((size_t)b * H + h) * kMlaRope + r] << 16);
    }
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

// Workgroup = (sequence, tile of 256 or 512 positions): 8 waves x 16 heads, one workgroup per CU,
// so the tile is read from memory and staged once for all 128 heads.  A wave keeps the float32
// query of its 16 heads as bf16 hi + lo MFMA A fragments in registers for the whole tile (144
// VGPRs: MFMA A operands live in VGPRs, and 32 heads would not fit).  The tile goes 64 rows at a
// time from memory straight into LDS (global_load_lds_dwordx4: lane l of a wave load lands 16 l
// bytes past the wave's LDS base; rows padded by two 16-byte chunks), double-buffered: the next
// sub-tile is in flight while the MFMAs read the current one, and one barrier per sub-tile
// separates the two.  A sub-tile's logits are stored at the start of the next, so that barrier
// waits only for the next sub-tile's loads.
__global__ __launch_bounds__(kScoreThreads, 1) void mla_scores_kernel(const float* __restrict__ q_abs,
                                                                   const uint16_t* __restrict__ lat,
                                                                   const int32_t* __restrict__ lengths,
                                                                   float* __restrict__ probs,
                                                                   float2* __restrict__ part, int H, int max_len,
                                                                   int ntiles, int tile_len, float scale) {
  __shared__ __align__(16) uint16_t sl[2][kScoreBuf];
  const int tile = blockIdx.x, b = blockIdx.y;
  if (tile >= ntiles) return;
  const int n = clamp_len(lengths, b, max_len);
  const int row0 = tile * tile_len;
  if (row0 >= n) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kc = lane >> 4, col = lane & 15;
  const int hbase = 16 * wid;                      // this wave's heads: hbase .. hbase + 15
  const bool active = hbase < H;                   // H is a multiple of 16

  // query fragments (head hbase + col, k-chunk kc of every k-step), hi and lo parts
  bf16x8_t ahi[kKSteps], alo[kKSteps];
  if (active) {
    const float* qa = q_abs + ((size_t)b * H + hbase + col) * kMlaD;
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

  const uint16_t* lb = lat + (size_t)b * max_len * kMlaD;
  const int nsub = min(tile_len, n - row0 + kSub - 1) / kSub;   // sub-tiles with valid rows
  // sub-tile sub -> LDS buffer: chunk k of the buffer is chunk ch of row r (pad chunks and rows
  // past the sequence load the sequence's row 0; their columns are never written)
  auto dma = [&](int sub, uint16_t* dst) {
    const int p_sub = row0 + sub * kSub;
    for (int i = wid; i < kScoreLoads; i += kScoreThreads / kWave) {
      const int k = kWave * i + lane;
      const int r = k / kScoreRowChunks, ch = k - r * kScoreRowChunks;
      const uint16_t* src = lb;
      if (k < kScoreChunks && ch < kMlaD / 8 && p_sub + r < n) src = lb + (size_t)(p_sub + r) * kMlaD + 8 * ch;
      __builtin_amdgcn_global_load_lds(src, dst + 8 * kWave * i, 16, 0, 0);
    }
  };
  // logits of the last sub-tile: [16-row block][head row i], rows from lpos
  float lv[kSub / 16][4];
  int lpos = -1;
  auto store_held = [&]() {
#pragma unroll
    for (int blk = 0; blk < kSub / 16; ++blk) {
      const int pos = lpos + 16 * blk + col;
      if (pos < n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) probs[((size_t)b * H + hbase + 4 * kc + i) * max_len + pos] = lv[blk][i];
      }
    }
  };
  dma(0, sl[0]);
  __syncthreads();
#pragma unroll 1
  for (int sub = 0; sub < nsub; ++sub) {
    const int buf = sub & 1;
    if (sub + 1 < nsub) dma(sub + 1, sl[buf ^ 1]);   // in flight during this sub-tile's MFMAs
    if (lpos >= 0) store_held();
    const int p_sub = row0 + sub * kSub;
    if (active) {
#pragma unroll
      for (int pr = 0; pr < kSub / 32; ++pr) {
        // two 16-row blocks x (hi, lo): four independent MFMA chains per k-step
        f32x4_t acc[2][2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) acc[blk][0] = acc[blk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const uint16_t* srow = &sl[buf][(32 * pr + col) * kLdsRow + 8 * kc];
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(srow + 32 * s);
          const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(srow + 16 * kLdsRow + 32 * s);
          acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[s], b0, acc[0][0], 0, 0, 0);
          acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[s], b1, acc[1][0], 0, 0, 0);
          acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[s], b0, acc[0][1], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[s], b1, acc[1][1], 0, 0, 0);
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const bool valid = p_sub + 32 * pr + 16 * blk + col < n;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lv[2 * pr + blk][i] = (acc[blk][0][i] + acc[blk][1][i]) * scale;
            if (valid && part) online_ms(m_run[i], s_run[i], lv[2 * pr + blk][i]);
          }
        }
      }
      lpos = p_sub;
    }
    __syncthreads();                                 // the next sub-tile landed; this buffer is free
  }
  if (lpos >= 0) store_held();
  if (active && part) {
    // merge (max, sum) over the 16 lanes of each row group (the tile's positions); part is NULL
    // when the caller wants no tile stats
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float m2 = __shfl_xor(m_run[i], o, kWave);
        const float s2 = __shfl_xor(s_run[i], o, kWave);
        merge_ms(m_run[i], s_run[i], m2, s2);
      }
      if (col == 0) part[((size_t)b * H + hbase + 4 * kc + i) * ntiles + tile] = make_float2(m_run[i], s_run[i]);
    }
  }
}

// Workgroup = (32 output rows, head), so a head's 128 KB of W_UV is read by
// four workgroups.  Eight lanes per row: lane p holds the 16-byte chunks p, p + 8,
// ..., p + 56 of the row (64 latent dims), all eight loads issued together, and
// each wave load covers 8 rows x 128 contiguous bytes.  o_lat of the head sits in
// LDS; the eight lanes' sums meet by butterfly shuffles.
constexpr int kOutRows = 32;                      // output rows per workgroup
__global__ __launch_bounds__(256) void mla_out_proj_kernel(const uint16_t* __restrict__ w_uv,
                                                           const float* __restrict__ o_lat, int64_t lat_b_stride,
                                                           float* __restrict__ out, int B, int H, int dv) {
  const int h = blockIdx.y;
  extern __shared__ float sol[];                    // [B][512]
  for (int i = threadIdx.x; i < B * kMlaLatent; i += blockDim.x) {
    const int b = i / kMlaLatent, k = i - (i / kMlaLatent) * kMlaLatent;
    sol[i] = o_lat[(size_t)b * lat_b_stride + (size_t)h * kMlaLatent + k];
  }
  const int p = threadIdx.x & 7;
  const int r = blockIdx.x * kOutRows + (threadIdx.x >> 3);
  const bool ok = r < dv;
  const uint16_t* wr = w_uv + ((size_t)h * dv + (ok ? r : 0)) * kMlaLatent;
  constexpr int kChunks = kMlaLatent / 8 / 8;       // 16-byte chunks per lane (8)
  Vec16 wv[kChunks];
#pragma unroll
  for (int u = 0; u < kChunks; ++u) wv[u] = ld16(wr + 8 * (p + 8 * u));
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      float x[8];
      widen16<SPC_BF16>(wv[u], x);
      const int k = 8 * (p + 8 * u);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        if (b0 + bb >= B) break;
        const float* o = sol + (b0 + bb) * kMlaLatent + k;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[bb] = fmaf(x[e], o[e], acc[bb]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      float t = acc[bb];
      t += __shfl_xor(t, 1, kWave);
      t += __shfl_xor(t, 2, kWave);
      t += __shfl_xor(t, 4, kWave);
      if (ok && p == 0 && b0 + bb < B) out[((size_t)(b0 + bb) * H + h) * dv + r] = t;
    }
  }
}

}  // namespace

hipError_t launch_mla_absorb(int B, int H, int dn, const void* w_uk, const void* q_nope, const void* q_rope,
                             float* q_abs, hipStream_t st) {
  mla_absorb_kernel<<<dim3(kAbsorbParts, H), 256,
                      ((size_t)B * dn + (size_t)kAbsorbGroups * 4 * kAbsorbDims) * sizeof(float), st>>>(
      static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
      q_abs, B, H, dn);
  return hipGetLastError();
}

namespace {

// One workgroup per (head, part): the head's newly loaded rows of every sequence
// are taken 64 per pass, part p taking passes p, p + 2, ...  Eight waves: wave
// w < 4 owns key dims [32 w, 32 w + 32) (W_UK), wave w >= 4 the same value dims
// (W_UV), and keeps those weight rows in registers as MFMA A fragments for the
// whole kernel (16 k-steps x 2 blocks of 16 dims).  A pass's latent rows go from
// memory straight into LDS (global_load_lds_dwordx4: lane l of a wave load lands
// 16 l bytes past the wave's LDS base), double-buffered: the next pass is in
// flight while this pass's MFMAs read the current one, and no registers hold it.
// Every wave reads the rows as B fragments, so each gathered row is read from
// memory once and yields its K and its V.  The load-list entries of a pass are
// fetched into registers two passes ahead.
// C^T [dims x rows] = W [dims x 512] x latent^T [512 x rows] on
// v_mfma_f32_16x16x32_bf16; a lane ends with 4 consecutive dims of one row,
// rounded to bf16 (nearest even) and stored as 8 bytes.
constexpr int kExpDims = 128;                     // nope and value dims per head
constexpr int kExpOut = kExpDims + kMlaRope + kExpDims;   // slot row: K nope || rope || V
constexpr int kExpKSteps = kMlaLatent / 32;
constexpr int kExpThreads = 512;                  // 8 waves: 4 on K, 4 on V
constexpr int kExpRows = 64;                      // rows per pass
constexpr int kExpRowChunks = kMlaLatent / 8 + 1; // 16-byte chunks per padded LDS row (one pad chunk)
constexpr int kExpLRow = kExpRowChunks * 8;       // padded LDS row (elements): fragment rows on distinct banks
constexpr int kExpChunks = kExpRows * kExpRowChunks;
constexpr int kExpLoads = (kExpChunks + kWave - 1) / kWave;   // wave loads of 64 chunks per pass
constexpr int kExpBuf = kExpLoads * kWave * 8;    // LDS elements of a pass buffer

__global__ __launch_bounds__(kExpThreads, 1) void mla_expand_kernel(
    const uint16_t* __restrict__ lat, const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope, const int32_t* __restrict__ load_pos,
    const int32_t* __restrict__ load_slot, const int32_t* __restrict__ load_count, uint16_t* __restrict__ kv,
    uint16_t* __restrict__ q_exp, int B, int H, int max_len, int K) {
  __shared__ __align__(16) uint16_t sa[kExpBuf];
  __shared__ __align__(16) uint16_t sb[kExpBuf];
  __shared__ int s_pref[kMlaMaxBatch + 1];
  __shared__ int s_b[2][kExpRows];                 // sequence of a pass row, or -1
  __shared__ int s_pos[2][kExpRows];
  __shared__ int s_slot[2][kExpRows];
  const int h = blockIdx.x >> 1, part = blockIdx.x & 1;
  if (h >= H) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, col = lane & 15, kc = lane >> 4;
  const bool isv = wid >= 4;
  const int d0 = 32 * (wid & 3);
  bf16x8_t a[2][kExpKSteps];                      // this wave's weight rows, for the whole kernel
  {
    const uint16_t* w = (isv ? w_uv : w_uk) + ((size_t)h * kExpDims + d0) * kMlaLatent;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int s = 0; s < kExpKSteps; ++s)
        a[db][s] = *reinterpret_cast<const bf16x8_t*>(w + (size_t)(16 * db + col) * kMlaLatent + 32 * s + 8 * kc);
  }
  if (tid == 0) {
    int acc = 0;
    for (int b = 0; b < B; ++b) {
      s_pref[b] = acc;
      const int c = load_count[(size_t)b * H + h];
      acc += c < 0 ? 0 : (c > K ? K : c);
    }
    s_pref[B] = acc;
  }
  if (part == 0 && q_exp != nullptr) {             // the head's query against the expanded keys
    for (int i = tid; i < B * (kExpDims + kMlaRope); i += kExpThreads) {
      const int b = i / (kExpDims + kMlaRope), d = i - b * (kExpDims + kMlaRope);
      q_exp[((size_t)b * H + h) * (kExpDims + kMlaRope) + d] =
          d < kExpDims ? q_nope[((size_t)b * H + h) * kExpDims + d]
                       : q_rope[((size_t)b * H + h) * kMlaRope + (d - kExpDims)];
    }
  }
  __syncthreads();
  const int R = s_pref[B];
  const int npass = (R + kExpRows - 1) / kExpRows;
  int p = part;
  if (p >= npass) return;                          // uniform: no barrier follows for this workgroup

  // a pass's load-list entries: fetched by 64 threads into registers, published to LDS later
  int e_b = -1, e_pos = 0, e_slot = 0;
  auto fetch = [&](int pass) {
    e_b = -1;
    if (tid < kExpRows) {
      const int rr = pass * kExpRows + tid;
      if (rr < R) {
        int b = 0;
        for (int j = 1; j < B; ++j) b += rr >= s_pref[j];
        const size_t li = ((size_t)b * H + h) * K + (rr - s_pref[b]);
        e_pos = load_pos[li];
        e_slot = load_slot[li];
        e_b = b;
      }
    }
  };
  auto publish = [&](int buf) {
    if (tid < kExpRows) {
      const bool ok = e_b >= 0 && e_pos >= 0 && e_pos < max_len && e_slot >= 0 && e_slot < K;
      s_b[buf][tid] = ok ? e_b : -1;
      s_pos[buf][tid] = ok ? e_pos : 0;
      s_slot[buf][tid] = ok ? e_slot : 0;
    }
  };
  // the rows of the entries in s_*[buf] -> LDS (pad chunks and empty rows load latent row 0)
  auto dma = [&](int buf, uint16_t* dst) {
    for (int i = wid; i < kExpLoads; i += kExpThreads / kWave) {
      const int k = kWave * i + lane;
      const int r = k / kExpRowChunks, ch = k - r * kExpRowChunks;
      const uint16_t* src = lat;
      if (k < kExpChunks && ch < kMlaLatent / 8) {
        const int b = s_b[buf][r];
        if (b >= 0) src = lat + ((size_t)b * max_len + s_pos[buf][r]) * (kMlaLatent + kMlaRope) + 8 * ch;
      }
      __builtin_amdgcn_global_load_lds(src, dst + 8 * kWave * i, 16, 0, 0);
    }
  };
  auto pass_body = [&](int buf, const uint16_t* rows) {
    f32x4_t acc[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) { acc[rb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f}; acc[rb][1] = acc[rb][0]; }
#pragma unroll
    for (int s = 0; s < kExpKSteps; ++s) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(rows + (16 * rb + col) * kExpLRow + 32 * s + 8 * kc);
        acc[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][s], bf, acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][s], bf, acc[rb][1], 0, 0, 0);
      }
    }
    // lane (col, kc): dims d0 + 16 db + 4 kc .. + 3 of row 16 rb + col
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = 16 * rb + col;
      const int b = s_b[buf][row];
      if (b < 0) continue;
      uint16_t* dst = kv + (((size_t)b * H + h) * K + s_slot[buf][row]) * kExpOut;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const uint2 w2 = make_uint2(bf16_bits(acc[rb][db][0]) | (bf16_bits(acc[rb][db][1]) << 16),
                                    bf16_bits(acc[rb][db][2]) | (bf16_bits(acc[rb][db][3]) << 16));
        *reinterpret_cast<uint2*>(dst + (isv ? kExpDims + kMlaRope : 0) + d0 + 16 * db + 4 * kc) = w2;
      }
      if (!isv && rb == (wid & 3)) {               // the rotary dims of the row, copied as they are
        const uint16_t* src = lat + ((size_t)b * max_len + s_pos[buf][row]) * (kMlaLatent + kMlaRope) + kMlaLatent;
        *reinterpret_cast<uint4*>(dst + kExpDims + 8 * kc) = *reinterpret_cast<const uint4*>(src + 8 * kc);
        *reinterpret_cast<uint4*>(dst + kExpDims + 8 * (kc + 4)) = *reinterpret_cast<const uint4*>(src + 8 * (kc + 4));
      }
    }
  };

  fetch(p);
  publish(0);
  if (p + 2 < npass) fetch(p + 2);
  __syncthreads();
  dma(0, sa);
  publish(1);                                      // entries of pass p + 2 (unused if there is none)
  __syncthreads();                                 // pass p's rows are in sa
#pragma unroll 1
  for (;;) {
    // even step: rows of pass p in sa (entries s_*[0]); pass p + 2 (entries s_*[1]) -> sb
    bool more = p + 2 < npass;
    if (more) dma(1, sb);
    if (p + 4 < npass) fetch(p + 4);
    pass_body(0, sa);
    __syncthreads();                               // sb loaded; sa and s_*[0] free
    if (!more) break;
    publish(0);                                    // entries of pass p + 4
    __syncthreads();
    p += 2;
    // odd step: rows of pass p in sb (entries s_*[1]); pass p + 2 (entries s_*[0]) -> sa
    more = p + 2 < npass;
    if (more) dma(0, sa);
    if (p + 4 < npass) fetch(p + 4);
    pass_body(1, sb);
    __syncthreads();
    if (!more) break;
    publish(1);
    __syncthreads();
    p += 2;
  }
}

}  // namespace

// 512-position tiles halve the workgroups and the query-fragment setup per position; they are
// taken when the grid still holds a workgroup for each of the 256 CUs
int mla_score_tile(const spc_shape& s) {
  const long wgs = (long)s.batch * ((s.max_len + kMlaScoreTileLarge - 1) / kMlaScoreTileLarge);
  return wgs >= 256 ? kMlaScoreTileLarge : kMlaScoreTile;
}

hipError_t launch_mla_logits(const spc_shape& s, const float* q_abs, const void* latent, const int32_t* lengths,
                             float* logits, float2* stats, hipStream_t st) {
  if (s.n_q_heads > kScoreHeads || s.n_q_heads % 16 != 0) return hipErrorInvalidValue;
  const int tl = mla_score_tile(s);
  const int ntiles = (s.max_len + tl - 1) / tl;
  mla_scores_kernel<<<dim3(ntiles, s.batch), kScoreThreads, 0, st>>>(
      q_abs, static_cast<const uint16_t*>(latent), lengths, logits, stats, s.n_q_heads, s.max_len, ntiles, tl,
      s.scale);
  return hipGetLastError();
}

hipError_t launch_mla_expand(const spc_shape& s, const void* latent, const void* w_uk, const void* w_uv,
                             const void* q_nope, const void* q_rope, const int32_t* load_pos,
                             const int32_t* load_slot, const int32_t* load_count, void* kv_exp, void* q_exp,
                             hipStream_t st) {
  mla_expand_kernel<<<dim3(2 * s.n_q_heads), kExpThreads, 0, st>>>(
      static_cast<const uint16_t*>(latent), static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
      static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope), load_pos, load_slot, load_count,
      static_cast<uint16_t*>(kv_exp), static_cast<uint16_t*>(q_exp), s.batch, s.n_q_heads, s.max_len, s.budget);
  return hipGetLastError();
}

hipError_t launch_mla_out_proj(int B, int H, int dv, const void* w_uv, const float* o_lat, int64_t lat_b_stride,
                               float* out, hipStream_t st) {
  mla_out_proj_kernel<<<dim3((dv + kOutRows - 1) / kOutRows, H), 256, (size_t)B * kMlaLatent * sizeof(float), st>>>(
      static_cast<const uint16_t*>(w_uv), o_lat, lat_b_stride, out, B, H, dv);
  return hipGetLastError();
}

}  // namespace spc
