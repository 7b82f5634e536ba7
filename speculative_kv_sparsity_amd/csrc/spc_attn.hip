// Stage 4 - sparse decode attention over the resident sparse KV only.
//
//   out[b][l][i] = sum_r softmax_r(scale * q_l[b][i] . K[r]) V[r]
// over the rows r of query head i's group (SpeContext blog section 4:
// llm.forward(..., sparse_kv=resident_kv); AttentionWeight formula of blog
// section 2).
//
// attn_split_kernel  split-K: one workgroup per (b, layer, group, head chunk,
//   split of 64 or 128 rows).  The GQC query heads of the chunk share every
//   K/V row read.  Every lane issues ALL of its K and V loads up front, so a
//   workgroup has its whole tile in flight at once.  The loads go through
//   buffer resources over the head's rows: a padding row (empty slot, past the
//   count) gets an offset past the range and reads zeros, so no load waits
//   behind a branch.  They are nontemporal (each row is read once per step).
//     K: 8 lanes per row (lane p holds the 16-byte chunks p, p+8, ...; one wave
//        load covers 8 rows x 128 contiguous bytes); v_dot2_f32_bf16 on packed
//        pairs and DPP 8-lane sums give every lane of the group the logits.
//     softmax: each wave keeps its own max per head; the exp weights of its
//        rows go to LDS.
//     V: 32 lanes per row, each lane owning d/32 fixed output dims; the two
//        wave halves take alternate rows, so one permlane swap finishes the
//        wave's sums, and the four waves are merged through LDS with their
//        max-rescaling.
//   Writes the split's (max, sum) and unnormalised output per head.
// attn_split_latent_kernel  the same for MLA latent rows, where V is the first
//   v_dim elements of the K row (read once, used twice) and one head per group.
// attn_combine_kernel  merges the splits of every head with their log-sum-exp
//   weights into the float32 output (one workgroup per head).
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kLatentTilesSmall = 4;          // MLA: 16-row tiles per wave and split (few instances)
constexpr int kLatentTilesLarge = 16;         // (enough instances x splits to fill the chip)
constexpr int kLatentTilesWhole = 32;         // (a budget of <= 2048 rows in one split per head)
constexpr int kSplitRowsWide = 160;           // the wider splits of split_rows (5 iterations of 8 rows per wave)

struct QL { int64_t b, layer, head; };        // byte strides
struct KL { int64_t b, layer, head, row, kv; };

// Loads of 4, 8 or 16 bytes for the V layout, through a buffer resource (zeros past its range),
// nontemporal: the split kernel reads each slot row once per step.
template <int BYTES> struct VLoad;
template <> struct VLoad<4> {
  uint32_t w[1];
  __device__ __forceinline__ void load_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kLoadNontemporal);
  }
};
template <> struct VLoad<8> {
  uint32_t w[2];
  __device__ __forceinline__ void load_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kLoadNontemporal);
    w[0] = (uint32_t)v.x; w[1] = (uint32_t)v.y;
  }
};
template <> struct VLoad<16> {
  uint32_t w[4];
  __device__ __forceinline__ void load_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const Vec16 v = ld16_buffer<kLoadNontemporal>(r, off);
    w[0] = v.w[0]; w[1] = v.w[1]; w[2] = v.w[2]; w[3] = v.w[3];
  }
};

template <int DT, int N>
__device__ __forceinline__ void widen_words(const uint32_t* w, float* out) {
  if (DT == SPC_BF16) {
#pragma unroll
    for (int i = 0; i < N; ++i) { out[2 * i] = bf_lo(w[i]); out[2 * i + 1] = bf_hi(w[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = __uint_as_float(w[i]);
  }
}

// Row ids of a split: -1 for an empty slot / invalid position / past the count.
__device__ __forceinline__ int32_t split_row(const int32_t* rl, int idx, int cnt, int mode, int max_rows) {
  if (idx >= cnt) return -1;
  const int32_t v = rl[idx];
  return mode == SPC_ROWS_SLOTS ? (v >= 0 ? idx : -1) : (v >= 0 && v < max_rows ? v : -1);
}

// NI: K iterations of 8 rows per wave (rows per wave = 8 NI).  D: key width, DV: value width.
template <int DT, int D, int DV, int GQC, int NI>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(
    const char* __restrict__ q, QL ql, const char* __restrict__ kv, KL kl, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ row_count, int mode, int Hq, int Hkv, int n_groups, int K, int layer_begin,
    int n_lay, int nsplit, int nhc, int max_rows, float scale, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
  constexpr int EB = DT == SPC_BF16 ? 2 : 4;
  constexpr int CPLK = D * EB / 16 / 8;              // K: 16-byte chunks per lane
  constexpr int RPW = 8 * NI;                        // rows per wave
  constexpr int RPS = 4 * RPW;                       // rows per split
  constexpr int EPL = DV / 32;                       // V: dims per lane
  constexpr int VB = EPL * EB;                       // V: bytes per lane and row
  constexpr int NV = RPW / 2;                        // V: rows per lane
  static_assert(D * EB % 128 == 0 && DV % 32 == 0, "row layout");

  const int split = blockIdx.x;
  const int hcix = blockIdx.z;
  const int inst = blockIdx.y;                       // ((b * n_lay + lo) * n_groups + r)
  const int r = inst % n_groups;
  const int bl = inst / n_groups;
  const int lo = bl % n_lay;
  const int b = bl / n_lay;
  const int layer = layer_begin + lo;
  const int GQ = Hq / n_groups;
  const int h0 = r * GQ + hcix * GQC;
  const int kvh = h0 / (Hq / Hkv);                   // the chunk's heads share one KV head

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int p = lane & 7, rr = lane >> 3;
  const int half = lane >> 5, vl = lane & 31;

  __shared__ int32_t sRow[RPS];
  __shared__ float sW[4][RPW][GQC];
  __shared__ float s_m[4][GQC], s_l[4][GQC];
  __shared__ float red[4][GQC][DV];

  const int32_t* rl = rows + ((size_t)b * n_groups + r) * K;
  int cnt = K;
  if (mode == SPC_ROWS_GATHER) {
    cnt = row_count[(size_t)b * n_groups + r];
    cnt = cnt < 0 ? 0 : (cnt > K ? K : cnt);
  }
  const int i0 = split * RPS;
  for (int i = tid; i < RPS; i += kThreads) sRow[i] = split_row(rl, i0 + i, cnt, mode, max_rows);
  __syncthreads();

  const char* kbase = kv + b * kl.b + layer * kl.layer + (int64_t)kvh * kl.head;
  // buffer resources over the head's key rows and value rows (the host keeps each under 2 GiB):
  // a padding row's offset lies past the range and reads zeros, with no branch
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(kbase), (short)0, (int)((int64_t)max_rows * kl.row), kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(kbase + kl.kv), (short)0, (int)((int64_t)max_rows * kl.row), kBufferRsrcWord3);
  const int wrow = wid * RPW;                        // first row of this wave within the split
  int32_t rowk[NI];
  Vec16 kc[NI][CPLK];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    rowk[it] = sRow[wrow + it * 8 + rr];
    const uint32_t off = rowk[it] >= 0 ? (uint32_t)rowk[it] * (uint32_t)kl.row + 16u * p : kBufferOutOfRange;
#pragma unroll
    for (int c = 0; c < CPLK; ++c) kc[it][c] = ld16_buffer<kLoadNontemporal>(krs, off + 128u * c);
  }
  int32_t rowv[NV];
  VLoad<VB> vv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    rowv[i] = sRow[wrow + 2 * i + half];
    const uint32_t off = rowv[i] >= 0 ? (uint32_t)rowv[i] * (uint32_t)kl.row + vl * VB : kBufferOutOfRange;
    vv[i].load_buffer(vrs, off);
  }
  Vec16 qv[GQC][CPLK];
#pragma unroll
  for (int h = 0; h < GQC; ++h) {
    const char* qh = q + b * ql.b + layer * ql.layer + (int64_t)(h0 + h) * ql.head;
#pragma unroll
    for (int c = 0; c < CPLK; ++c) qv[h][c] = ld16(qh + (p + 8 * c) * 16);
  }

  // logits (every lane of an 8-lane group holds its row's logits for all heads)
  float lg[NI][GQC];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
#pragma unroll
    for (int h = 0; h < GQC; ++h) {
      float a = 0.f;
      if (rowk[it] >= 0) {
#pragma unroll
        for (int c = 0; c < CPLK; ++c) a = dot16<DT>(kc[it][c], qv[h][c], a);
      }
      a = sum8(a);
      lg[it][h] = rowk[it] >= 0 ? a * scale : -INFINITY;
    }
  }
  // per-wave max, exp weights to LDS, per-wave sums
  float mw[GQC], lw[GQC];
#pragma unroll
  for (int h = 0; h < GQC; ++h) {
    float m = -INFINITY;
#pragma unroll
    for (int it = 0; it < NI; ++it) m = fmaxf(m, lg[it][h]);
    mw[h] = max_across_rows8(m);
    float sum = 0.f;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const float e = lg[it][h] == -INFINITY ? 0.f : __expf(lg[it][h] - mw[h]);
      lg[it][h] = e;
      sum += e;
    }
    lw[h] = sum_across_rows8(sum);
  }
  if (p == 0) {
#pragma unroll
    for (int it = 0; it < NI; ++it)
#pragma unroll
      for (int h = 0; h < GQC; ++h) sW[wid][it * 8 + rr][h] = lg[it][h];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQC; ++h) { s_m[wid][h] = mw[h]; s_l[wid][h] = lw[h]; }
  }
  __syncthreads();

  // weighted V rows: lane (half, vl) accumulates dims vl*EPL .. +EPL of rows 2i + half
  float acc[GQC][EPL];
#pragma unroll
  for (int h = 0; h < GQC; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (rowv[i] >= 0) {
      float x[EPL];
      widen_words<DT, VB / 4>(vv[i].w, x);
#pragma unroll
      for (int h = 0; h < GQC; ++h) {
        const float w = sW[wid][2 * i + half][h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w, x[e], acc[h][e]);
      }
    }
  }
  // merge the halves, then the waves (rescaled to the workgroup max)
  float fw[GQC];
#pragma unroll
  for (int h = 0; h < GQC; ++h) {
    const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    fw[h] = mw[h] == -INFINITY ? 0.f : __expf(mw[h] - M);
  }
#pragma unroll
  for (int h = 0; h < GQC; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = add_xor32(acc[h][e]);
  if (half == 0) {
#pragma unroll
    for (int h = 0; h < GQC; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wid][h][vl * EPL + e] = acc[h][e] * fw[h];
  }
  __syncthreads();
  const size_t pbase = ((size_t)inst * nhc + hcix) * nsplit + split;
  for (int t = tid; t < GQC * DV; t += kThreads) {
    const int h = t / DV, d = t - (t / DV) * DV;
    part_o[(pbase * GQC + h) * DV + d] = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
  }
  if (tid < GQC) {
    const int h = tid;
    const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) L += s_m[w][h] == -INFINITY ? 0.f : s_l[w][h] * __expf(s_m[w][h] - M);
    }
    part_ml[pbase * GQC + h] = make_float2(M, L);
  }
}

// MLA latent rows: V is the first DV elements of the K row; one head per group; the
// query is the float32 absorbed query (q_l strides in float32 elements).
//
// The per-row work is a GEMV on both sides (576 dims against the query, 512 dims
// into the output), so the kernel keeps it on packed bf16 dot products:
//   logits: the float32 query is held as a bf16 pair (hi + lo, ~16 mantissa bits);
//     v_dot2_f32_bf16 of a packed pair of latent elements with the hi and with the
//     lo pair gives two MACs per instruction with no widening of the row.
//   output: the two rows a lane holds in a tile are interleaved per element with
//     v_perm_b32 (row0[d], row1[d]), and dot2 against the pair of their weights
//     (again hi + lo bf16) adds both rows' contributions to dims d at once.
// Each wave walks T tiles of 16 rows (8 lanes per row, 2 rows per lane) with an
// online softmax, so the 8-lane-group reduction and the cross-wave merge are paid
// once per 64 T rows instead of once per 16.
//
// A selected row is read by several heads of its sequence (about 8 of 128 at 32K positions and a
// budget of 2048), so the grid is one-dimensional and ordered for the L2 of each XCD: the
// dispatcher deals block ids round-robin over the 8 XCDs, and the ids of XCD x run, in order,
// every head of (sequence, layer, split) groups x, x + 8, ... .  The heads of a group in flight
// together on one XCD walk their ascending row lists at about the same pace, so a row one of
// them reads is often still in that L2 for the others.
//
// With fewer than 8 such groups (n_glob = 1, 2 or 4: `parts` = 8 / n_glob), each group is shared by
// `parts` XCDs, each taking a contiguous range of its heads, so that no XCD idles.  FIN: the head
// has one split, and the workgroup writes the normalised output itself (no merge launch); PROJ (with
// FIN): it writes the head's output projection instead, W_UV[head] (bf16 [dv][DV]) times the
// normalised output held in LDS, two threads per output row.
template <int D, int DV, int T, bool FIN, bool PROJ>
__global__ __launch_bounds__(kThreads) void attn_split_latent_kernel(
    const char* __restrict__ q, QL ql, const char* __restrict__ kv, KL kl, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ row_count, int mode, int Hq, int Hkv, int n_groups, int K, int layer_begin,
    int n_lay, int nsplit, int n_glob, int parts, int max_rows, float scale, float* __restrict__ part_o,
    float2* __restrict__ part_ml, float* __restrict__ out, int n_layers, const uint16_t* __restrict__ w_uv, int dv) {
  static_assert(FIN || !PROJ, "the projection needs the whole output of the head");
  constexpr int EB = 2;
  constexpr int CPLK = D * EB / 16 / 8;              // 16-byte chunks per lane of a row (9)
  constexpr int CPLV = DV * EB / 16 / 8;             // of them in the value part (8)
  constexpr int RPT = 16;                            // rows per wave tile (8 lanes per row, 2 rows per lane)
  constexpr int RPS = 4 * RPT * T;
  static_assert(CPLV <= CPLK && D * EB % 128 == 0 && DV * EB % 128 == 0, "latent row layout");
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  int r, gidx;                                         // head (one per group); (sequence, layer, split) group
  if (parts > 1) {
    const int hpp = (n_groups + parts - 1) / parts;
    gidx = xcd % n_glob;
    r = (xcd / n_glob) * hpp + j;
    if (j >= hpp || r >= n_groups) return;
  } else {
    r = j % n_groups;
    gidx = (j / n_groups) * 8 + xcd;
  }
  if (gidx >= n_glob) return;
  const int split = gidx % nsplit;
  const int bl = gidx / nsplit;
  const int inst = bl * n_groups + r;
  const int lo = bl % n_lay;
  const int b = bl / n_lay;
  const int layer = layer_begin + lo;
  const int kvh = r / (n_groups / Hkv);
  const int head = r * (Hq / n_groups);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int p = lane & 7, rr = lane >> 3;
  __shared__ int32_t sRow[RPS];
  __shared__ float s_m[4], s_l[4];
  __shared__ float red[4][DV];
  const int32_t* rl = rows + ((size_t)b * n_groups + r) * K;
  int cnt = K;
  if (mode == SPC_ROWS_GATHER) {
    cnt = row_count[(size_t)b * n_groups + r];
    cnt = cnt < 0 ? 0 : (cnt > K ? K : cnt);
  }
  const int i0 = split * RPS;
  for (int i = tid; i < RPS; i += kThreads) sRow[i] = split_row(rl, i0 + i, cnt, mode, max_rows);
  __syncthreads();
  const char* kbase = kv + b * kl.b + layer * kl.layer + (int64_t)kvh * kl.head;
  // a buffer resource over the head's rows (the host keeps them under 2 GiB)
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(kbase), (short)0, (int)((int64_t)max_rows * kl.row), kBufferRsrcWord3);

  // query chunk p + 8c as hi / lo bf16 pairs
  uint32_t qhi[CPLK][4], qlo[CPLK][4];
  const float* qh = reinterpret_cast<const float*>(q + b * ql.b + layer * ql.layer + (int64_t)head * ql.head);
#pragma unroll
  for (int c = 0; c < CPLK; ++c) {
    const float4 a0 = *reinterpret_cast<const float4*>(qh + 8 * (p + 8 * c));
    const float4 a1 = *reinterpret_cast<const float4*>(qh + 8 * (p + 8 * c) + 4);
    const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      qhi[c][w] = pack_bf16_hi(x[2 * w], x[2 * w + 1]);
      qlo[c][w] = pack_bf16_lo(x[2 * w], x[2 * w + 1], qhi[c][w]);
    }
  }
  float M = -INFINITY, lsum = 0.f;
  float acc[CPLV * 8];
#pragma unroll
  for (int e = 0; e < CPLV * 8; ++e) acc[e] = 0.f;

#pragma unroll 1
  for (int t = 0; t < T; ++t) {
    const int base = (t * 4 + wid) * RPT;
    int32_t row[2];
    Vec16 kc[2][CPLK];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      row[j] = sRow[base + 8 * j + rr];
      // a padding row's offset lies past the resource and reads zeros: its weight 0 must not meet NaN
      const uint32_t off = row[j] >= 0 ? (uint32_t)row[j] * (uint32_t)kl.row + 16u * p : kBufferOutOfRange;
#pragma unroll
      for (int c = 0; c < CPLK; ++c) kc[j][c] = ld16_buffer(krs, off + 128u * c);
    }
    float lg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < CPLK; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          a = dot2_bf16(kc[j][c].w[w], qhi[c][w], a);
          a = dot2_bf16(kc[j][c].w[w], qlo[c][w], a);
        }
      a = sum8(a);
      lg[j] = row[j] >= 0 ? a * scale : -INFINITY;
    }
    // online softmax: the wave's running max, rescaling the accumulators when it grows
    const float mt = max_across_rows8(fmaxf(lg[0], lg[1]));
    if (mt > M) {                                     // wave-uniform
      const float alpha = M == -INFINITY ? 0.f : __expf(M - mt);
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < CPLV * 8; ++e) acc[e] *= alpha;
      M = mt;
    }
    const float w0 = lg[0] == -INFINITY ? 0.f : __expf(lg[0] - M);
    const float w1 = lg[1] == -INFINITY ? 0.f : __expf(lg[1] - M);
    lsum += w0 + w1;
    const uint32_t whi = pack_bf16_hi(w0, w1);
    const uint32_t wlo = pack_bf16_lo(w0, w1, whi);
#pragma unroll
    for (int c = 0; c < CPLV; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // (row0[2w], row1[2w]) and (row0[2w+1], row1[2w+1]) of chunk c
        const uint32_t pl = __builtin_amdgcn_perm(kc[1][c].w[w], kc[0][c].w[w], 0x05040100u);
        const uint32_t ph = __builtin_amdgcn_perm(kc[1][c].w[w], kc[0][c].w[w], 0x07060302u);
        float& a0 = acc[c * 8 + 2 * w];
        float& a1 = acc[c * 8 + 2 * w + 1];
        a0 = dot2_bf16(pl, wlo, dot2_bf16(pl, whi, a0));
        a1 = dot2_bf16(ph, wlo, dot2_bf16(ph, whi, a1));
      }
  }
  // PROJ: this thread's first output row of W_UV[head] (half of it), requested now so that the
  // loads overlap the merge below; they do not depend on the attention
  constexpr int kHalfChunks = DV / 2 / 8;            // 16-byte chunks of bf16 weights per half row
  constexpr int kPre = kHalfChunks / 2;              // of them requested before the merge (registers)
  const int half = tid & 1;
  const char* wrow = reinterpret_cast<const char*>(w_uv + ((size_t)head * dv + (tid >> 1)) * DV + half * (DV / 2));
  Vec16 wpre[PROJ ? kHalfChunks : 1];
  if (PROJ && (tid >> 1) < dv) {
#pragma unroll
    for (int c = 0; c < (PROJ ? kPre : 0); ++c) wpre[c] = ld16(wrow + 16 * c);
  }
  // wave totals (the 8 lanes that share p hold different rows), then the cross-wave merge
  const float lw = sum_across_rows8(lsum);
#pragma unroll
  for (int e = 0; e < CPLV * 8; ++e) acc[e] = sum_across_rows8(acc[e]);
  if (lane == 0) { s_m[wid] = M; s_l[wid] = lw; }
  __syncthreads();
  const float MM = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  const float fw = M == -INFINITY ? 0.f : __expf(M - MM);
  if (rr == 0) {
#pragma unroll
    for (int c = 0; c < CPLV; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wid][(p + 8 * c) * 8 + e] = acc[c * 8 + e] * fw;
  }
  __syncthreads();
  float L = 0.f;
  if (MM != -INFINITY) {
#pragma unroll
    for (int w = 0; w < 4; ++w) L += s_m[w] == -INFINITY ? 0.f : s_l[w] * __expf(s_m[w] - MM);
  }
  if (FIN) {
    // the head's only split: out = sum / L (no rows: zeros), as the merge would write it
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (!PROJ) {
      float* o = out + (((size_t)b * n_layers + layer) * Hq + head) * DV;
      for (int d = tid; d < DV; d += kThreads) o[d] = (red[0][d] + red[1][d] + red[2][d] + red[3][d]) * inv;
      return;
    }
    // out[b][head][0:dv) = W_UV[head] o: o in red[0] (each dim owned by one thread), then thread
    // (r, half) takes the dims [half DV/2, (half + 1) DV/2) of output row r (its first row's weights
    // requested before the barrier, half of them before the merge)
    if ((tid >> 1) < dv) {
#pragma unroll
      for (int c = kPre; c < kHalfChunks; ++c) wpre[c] = ld16(wrow + 16 * c);
    }
    for (int d = tid; d < DV; d += kThreads) red[0][d] = (red[0][d] + red[1][d] + red[2][d] + red[3][d]) * inv;
    __syncthreads();
    const float* oh = &red[0][half * (DV / 2)];
    auto dot_half = [&](const Vec16* w, int nchunk, int c0, float acc) {
#pragma unroll
      for (int c = 0; c < nchunk; ++c) {
        const float4 o0 = *reinterpret_cast<const float4*>(oh + 8 * (c0 + c));
        const float4 o1 = *reinterpret_cast<const float4*>(oh + 8 * (c0 + c) + 4);
        acc = fmaf(bf_lo(w[c].w[0]), o0.x, acc); acc = fmaf(bf_hi(w[c].w[0]), o0.y, acc);
        acc = fmaf(bf_lo(w[c].w[1]), o0.z, acc); acc = fmaf(bf_hi(w[c].w[1]), o0.w, acc);
        acc = fmaf(bf_lo(w[c].w[2]), o1.x, acc); acc = fmaf(bf_hi(w[c].w[2]), o1.y, acc);
        acc = fmaf(bf_lo(w[c].w[3]), o1.z, acc); acc = fmaf(bf_hi(w[c].w[3]), o1.w, acc);
      }
      return acc;
    };
    if ((tid >> 1) < dv) {                             // the first row: weights already requested
      float a = dot_half(wpre, kHalfChunks, 0, 0.f);
      a += __shfl_xor(a, 1, kWave);
      if (half == 0) out[((size_t)b * Hq + head) * dv + (tid >> 1)] = a;
    }
    for (int r = (tid >> 1) + kThreads / 2; r < dv; r += kThreads / 2) {   // rows past the first 128
      const char* wr = reinterpret_cast<const char*>(w_uv + ((size_t)head * dv + r) * DV + half * (DV / 2));
      constexpr int kGroup = 8;
      float a = 0.f;
#pragma unroll 1
      for (int c0 = 0; c0 < kHalfChunks; c0 += kGroup) {
        Vec16 w[kGroup];
#pragma unroll
        for (int c = 0; c < kGroup; ++c) w[c] = ld16(wr + 16 * (c0 + c));
        a = dot_half(w, kGroup, c0, a);
      }
      a += __shfl_xor(a, 1, kWave);
      if (half == 0) out[((size_t)b * Hq + head) * dv + r] = a;
    }
    return;
  }
  const size_t pbase = (size_t)inst * nsplit + split;
  for (int d = tid; d < DV; d += kThreads) part_o[pbase * DV + d] = red[0][d] + red[1][d] + red[2][d] + red[3][d];
  if (tid == 0) part_ml[pbase] = make_float2(MM, L);
}

// One workgroup per head: every thread first issues the loads of its
// partial-output vectors (4 dims, every (256 / (DV/4))-th split), then wave 0
// turns the splits' (max, sum) into weights exp(m_s - M) and 1 / L in LDS, and
// each thread folds its splits; the split groups are summed through LDS.  The
// partial loads do not wait for the weights, so the whole merge costs about one
// memory round trip.
constexpr int kCombineThreads = 256;
constexpr int kCombineRegs = 8;           // partial vectors a thread keeps in flight per round
template <int GQC>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const float* __restrict__ part_o,
                                                                       const float2* __restrict__ part_ml,
                                                                       float* __restrict__ out, int DV, int Hq,
                                                                       int n_layers, int n_groups, int layer_begin,
                                                                       int n_lay, int nsplit, int nhc) {
  __shared__ float s_w[kCombineMaxSplits];
  __shared__ float s_l[kCombineMaxSplits];
  __shared__ float s_inv;
  __shared__ float4 s_acc[kCombineThreads];
  const int ih = blockIdx.x;                 // ((inst * nhc + hcix) * GQC + h)
  const int h = ih % GQC;
  const int ic = ih / GQC;                   // inst * nhc + hcix
  const int hcix = ic % nhc;
  const int inst = ic / nhc;
  const int r = inst % n_groups;
  const int bl = inst / n_groups;
  const int lo = bl % n_lay;
  const int b = bl / n_lay;
  const int head = r * (Hq / n_groups) + hcix * GQC + h;
  const size_t pb = (size_t)ic * nsplit;
  const int tid = threadIdx.x;
  const int DV4 = DV / 4;
  const int ngrp = kCombineThreads / DV4;    // split groups (DV4 divides 256)
  const int d4 = tid % DV4, sg = tid / DV4;
  const float4* po = reinterpret_cast<const float4*>(part_o);
  // this thread's first round of partial vectors, issued before the weights exist
  float4 x[kCombineRegs];
#pragma unroll
  for (int u = 0; u < kCombineRegs; ++u) {
    const int sp = sg + u * ngrp;
    x[u] = sp < nsplit ? po[((pb + sp) * GQC + h) * DV4 + d4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid < kWave) {
    // (max, sum) of every split: the split's max goes to s_w, its sum to s_l, one load each
    float M = -INFINITY;
    for (int sp = tid; sp < nsplit; sp += kWave) {
      const float2 ml = part_ml[(pb + sp) * GQC + h];
      s_w[sp] = ml.y > 0.f ? ml.x : -INFINITY;
      s_l[sp] = ml.y;
      M = fmaxf(M, s_w[sp]);
    }
    M = wave_max(M);
    float L = 0.f;
    for (int sp = tid; sp < nsplit; sp += kWave) {     // each lane rereads only its own entries
      const float w = s_w[sp] == -INFINITY ? 0.f : __expf(s_w[sp] - M);
      s_w[sp] = w;
      L += s_l[sp] * w;
    }
    L = wave_sum(L);
    if (tid == 0) s_inv = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += kCombineRegs * ngrp) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < kCombineRegs; ++u) {
        const int sp = s0 + sg + u * ngrp;
        x[u] = sp < nsplit ? po[((pb + sp) * GQC + h) * DV4 + d4] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineRegs; ++u) {
      const int sp = s0 + sg + u * ngrp;
      const float w = sp < nsplit ? s_w[sp] : 0.f;
      if (w > 0.f) {                         // a split without rows contributes nothing
        acc.x = fmaf(w, x[u].x, acc.x); acc.y = fmaf(w, x[u].y, acc.y);
        acc.z = fmaf(w, x[u].z, acc.z); acc.w = fmaf(w, x[u].w, acc.w);
      }
    }
  }
  s_acc[tid] = acc;
  __syncthreads();
  if (tid < DV4) {
    float4 t = s_acc[tid];
    for (int g = 1; g < ngrp; ++g) {
      const float4 v = s_acc[g * DV4 + tid];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    const float inv = s_inv;
    reinterpret_cast<float4*>(out + (((size_t)b * n_layers + layer_begin + lo) * Hq + head) * DV)[tid] =
        make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
}

// Query heads per workgroup: they must share both the selection group and the KV head, so the
// chunk divides the smaller of the two head counts (one divides the other).
int head_chunk(const spc_shape& s) {
  const int GQ = s.n_q_heads / s.n_groups, per_kv = s.n_q_heads / s.n_kv_heads;
  const int g = GQ < per_kv ? GQ : per_kv;
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

// rows per split = 4 waves x 8 rows x NI of the instantiation launched below
// (NI = 4, or 2 where registers are tight: 8 heads per workgroup); MLA latent rows:
// 4 waves x 4, 16 or 32 tiles of 16 rows (32 for budgets of up to 2048 rows once there are >= 512
// heads: one split per head, 512 workgroups at two per CU; else 16 once the launch has >= 1024
// workgroups)
int latent_tiles(const spc_shape& s) {
  constexpr int kWhole = 4 * 16 * kLatentTilesWhole;
  constexpr int kLarge = 4 * 16 * kLatentTilesLarge;
  const long heads = (long)s.batch * s.n_layers * s.n_q_heads;
  if (s.budget <= kWhole && heads >= 512) return kLatentTilesWhole;   // one split per head, a full round
  const long wgs = heads * ((s.budget + kLarge - 1) / kLarge);
  return wgs >= 1024 ? kLatentTilesLarge : kLatentTilesSmall;
}
int rows_per_split(const spc_shape& s) {
  if (s.head_dim > 256) return 4 * 16 * latent_tiles(s);
  return head_chunk(s) >= 8 ? 64 : 128;
}

// Rows per split of one call over n_lay layers.  The bf16 128-dim kernels with up to 4 heads
// per workgroup also come with 5 iterations per wave (160 rows, still 4 workgroups per CU,
// 1024 resident on the chip).  A launch runs in rounds of 1024 workgroups, each round about
// as long as its split's rows; where 128-row splits leave a short last round (28 layers of
// 8 groups x 4 head chunks x 16 splits = 3.5 rounds), the 160-row split needs fewer rounds
// for fewer total row-times, and it is taken.  Never fewer splits than that: the workspace is
// sized for rows_per_split.
int split_rows(const spc_shape& s, int n_lay) {
  const int base = rows_per_split(s);
  if (s.dtype != SPC_BF16 || s.head_dim != 128 || s.v_dim != 128 || base != 128) return base;
  constexpr long kResident = 1024;
  const long per_split = (long)s.batch * n_lay * s.n_q_heads / head_chunk(s);   // workgroups per split index
  auto cost = [&](int rows) {
    const long wgs = per_split * ((s.budget + rows - 1) / rows);
    return ((wgs + kResident - 1) / kResident) * rows;
  };
  return cost(kSplitRowsWide) < cost(base) ? kSplitRowsWide : base;
}

struct SplitArgs {
  const char* q; QL ql; const char* kv; KL kl; const int32_t* rows; const int32_t* row_count; int mode;
  int layer_begin, n_lay, nsplit, nhc, max_rows; float* part_o; float2* part_ml;
};

template <int DT, int D, int DV, int GQC, int NI>
hipError_t launch_split(const spc_shape& s, dim3 grid, hipStream_t st, const SplitArgs& a) {
  attn_split_kernel<DT, D, DV, GQC, NI><<<grid, kThreads, 0, st>>>(
      a.q, a.ql, a.kv, a.kl, a.rows, a.row_count, a.mode, s.n_q_heads, s.n_kv_heads, s.n_groups, s.budget,
      a.layer_begin, a.n_lay, a.nsplit, a.nhc, a.max_rows, s.scale, a.part_o, a.part_ml);
  return hipGetLastError();
}

template <int DT, int D, int DV = D>
hipError_t launch_split_gqc(int gqc, const spc_shape& s, dim3 grid, hipStream_t st, const SplitArgs& a) {
  switch (gqc) {
    case 1: return launch_split<DT, D, DV, 1, 4>(s, grid, st, a);
    case 2: return launch_split<DT, D, DV, 2, 4>(s, grid, st, a);
    case 4: return launch_split<DT, D, DV, 4, 4>(s, grid, st, a);
    case 8: return launch_split<DT, D, DV, 8, 2>(s, grid, st, a);
    default: return hipErrorInvalidValue;
  }
}

// the 160-row splits of split_rows (bf16, 128-dim keys and values, up to 4 heads per workgroup)
hipError_t launch_split_wide(int gqc, const spc_shape& s, dim3 grid, hipStream_t st, const SplitArgs& a) {
  static_assert(kSplitRowsWide == 4 * 8 * 5, "160 rows = 4 waves x 8 rows x 5 iterations");
  switch (gqc) {
    case 1: return launch_split<SPC_BF16, 128, 128, 1, 5>(s, grid, st, a);
    case 2: return launch_split<SPC_BF16, 128, 128, 2, 5>(s, grid, st, a);
    case 4: return launch_split<SPC_BF16, 128, 128, 4, 5>(s, grid, st, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_supported(const spc_shape& s) {
  if (s.dtype == SPC_F32) return s.head_dim == 128 && s.v_dim == 128;
  if (s.head_dim == 576) return s.v_dim == 512 && head_chunk(s) == 1;   // MLA latent: one head per group
  if (s.head_dim == 192) return s.v_dim == 128;   // MLA rows expanded per head: nope 128 + rope 64 keys
  return (s.head_dim == 128 && s.v_dim == 128) || (s.head_dim == 64 && s.v_dim == 64);
}

int attn_splits(const spc_shape& s) { return (s.budget + rows_per_split(s) - 1) / rows_per_split(s); }

// sized for rows_per_split: a call's split_rows is never smaller, so its partials fit
size_t attn_ws_bytes_layers(const spc_shape& s, int n_lay) {
  const size_t nsplit = (size_t)(s.budget + rows_per_split(s) - 1) / rows_per_split(s);
  const size_t heads = (size_t)s.batch * n_lay * s.n_q_heads;        // one partial per head per split
  return heads * nsplit * ((size_t)s.v_dim * sizeof(float) + sizeof(float2));
}

size_t attn_ws_bytes(const spc_shape& s) { return attn_ws_bytes_layers(s, s.n_layers); }

namespace {

struct AttnGeom {
  int n_lay, rows, nsplit, gqc, nhc;
  size_t n_inst;
  float* part_o;
  float2* part_ml;
};

AttnGeom attn_geom(const spc_shape& s, int layer_begin, int layer_end, void* ws) {
  AttnGeom g;
  g.n_lay = layer_end - layer_begin;
  g.rows = split_rows(s, g.n_lay);
  g.nsplit = (s.budget + g.rows - 1) / g.rows;
  g.gqc = head_chunk(s);
  g.nhc = s.n_q_heads / s.n_groups / g.gqc;
  g.n_inst = (size_t)s.batch * g.n_lay * s.n_groups;
  g.part_o = static_cast<float*>(ws);
  g.part_ml = reinterpret_cast<float2*>(g.part_o + g.n_inst * g.nhc * g.nsplit * g.gqc * s.v_dim);
  return g;
}

}  // namespace

namespace {

// fin_out: the attention output, written by the split kernel itself where the shape has one split per
// head (MLA latent rows; the caller then launches no merge), else NULL
// proj_w (with fin_out): W_UV, and fin_out receives the output projection [B][H][proj_dv] instead
hipError_t launch_partial(const spc_shape& s, const void* q, const spc_q_layout& qlay, const void* kv,
                          const spc_kv_layout& klay, const int32_t* rows, const int32_t* row_count, int mode,
                          int layer_begin, int layer_end, void* ws, float* fin_out, hipStream_t st,
                          const uint16_t* proj_w = nullptr, int proj_dv = 0) {
  const int eb = s.dtype == SPC_BF16 ? 2 : 4;
  const AttnGeom g = attn_geom(s, layer_begin, layer_end, ws);
  SplitArgs a;
  a.q = static_cast<const char*>(q);
  const int qeb = mla_shape(s) ? 4 : eb;          // MLA: float32 absorbed query
  a.ql = QL{qlay.s_b * qeb, qlay.s_layer * qeb, qlay.s_head * qeb};
  a.kv = static_cast<const char*>(kv);
  a.kl = KL{klay.s_b * eb, klay.s_layer * eb, klay.s_head * eb, klay.s_row * eb, klay.s_kv * eb};
  a.rows = rows;
  a.row_count = row_count;
  a.mode = mode;
  a.layer_begin = layer_begin;
  a.n_lay = g.n_lay;
  a.nsplit = g.nsplit;
  a.nhc = g.nhc;
  a.max_rows = mode == SPC_ROWS_SLOTS ? s.budget : s.max_len;
  a.part_o = g.part_o;
  a.part_ml = g.part_ml;
  const int gqc = g.gqc;
  const dim3 grid(g.nsplit, (unsigned)g.n_inst, g.nhc);
  hipError_t e = hipErrorInvalidValue;
  if (s.dtype == SPC_F32) {
    e = launch_split_gqc<SPC_F32, 128>(gqc, s, grid, st, a);
  } else if (s.head_dim == 128 && g.rows == kSplitRowsWide) {
    e = launch_split_wide(gqc, s, grid, st, a);
  } else if (s.head_dim == 128) {
    e = launch_split_gqc<SPC_BF16, 128>(gqc, s, grid, st, a);
  } else if (s.head_dim == 64) {
    e = launch_split_gqc<SPC_BF16, 64>(gqc, s, grid, st, a);
  } else if (s.head_dim == 192) {
    e = launch_split_gqc<SPC_BF16, 192, 128>(gqc, s, grid, st, a);
  } else if (s.head_dim == 576 && gqc == 1) {
    // one-dimensional grid: 8 XCD lanes x groups of every head (see the kernel)
    const int n_glob = s.batch * g.n_lay * g.nsplit;
    const int parts = n_glob < 8 && 8 % n_glob == 0 ? 8 / n_glob : 1;
    const dim3 lgrid((unsigned)(parts > 1 ? 8 * ((s.n_groups + parts - 1) / parts)
                                          : 8 * ((n_glob + 7) / 8) * s.n_groups));
    const int tiles = latent_tiles(s);
#define SPC_LATENT(TT, FF, PP)                                                                                \
  attn_split_latent_kernel<576, 512, TT, FF, PP><<<lgrid, kThreads, 0, st>>>(                                \
      a.q, a.ql, a.kv, a.kl, a.rows, a.row_count, a.mode, s.n_q_heads, s.n_kv_heads, s.n_groups, s.budget,     \
      a.layer_begin, a.n_lay, a.nsplit, n_glob, parts, a.max_rows, s.scale, a.part_o, a.part_ml, fin_out,      \
      s.n_layers, proj_w, proj_dv)
    if (fin_out && (tiles != kLatentTilesWhole || g.nsplit != 1)) return hipErrorInvalidValue;
    if (proj_w && (!fin_out || g.n_lay != 1)) return hipErrorInvalidValue;
    if (tiles == kLatentTilesWhole && proj_w)
      SPC_LATENT(kLatentTilesWhole, true, true);
    else if (tiles == kLatentTilesWhole && fin_out)
      SPC_LATENT(kLatentTilesWhole, true, false);
    else if (tiles == kLatentTilesWhole)
      SPC_LATENT(kLatentTilesWhole, false, false);
    else if (tiles == kLatentTilesLarge)
      SPC_LATENT(kLatentTilesLarge, false, false);
    else
      SPC_LATENT(kLatentTilesSmall, false, false);
#undef SPC_LATENT
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_attn_partial(const spc_shape& s, const void* q, const spc_q_layout& qlay, const void* kv,
                               const spc_kv_layout& klay, const int32_t* rows, const int32_t* row_count, int mode,
                               int layer_begin, int layer_end, void* ws, hipStream_t st) {
  return launch_partial(s, q, qlay, kv, klay, rows, row_count, mode, layer_begin, layer_end, ws, nullptr, st);
}

hipError_t launch_attn_merge(const spc_shape& s, int layer_begin, int layer_end, const void* ws, float* out,
                             hipStream_t st) {
  const AttnGeom g = attn_geom(s, layer_begin, layer_end, const_cast<void*>(ws));
  const dim3 g2((unsigned)(g.n_inst * g.nhc * g.gqc));
  switch (g.gqc) {
#define SPC_CASE(N)                                                                                         \
  case N:                                                                                                   \
    attn_combine_kernel<N><<<g2, kCombineThreads, 0, st>>>(g.part_o, g.part_ml, out, s.v_dim, s.n_q_heads,   \
                                                           s.n_layers, s.n_groups, layer_begin, g.n_lay,     \
                                                           g.nsplit, g.nhc);                                 \
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

bool latent_one_split(const spc_shape& s) {
  return s.head_dim == 576 && head_chunk(s) == 1 && latent_tiles(s) == kLatentTilesWhole;
}

hipError_t launch_mla_attn_out_proj(const spc_shape& s, const void* q, const spc_q_layout& qlay, const void* kv,
                                    const spc_kv_layout& klay, const int32_t* rows, const int32_t* row_count,
                                    int mode, int layer, int dv, const void* w_uv, float* o_lat, float* out, void* ws,
                                    hipStream_t st) {
  if (latent_one_split(s))                      // one launch: attention and projection per head
    return launch_partial(s, q, qlay, kv, klay, rows, row_count, mode, layer, layer + 1, ws, out, st,
                          static_cast<const uint16_t*>(w_uv), dv);
  const hipError_t e = launch_attn(s, q, qlay, kv, klay, rows, row_count, mode, layer, layer + 1, o_lat, ws, st);
  if (e != hipSuccess) return e;
  return launch_mla_out_proj(s.batch, s.n_q_heads, dv, w_uv, o_lat + (size_t)layer * s.n_q_heads * kMlaLatent,
                             (int64_t)s.n_layers * s.n_q_heads * kMlaLatent, out, st);
}

hipError_t launch_attn(const spc_shape& s, const void* q, const spc_q_layout& qlay, const void* kv,
                       const spc_kv_layout& klay, const int32_t* rows, const int32_t* row_count, int mode,
                       int layer_begin, int layer_end, float* out, void* ws, hipStream_t st) {
  // MLA latent rows with one split per head: the split kernel writes the output, no merge
  const bool fin = latent_one_split(s);
  const hipError_t e = launch_partial(s, q, qlay, kv, klay, rows, row_count, mode, layer_begin, layer_end, ws,
                                      fin ? out : nullptr, st);
  if (e != hipSuccess || fin) return e;
  return launch_attn_merge(s, layer_begin, layer_end, ws, out, st);
}

}  // namespace spc
