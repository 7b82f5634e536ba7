// Stage 4 - sparse decode attention over the resident sparse KV only.
//
//   out[b][l][i] = sum_r softmax_r(scale * q_l[b][i] . K[r]) V[r]
// over the rows r of query head i's group (SpeContext blog section 4:
// llm.forward(..., sparse_kv=resident_kv); AttentionWeight formula of blog
// section 2).
//
// attn_split_kernel  split-K: one workgroup per (b, layer, group, head chunk,
//   split of kAttnRowsPerSplit rows).  The GQC query heads of the chunk share
//   every K/V row read.  Three phases:
//     1. logits: 8 lanes per row (lane p holds the 16-byte chunks p, p+8, ...;
//        one wave load covers 8 rows x 128 contiguous bytes), v_dot2 on packed
//        bf16, DPP 8-lane sums; logits of the split go to LDS;
//     2. per head max and exp in LDS (exact two-pass softmax of the split);
//     3. V rows in the same lane layout; every lane accumulates its dims for
//        all GQC heads; lanes holding the same dims are summed across the wave
//        and the 4 waves through LDS.
//   Writes the split's (max, sum) and unnormalised output per head.
// attn_combine_kernel  merges the splits of a head with their log-sum-exp
//   weights into the float32 output.
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kRps = kAttnRowsPerSplit;
constexpr int kIters = kRps / 32;             // 4 waves x 8 rows per iteration

struct QL { int64_t b, layer, head; };        // byte strides
struct KL { int64_t b, layer, head, row, kv; };

template <int DT, int D, int DV, int GQC>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(
    const char* __restrict__ q, QL ql, const char* __restrict__ kv, KL kl, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ row_count, int mode, int Hq, int Hkv, int n_groups, int K, int layer_begin,
    int n_lay, int nsplit, int nhc, int max_rows, float scale, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
  constexpr int EB = DT == SPC_BF16 ? 2 : 4;
  constexpr int EPC = ElemsPerChunk<DT>::value;
  constexpr int CPLK = D * EB / 16 / 8;
  constexpr int CPLV = DV * EB / 16 / 8;
  static_assert(D * EB % 128 == 0 && DV * EB % 128 == 0, "rows must be whole 8 x 16-byte chunks");

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
  const int kvh = (r * GQ) / (Hq / Hkv);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int p = lane & 7, rr = lane >> 3;

  __shared__ float sP[GQC][kRps];
  __shared__ int32_t sRow[kRps];
  __shared__ float sM[GQC], sL[GQC];
  __shared__ float red[4][GQC][DV];

  const int32_t* rl = rows + ((size_t)b * n_groups + r) * K;
  int cnt = K;
  if (mode == SPC_ROWS_GATHER) {
    cnt = row_count[(size_t)b * n_groups + r];
    cnt = cnt < 0 ? 0 : (cnt > K ? K : cnt);
  }
  const int i0 = split * kRps;
  for (int i = tid; i < kRps; i += kThreads) {
    const int idx = i0 + i;
    int32_t row = -1;
    if (idx < cnt) {
      const int32_t v = rl[idx];
      row = mode == SPC_ROWS_SLOTS ? (v >= 0 ? idx : -1) : (v >= 0 && v < max_rows ? v : -1);
    }
    sRow[i] = row;
  }

  Vec16 qv[GQC][CPLK];
#pragma unroll
  for (int h = 0; h < GQC; ++h) {
    const char* qh = q + b * ql.b + layer * ql.layer + (int64_t)(h0 + h) * ql.head;
#pragma unroll
    for (int c = 0; c < CPLK; ++c) qv[h][c] = ld16(qh + (p + 8 * c) * 16);
  }
  const char* kbase = kv + b * kl.b + layer * kl.layer + (int64_t)kvh * kl.head;
  __syncthreads();

  // phase 1: logits
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int li = it * 32 + wid * 8 + rr;
    const int32_t row = sRow[li];
    float acc[GQC];
#pragma unroll
    for (int h = 0; h < GQC; ++h) acc[h] = 0.f;
    if (row >= 0) {
      Vec16 kc[CPLK];
      const char* kr = kbase + (int64_t)row * kl.row;
#pragma unroll
      for (int c = 0; c < CPLK; ++c) kc[c] = ld16(kr + (p + 8 * c) * 16);
#pragma unroll
      for (int h = 0; h < GQC; ++h)
#pragma unroll
        for (int c = 0; c < CPLK; ++c) acc[h] = dot16<DT>(kc[c], qv[h][c], acc[h]);
    }
#pragma unroll
    for (int h = 0; h < GQC; ++h) {
      const float t = sum8(acc[h]);
      if (p == h) sP[h][li] = row >= 0 ? t * scale : -INFINITY;
    }
  }
  __syncthreads();

  // phase 2: per-head max, exp, sum over the split
  for (int h = wid; h < GQC; h += 4) {
    float m = -INFINITY;
    for (int i = lane; i < kRps; i += 64) m = fmaxf(m, sP[h][i]);
    m = wave_max(m);
    float s = 0.f;
    for (int i = lane; i < kRps; i += 64) {
      const float x = sP[h][i];
      const float e = x == -INFINITY ? 0.f : __expf(x - m);
      sP[h][i] = e;
      s += e;
    }
    s = wave_sum(s);
    if (lane == 0) { sM[h] = m; sL[h] = s; }
  }
  __syncthreads();

  // phase 3: weighted sum of V rows
  float acc[GQC][CPLV * EPC];
#pragma unroll
  for (int h = 0; h < GQC; ++h)
#pragma unroll
    for (int e = 0; e < CPLV * EPC; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int li = it * 32 + wid * 8 + rr;
    const int32_t row = sRow[li];
    if (row >= 0) {
      const char* vr = kbase + (int64_t)row * kl.row + kl.kv;
      Vec16 vc[CPLV];
#pragma unroll
      for (int c = 0; c < CPLV; ++c) vc[c] = ld16(vr + (p + 8 * c) * 16);
      float w[GQC];
#pragma unroll
      for (int h = 0; h < GQC; ++h) w[h] = sP[h][li];
#pragma unroll
      for (int c = 0; c < CPLV; ++c) {
        float x[EPC];
        widen16<DT>(vc[c], x);
#pragma unroll
        for (int h = 0; h < GQC; ++h)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[h][c * EPC + e] = fmaf(w[h], x[e], acc[h][c * EPC + e]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GQC; ++h)
#pragma unroll
    for (int e = 0; e < CPLV * EPC; ++e) acc[h][e] = sum_across_rows8(acc[h][e]);
  if (rr == 0) {
#pragma unroll
    for (int h = 0; h < GQC; ++h)
#pragma unroll
      for (int c = 0; c < CPLV; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) red[wid][h][(p + 8 * c) * EPC + e] = acc[h][c * EPC + e];
  }
  __syncthreads();
  const size_t pbase = ((size_t)inst * nhc + hcix) * nsplit + split;
  for (int t = tid; t < GQC * DV; t += kThreads) {
    const int h = t / DV, d = t - (t / DV) * DV;
    const float v = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
    part_o[(pbase * GQC + h) * DV + d] = v;
  }
  if (tid < GQC) part_ml[pbase * GQC + tid] = make_float2(sM[tid], sL[tid]);
}

template <int GQC>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           float* __restrict__ out, int DV, int Hq, int n_layers,
                                                           int n_groups, int layer_begin, int n_lay, int nsplit,
                                                           int nhc) {
  const int inst = blockIdx.x;
  const int hcix = blockIdx.y;
  const int h = blockIdx.z;
  const int r = inst % n_groups;
  const int bl = inst / n_groups;
  const int lo = bl % n_lay;
  const int b = bl / n_lay;
  const int GQ = Hq / n_groups;
  const int head = r * GQ + hcix * GQC + h;
  const size_t pb = ((size_t)inst * nhc + hcix) * nsplit;
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float2 ml = part_ml[(pb + sp) * GQC + h];
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float L = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float2 ml = part_ml[(pb + sp) * GQC + h];
    if (ml.y > 0.f) L += ml.y * __expf(ml.x - M);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* o = out + (((size_t)b * n_layers + layer_begin + lo) * Hq + head) * DV;
  for (int d = threadIdx.x; d < DV; d += blockDim.x) {
    float acc = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float2 ml = part_ml[(pb + sp) * GQC + h];
      if (ml.y > 0.f) acc += part_o[((pb + sp) * GQC + h) * DV + d] * __expf(ml.x - M);
    }
    o[d] = acc * inv;
  }
}

int head_chunk(const spc_shape& s) {
  const int GQ = s.n_q_heads / s.n_groups;
  if (GQ % 8 == 0) return 8;
  if (GQ % 4 == 0) return 4;
  if (GQ % 2 == 0) return 2;
  return 1;
}

template <int DT, int D, int DV, int GQC>
hipError_t launch_split(const spc_shape& s, dim3 grid, hipStream_t st, const char* q, QL ql, const char* kv, KL kl,
                        const int32_t* rows, const int32_t* row_count, int mode, int layer_begin, int n_lay,
                        int nsplit, int nhc, float* part_o, float2* part_ml) {
  attn_split_kernel<DT, D, DV, GQC><<<grid, kThreads, 0, st>>>(q, ql, kv, kl, rows, row_count, mode, s.n_q_heads,
                                                               s.n_kv_heads, s.n_groups, s.budget, layer_begin,
                                                               n_lay, nsplit, nhc,
                                                               mode == SPC_ROWS_SLOTS ? s.budget : s.max_len, s.scale,
                                                               part_o, part_ml);
  return hipGetLastError();
}

template <int DT, int D, int DV>
hipError_t launch_split_gqc(int gqc, const spc_shape& s, dim3 grid, hipStream_t st, const char* q, QL ql,
                            const char* kv, KL kl, const int32_t* rows, const int32_t* row_count, int mode,
                            int layer_begin, int n_lay, int nsplit, int nhc, float* part_o, float2* part_ml) {
  switch (gqc) {
    case 1: return launch_split<DT, D, DV, 1>(s, grid, st, q, ql, kv, kl, rows, row_count, mode, layer_begin, n_lay, nsplit, nhc, part_o, part_ml);
    case 2: return launch_split<DT, D, DV, 2>(s, grid, st, q, ql, kv, kl, rows, row_count, mode, layer_begin, n_lay, nsplit, nhc, part_o, part_ml);
    case 4: return launch_split<DT, D, DV, 4>(s, grid, st, q, ql, kv, kl, rows, row_count, mode, layer_begin, n_lay, nsplit, nhc, part_o, part_ml);
    case 8: return launch_split<DT, D, DV, 8>(s, grid, st, q, ql, kv, kl, rows, row_count, mode, layer_begin, n_lay, nsplit, nhc, part_o, part_ml);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_supported(const spc_shape& s) {
  if (s.dtype == SPC_F32) return s.head_dim == 128 && s.v_dim == 128;
  return (s.head_dim == 128 && s.v_dim == 128) || (s.head_dim == 64 && s.v_dim == 64) ||
         (s.head_dim == 576 && s.v_dim == 512);
}

size_t attn_ws_bytes(const spc_shape& s) {
  const size_t nsplit = (size_t)(s.budget + kRps - 1) / kRps;
  const size_t heads = (size_t)s.batch * s.n_layers * s.n_q_heads;   // one partial per head per split
  return heads * nsplit * ((size_t)s.v_dim * sizeof(float) + sizeof(float2));
}

hipError_t launch_attn(const spc_shape& s, const void* q, const spc_q_layout& qlay, const void* kv,
                       const spc_kv_layout& klay, const int32_t* rows, const int32_t* row_count, int mode,
                       int layer_begin, int layer_end, float* out, void* ws, hipStream_t st) {
  const int eb = s.dtype == SPC_BF16 ? 2 : 4;
  const int n_lay = layer_end - layer_begin;
  const int nsplit = (s.budget + kRps - 1) / kRps;
  const int gqc = head_chunk(s);
  const int nhc = s.n_q_heads / s.n_groups / gqc;
  const QL ql{qlay.s_b * eb, qlay.s_layer * eb, qlay.s_head * eb};
  const KL kl{klay.s_b * eb, klay.s_layer * eb, klay.s_head * eb, klay.s_row * eb, klay.s_kv * eb};
  const size_t n_inst = (size_t)s.batch * n_lay * s.n_groups;
  float* part_o = static_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(part_o + n_inst * nhc * nsplit * gqc * s.v_dim);
  const dim3 grid(nsplit, (unsigned)n_inst, nhc);
  const char* qc = static_cast<const char*>(q);
  const char* kc = static_cast<const char*>(kv);
  hipError_t e = hipErrorInvalidValue;
  if (s.dtype == SPC_F32) {
    e = launch_split_gqc<SPC_F32, 128, 128>(gqc, s, grid, st, qc, ql, kc, kl, rows, row_count, mode, layer_begin,
                                            n_lay, nsplit, nhc, part_o, part_ml);
  } else if (s.head_dim == 128) {
    e = launch_split_gqc<SPC_BF16, 128, 128>(gqc, s, grid, st, qc, ql, kc, kl, rows, row_count, mode, layer_begin,
                                             n_lay, nsplit, nhc, part_o, part_ml);
  } else if (s.head_dim == 64) {
    e = launch_split_gqc<SPC_BF16, 64, 64>(gqc, s, grid, st, qc, ql, kc, kl, rows, row_count, mode, layer_begin,
                                           n_lay, nsplit, nhc, part_o, part_ml);
  } else if (s.head_dim == 576) {
    e = launch_split_gqc<SPC_BF16, 576, 512>(gqc, s, grid, st, qc, ql, kc, kl, rows, row_count, mode, layer_begin,
                                             n_lay, nsplit, nhc, part_o, part_ml);
  }
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)n_inst, nhc, gqc);
  switch (gqc) {
#define SPC_CASE(N)                                                                                       \
  case N:                                                                                                 \
    attn_combine_kernel<N><<<g2, 128, 0, st>>>(part_o, part_ml, out, s.v_dim, s.n_q_heads, s.n_layers,   \
                                               s.n_groups, layer_begin, n_lay, nsplit, nhc);              \
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

}  // namespace spc
