// Retrieval-head front end: from the new token of each sequence to the stage-1
// query and the new DLM key (SpeContext blog section 5 "C1": the head keeps the
// distilled model's embedding and Query/Key projections; paper summary section
// 4.1: EAGLE-3's single decoder layer, its 2K context extended with training-free
// YaRN; section 4.3).
//
//   x = emb[token];  q = rope(W_q x^), k = rope(W_k x^),  x^ = gamma * x / rms(x)
//
// The work is one GEMV pass over W_q and W_k ((H_q + H_kv) * d rows of `hidden`
// elements: 40 MiB in bf16 at hidden 4096), bound by HBM.  The RMS factor is a
// scalar per sequence, so it is applied after the GEMV: the GEMV sums
// W[r] . (gamma * x) and the sum of squares of x separately.
//
// front_gemv_kernel    grid (row blocks of 16 or 32, hidden slices of 1024).  The
//   slice of gamma * x of every sequence sits in LDS (float32, 4 KB per
//   sequence); each wave takes 4 or 8 rows, each lane two 16-byte chunks of a row
//   (all 16 loads in flight; one wave instruction reads 1 KB contiguous), and
//   a wave sum per (row, sequence) (DPP and permlane swaps, no LDS) gives the
//   slice's partial dot product.
//   Row-block 0 of each slice also writes the slice's sum of x^2.
// front_mfma_kernel    the same pass on MFMA for bf16 with more than 4 sequences.
// front_finish_kernel  one workgroup per (head, sequence), one thread per
//   rotary pair (i, i + d/2): sums the slice partials, scales by 1/rms, rotates
//   by position * theta'_i (angle reduced in double precision: positions reach
//   65536 radians at theta_0 = 1), applies the YaRN temperature, rounds to the
//   cache type and writes the query or appends the key.
#include "spc_common.h"
#include "spc_launch.h"

namespace spc {

namespace {

constexpr int kThreads = 256;

// RPW rows per wave: 4 for up to 4 sequences (more workgroups in flight), 8 beyond
// (each LDS read of x serves more rows).
template <int DT, int RPW>
__global__ __launch_bounds__(kThreads) void front_gemv_kernel(const int32_t* __restrict__ tokens,
                                                              const char* __restrict__ emb, int64_t vocab,
                                                              const char* __restrict__ gamma,
                                                              const char* __restrict__ wq, const char* __restrict__ wk,
                                                              int rows_q, int rows_total, int hidden, int B,
                                                              float* __restrict__ part, float* __restrict__ rms_part) {
  constexpr int EB = DT == SPC_BF16 ? 2 : 4;
  constexpr int EPC = ElemsPerChunk<DT>::value;            // elements per 16-byte chunk
  constexpr int CPL = kFrontSlice / EPC / kWave;           // chunks per lane of one row slice (2 bf16, 4 fp32)
  extern __shared__ __align__(16) float xs_dyn[];   // [B][kFrontSlice]: gamma * x over the slice
  float(*xs)[kFrontSlice] = reinterpret_cast<float(*)[kFrontSlice]>(xs_dyn);
  __shared__ float s_sq[kFrontMaxBatch][4];
  const int slice = blockIdx.y;
  const int k0 = slice * kFrontSlice;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int row0 = blockIdx.x * 4 * RPW + wid * RPW;

  // this wave's weight chunks first: they need nothing else
  Vec16 w[RPW][CPL];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r;
    if (row < rows_total) {
      const char* wr = row < rows_q ? wq + (size_t)row * hidden * EB : wk + (size_t)(row - rows_q) * hidden * EB;
#pragma unroll
      for (int c = 0; c < CPL; ++c) w[r][c] = ld16(wr + (size_t)k0 * EB + (size_t)(lane + kWave * c) * 16);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) w[r][c].w[0] = w[r][c].w[1] = w[r][c].w[2] = w[r][c].w[3] = 0u;
    }
  }
  // gamma * x of every sequence over the slice, and the slice's sum of x^2
  for (int b = 0; b < B; ++b) {
    const int t = tokens[b];
    const bool valid = t >= 0 && (int64_t)t < vocab;
    float sq = 0.f;
    for (int e = tid; e < kFrontSlice; e += kThreads) {
      float x = 0.f, g = 0.f;
      if (valid) {
        if (DT == SPC_BF16) {
          x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(emb)[(size_t)t * hidden + k0 + e] << 16);
          g = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(gamma)[k0 + e] << 16);
        } else {
          x = reinterpret_cast<const float*>(emb)[(size_t)t * hidden + k0 + e];
          g = reinterpret_cast<const float*>(gamma)[k0 + e];
        }
      }
      xs[b][e] = g * x;
      sq = fmaf(x, x, sq);
    }
    sq = wave_sum(sq);
    if (lane == 0) s_sq[b][wid] = sq;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < B) rms_part[(size_t)slice * kFrontMaxBatch + tid] =
      s_sq[tid][0] + s_sq[tid][1] + s_sq[tid][2] + s_sq[tid][3];

  for (int b = 0; b < B; ++b) {
    // the lane's elements of x: chunk (lane + 64 c) covers elements EPC*(lane + 64 c) ..
    float xv[CPL][EPC];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&xs[b][EPC * (lane + kWave * c) + e]);
        xv[c][e] = v.x; xv[c][e + 1] = v.y; xv[c][e + 2] = v.z; xv[c][e + 3] = v.w;
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float wf[EPC];
        widen16<DT>(w[r][c], wf);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc = fmaf(wf[e], xv[c][e], acc);
      }
      acc = sum_across_rows8(sum8(acc));          // DPP and permlane swaps: the wave total in every lane
      const int row = row0 + r;
      if (lane == 0 && row < rows_total) part[((size_t)slice * kFrontMaxBatch + b) * rows_total + row] = acc;
    }
  }
}

// bf16 with more than 4 sequences: the projection is a dense [rows x hidden] x
// [hidden x 16 sequences] product, so it runs on MFMA (v_mfma_f32_16x16x32_bf16):
// C^T[row][seq] = W[row][k] (gamma x)[seq][k].  A fragments are 16 contiguous bytes
// of a weight row, straight from memory (each weight read once); B fragments come
// from LDS, where gamma * x of the slice sits as a bf16 pair hi + lo (the product of
// two bf16 values has at most 16 significant bits, so hi + lo holds it exactly and
// the MFMAs add exact products in float32, as the GEMV does).  One wave per 16
// rows, four per workgroup; a lane ends with 4 consecutive rows of one sequence and
// writes them as one 16-byte vector into the same partial layout as the GEMV.
constexpr int kMfmaBatch = 16;
constexpr int kFrontKSteps = kFrontSlice / 32;
constexpr int kFrontAhead = 8;                    // k-steps of weight fragments in flight

__global__ __launch_bounds__(kThreads) void front_mfma_kernel(const int32_t* __restrict__ tokens,
                                                              const uint16_t* __restrict__ emb, int64_t vocab,
                                                              const uint16_t* __restrict__ gamma,
                                                              const uint16_t* __restrict__ wq,
                                                              const uint16_t* __restrict__ wk, int rows_q,
                                                              int rows_total, int hidden, int B,
                                                              float* __restrict__ part, float* __restrict__ rms_part) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint16_t xh[kMfmaBatch][kFrontSlice + 8];   // gamma * x, bf16 high part
  __shared__ __align__(16) uint16_t xl[kMfmaBatch][kFrontSlice + 8];   // and the remainder
  __shared__ float s_sq[kMfmaBatch][4];
  const int slice = blockIdx.y;
  const int k0 = slice * kFrontSlice;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, col = lane & 15, kc = lane >> 4;
  const int row = blockIdx.x * 64 + wid * 16 + col;           // this lane's weight row (A fragment row)
  const bool rok = row < rows_total;
  const uint16_t* wr = !rok ? wq : (row < rows_q ? wq + (size_t)row * hidden : wk + (size_t)(row - rows_q) * hidden);
  wr += k0 + 8 * kc;
  // the first k-steps' weight fragments go out before anything else
  bf16x8_t ring[kFrontAhead + 1];
  auto load_a = [&](int s, bf16x8_t& a) {
    if (rok) {
      a = *reinterpret_cast<const bf16x8_t*>(wr + 32 * s);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (__bf16)0.f;
    }
  };
#pragma unroll
  for (int s = 0; s < kFrontAhead; ++s) load_a(s, ring[s]);
  // gamma * x of every sequence over the slice (hi + lo), and the slice's sum of x^2: thread t
  // takes the 16-byte chunk t % 128 of sequence 2 i + t / 128 in round i (all loads issued first)
  constexpr int kChunksPerSlice = kFrontSlice / 8;
  constexpr int kRounds = kMfmaBatch * kChunksPerSlice / kThreads;
  static_assert(kThreads % kChunksPerSlice == 0 && kRounds * kThreads == kMfmaBatch * kChunksPerSlice,
                "setup split");
  const int ch = tid % kChunksPerSlice, sub = tid / kChunksPerSlice;
  const uint4 gv = *reinterpret_cast<const uint4*>(gamma + k0 + 8 * ch);
  uint4 xv[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int b = (kThreads / kChunksPerSlice) * i + sub;
    const int t = b < B ? tokens[b] : -1;
    xv[i] = t >= 0 && (int64_t)t < vocab ? *reinterpret_cast<const uint4*>(emb + (size_t)t * hidden + k0 + 8 * ch)
                                         : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int b = (kThreads / kChunksPerSlice) * i + sub;
    const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
    uint32_t hw[4], lw[4];
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = bf_lo(xw[j]), x1 = bf_hi(xw[j]);
      const float p0 = bf_lo(gw[j]) * x0, p1 = bf_hi(gw[j]) * x1;
      hw[j] = pack_bf16_hi(p0, p1);
      lw[j] = pack_bf16_lo(p0, p1, hw[j]);
      sq = fmaf(x0, x0, fmaf(x1, x1, sq));
    }
    *reinterpret_cast<uint4*>(&xh[b][8 * ch]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(&xl[b][8 * ch]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    sq = wave_sum(sq);
    if (lane == 0) s_sq[b][wid % (kChunksPerSlice / kWave)] = sq;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < B) rms_part[(size_t)slice * kFrontMaxBatch + tid] = s_sq[tid][0] + s_sq[tid][1];
  f32x4_t acc_h = {0.f, 0.f, 0.f, 0.f}, acc_l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kFrontKSteps; ++s) {
    if (s + kFrontAhead < kFrontKSteps) load_a(s + kFrontAhead, ring[(s + kFrontAhead) % (kFrontAhead + 1)]);
    const bf16x8_t a = ring[s % (kFrontAhead + 1)];
    const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&xh[col][32 * s + 8 * kc]);
    const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&xl[col][32 * s + 8 * kc]);
    acc_h = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc_h, 0, 0, 0);
    acc_l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc_l, 0, 0, 0);
  }
  // lane (col, kc): rows blockIdx.x * 64 + wid * 16 + 4 kc .. + 3 of sequence col
  const int r0 = blockIdx.x * 64 + wid * 16 + 4 * kc;
  if (col < B && r0 < rows_total) {
    float* dst = part + ((size_t)slice * kFrontMaxBatch + col) * rows_total + r0;
    *reinterpret_cast<float4*>(dst) =
        make_float4(acc_h[0] + acc_l[0], acc_h[1] + acc_l[1], acc_h[2] + acc_l[2], acc_h[3] + acc_l[3]);
  }
}

struct RopeFreqs {
  double theta[kFrontMaxHeadDim / 2];
};

template <int DT>
__global__ void front_finish_kernel(const int32_t* __restrict__ tokens, const int32_t* __restrict__ positions,
                                    int64_t vocab, const float* __restrict__ part, const float* __restrict__ rms_part,
                                    int nslice, int hidden, float eps, RopeFreqs fr, float mscale, int Hq, int Hkv,
                                    int d, int max_len, int rows_total, char* __restrict__ q_out,
                                    char* __restrict__ dlm_k) {
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;   // i < d/2
  const int t = tokens[b];
  const bool valid = t >= 0 && (int64_t)t < vocab;
  const int pos = positions[b];
  float o1 = 0.f, o2 = 0.f;
  if (valid) {
    float v1 = 0.f, v2 = 0.f, sq = 0.f;
    const int r1 = h * d + i, r2 = r1 + d / 2;
    for (int sl = 0; sl < nslice; ++sl) {
      const float* ps = part + ((size_t)sl * kFrontMaxBatch + b) * rows_total;
      v1 += ps[r1];
      v2 += ps[r2];
      sq += rms_part[(size_t)sl * kFrontMaxBatch + b];
    }
    const float inv = 1.f / sqrtf(sq / (float)hidden + eps);
    v1 *= inv;
    v2 *= inv;
    const double ang = fmod((double)pos * fr.theta[i], 6.283185307179586476925);
    const float c = (float)cos(ang), sn = (float)sin(ang);
    o1 = mscale * (v1 * c - v2 * sn);
    o2 = mscale * (v2 * c + v1 * sn);
  }
  char* dst;
  if (h < Hq) {
    dst = q_out + ((size_t)b * Hq + h) * d * (DT == SPC_BF16 ? 2 : 4);
  } else {
    if (pos < 0 || pos >= max_len) return;
    dst = dlm_k + (((size_t)b * Hkv + (h - Hq)) * max_len + pos) * d * (DT == SPC_BF16 ? 2 : 4);
  }
  if (DT == SPC_BF16) {
    reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)bf16_bits(o1);
    reinterpret_cast<uint16_t*>(dst)[i + d / 2] = (uint16_t)bf16_bits(o2);
  } else {
    reinterpret_cast<float*>(dst)[i] = o1;
    reinterpret_cast<float*>(dst)[i + d / 2] = o2;
  }
}

}  // namespace

size_t front_ws_bytes(const spc_shape& s) {
  const size_t rows = (size_t)(s.n_q_heads + s.n_kv_heads) * s.head_dim;
  return (size_t)kFrontMaxSlices * kFrontMaxBatch * (rows + 1) * sizeof(float);
}

hipError_t launch_front(const spc_shape& s, int hidden, int64_t vocab, const spc_rope& rope, float eps,
                        const int32_t* tokens, const int32_t* positions, const void* emb, const void* gamma,
                        const void* wq, const void* wk, void* q_out, void* dlm_k, void* ws, hipStream_t st) {
  const int d = s.head_dim;
  const int rows_q = s.n_q_heads * d;
  const int rows_total = (s.n_q_heads + s.n_kv_heads) * d;
  const int nslice = hidden / kFrontSlice;
  float* rms_part = static_cast<float*>(ws);
  float* part = rms_part + (size_t)kFrontMaxSlices * kFrontMaxBatch;
  const int rpw = s.batch <= 4 ? 4 : 8;
  const dim3 g1((rows_total + 4 * rpw - 1) / (4 * rpw), nslice);
  const char* e = static_cast<const char*>(emb);
  const char* g = static_cast<const char*>(gamma);
  const char* q = static_cast<const char*>(wq);
  const char* k = static_cast<const char*>(wk);
  const size_t lds = (size_t)s.batch * kFrontSlice * sizeof(float);
  if (s.dtype == SPC_BF16 && s.batch > 4) {
    const dim3 gm((rows_total + 63) / 64, nslice);
    front_mfma_kernel<<<gm, kThreads, 0, st>>>(tokens, static_cast<const uint16_t*>(emb), vocab,
                                               static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(wq),
                                               static_cast<const uint16_t*>(wk), rows_q, rows_total, hidden, s.batch,
                                               part, rms_part);
  } else {
#define SPC_GEMV(DT_, RPW_)                                                                             \
  front_gemv_kernel<DT_, RPW_><<<g1, kThreads, lds, st>>>(tokens, e, vocab, g, q, k, rows_q, rows_total, hidden, \
                                                          s.batch, part, rms_part)
  if (s.dtype == SPC_BF16) {
    SPC_GEMV(SPC_BF16, 4);            // bf16 beyond 4 sequences takes the MFMA kernel above
  } else {
    if (rpw == 4) SPC_GEMV(SPC_F32, 4); else SPC_GEMV(SPC_F32, 8);
  }
#undef SPC_GEMV
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // rotary frequencies in double precision, extended by YaRN's "NTK-by-parts" when factor > 1
  RopeFreqs fr;
  for (int i = 0; i < d / 2; ++i) {
    const double th = pow((double)rope.base, -2.0 * i / d);
    double v = th;
    if (rope.factor > 1.f) {
      const double r = rope.orig_max_pos * th / 6.283185307179586476925;   // rotations over the trained context
      double gmm = (r - rope.beta_slow) / ((double)rope.beta_fast - rope.beta_slow);
      gmm = gmm < 0.0 ? 0.0 : (gmm > 1.0 ? 1.0 : gmm);
      v = gmm * th + (1.0 - gmm) * th / rope.factor;
    }
    fr.theta[i] = v;
  }
  const float mscale = rope.factor > 1.f ? (float)(0.1 * log((double)rope.factor) + 1.0) : 1.f;
  const dim3 g2(s.n_q_heads + s.n_kv_heads, s.batch);
  if (s.dtype == SPC_BF16)
    front_finish_kernel<SPC_BF16><<<g2, d / 2, 0, st>>>(tokens, positions, vocab, part, rms_part, nslice, hidden,
                                                        eps, fr, mscale, s.n_q_heads, s.n_kv_heads, d, s.max_len,
                                                        rows_total, static_cast<char*>(q_out),
                                                        static_cast<char*>(dlm_k));
  else
    front_finish_kernel<SPC_F32><<<g2, d / 2, 0, st>>>(tokens, positions, vocab, part, rms_part, nslice, hidden,
                                                       eps, fr, mscale, s.n_q_heads, s.n_kv_heads, d, s.max_len,
                                                       rows_total, static_cast<char*>(q_out),
                                                       static_cast<char*>(dlm_k));
  return hipGetLastError();
}

}  // namespace spc
