// Internal device helpers shared by the HIP kernels of libspc (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spc.h"

namespace spc {

constexpr int kWave = 64;

// ---------------------------------------------------------------- element access

// A 16-byte vector of stored elements: 8 bf16 or 4 fp32.
struct alignas(16) Vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ Vec16 ld16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  Vec16 r;
  r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  return r;
}

// Buffer-resource loads (raw, stride 0): an offset at or past the resource's byte count reads
// zeros, which turns a padding row's load into zeros with no branch.  Word 3 of the resource
// for gfx9-family parts: 32-bit data format, no swizzle.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr uint32_t kBufferOutOfRange = 0x80000000u;   // past any range the host allows (< 2 GiB)
// AUX: the load's cache-policy bits (2: nontemporal, for data read once).
constexpr int kLoadNontemporal = 2;
template <int AUX = 0>
__device__ __forceinline__ Vec16 ld16_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
  Vec16 o;
  o.w[0] = (uint32_t)v.x; o.w[1] = (uint32_t)v.y; o.w[2] = (uint32_t)v.z; o.w[3] = (uint32_t)v.w;
  return o;
}

__device__ __forceinline__ void st16(void* p, const Vec16& r) {
  *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
}

// bf16 is the upper half of an fp32: widening is a shift.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c on packed bf16 pairs (v_dot2_f32_bf16), fp32 result.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Round-to-nearest-even bf16 of a float, as the upper 16 bits of a word.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// Packed bf16 pair (lo = a, hi = b) of two floats, and of their rounding remainders:
// a ~= hi.lo + lo.lo and b ~= hi.hi + lo.hi to ~16 mantissa bits (finite inputs).
__device__ __forceinline__ uint32_t pack_bf16_hi(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }
__device__ __forceinline__ uint32_t pack_bf16_lo(float a, float b, uint32_t hi) {
  return bf16_bits(a - bf_lo(hi)) | (bf16_bits(b - bf_hi(hi)) << 16);
}
// Dot product of two 16-byte chunks (8 bf16 or 4 fp32), accumulated into c.
template <int DT>
__device__ __forceinline__ float dot16(const Vec16& a, const Vec16& b, float c);

template <>
__device__ __forceinline__ float dot16<SPC_BF16>(const Vec16& a, const Vec16& b, float c) {
  c = dot2_bf16(a.w[0], b.w[0], c);
  c = dot2_bf16(a.w[1], b.w[1], c);
  c = dot2_bf16(a.w[2], b.w[2], c);
  c = dot2_bf16(a.w[3], b.w[3], c);
  return c;
}

template <>
__device__ __forceinline__ float dot16<SPC_F32>(const Vec16& a, const Vec16& b, float c) {
  c = fmaf(__uint_as_float(a.w[0]), __uint_as_float(b.w[0]), c);
  c = fmaf(__uint_as_float(a.w[1]), __uint_as_float(b.w[1]), c);
  c = fmaf(__uint_as_float(a.w[2]), __uint_as_float(b.w[2]), c);
  c = fmaf(__uint_as_float(a.w[3]), __uint_as_float(b.w[3]), c);
  return c;
}

// Elements per 16-byte chunk.
template <int DT> struct ElemsPerChunk;
template <> struct ElemsPerChunk<SPC_BF16> { static constexpr int value = 8; };
template <> struct ElemsPerChunk<SPC_F32> { static constexpr int value = 4; };

// Widen a 16-byte chunk into EPC floats.
template <int DT>
__device__ __forceinline__ void widen16(const Vec16& a, float* out);

template <>
__device__ __forceinline__ void widen16<SPC_BF16>(const Vec16& a, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf_lo(a.w[i]);
    out[2 * i + 1] = bf_hi(a.w[i]);
  }
}

template <>
__device__ __forceinline__ void widen16<SPC_F32>(const Vec16& a, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(a.w[i]);
}

// ---------------------------------------------------------------- cross-lane

// DPP move within rows of 16 lanes (bound_ctrl: out-of-range reads give 0).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i within each 8-lane half row

// Sum over each aligned group of 8 lanes; every lane of the group gets the total.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Max / sum over lanes that share (lane & 7): the 8 lanes l, l+8, ..., l+56.

constexpr int kDppRowRor8 = 0x128;      // lane i <- lane (i+8) mod 16 within each 16-lane row

// Sum of a lane's value and its partner's across the 16-lane-row pairs (l ^ 16)
// and the wave halves (l ^ 32), with gfx950's permlane swaps: each swap hands
// every lane its partner's value in one of the two results.
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// max over the 8 lanes that share lane & 7 (l ^ 8 by DPP, l ^ 16 and l ^ 32 by permlane swaps)
__device__ __forceinline__ float max_across_rows8(float v) {
  v = fmaxf(v, dpp_f<kDppRowRor8>(v));
  v = max_xor16(v);
  return max_xor32(v);
}

__device__ __forceinline__ float sum_across_rows8(float v) {
  v += dpp_f<kDppRowRor8>(v);
  v = add_xor16(v);
  return add_xor32(v);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  // bound_ctrl off and old = 0: lanes without a source lane read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Inclusive scan of a uint32 over the wave: DPP row shifts scan each 16-lane
// row, then the three lower row totals are broadcast with readlane.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & (kWave - 1);
  x += dpp_u<0x111>(x);   // row_shr:1
  x += dpp_u<0x112>(x);   // row_shr:2
  x += dpp_u<0x114>(x);   // row_shr:4
  x += dpp_u<0x118>(x);   // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  if (lane >= 16) x += r0;
  if (lane >= 32) x += r1;
  if (lane >= 48) x += r2;
  return x;
}

// Exclusive scan over the block (blockDim.x a multiple of 64, <= 1024).
// `smem` holds >= 16 words; returns the exclusive prefix, `total` the block sum.
// Ends with a barrier so smem can be reused right away.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* smem, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) smem[wid] = incl;
  __syncthreads();
  uint32_t base = 0u, tot = 0u;
  for (int w = 0; w < nw; ++w) {
    const uint32_t t = smem[w];
    base += w < wid ? t : 0u;
    tot += t;
  }
  total = tot;
  __syncthreads();
  return base + incl - v;
}

__device__ __forceinline__ int clamp_len(const int32_t* lengths, int b, int max_len) {
  int n = lengths[b];
  return n < 0 ? 0 : (n > max_len ? max_len : n);
}

}  // namespace spc
