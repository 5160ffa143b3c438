// Device-side helpers shared by the libmhc kernels (gfx950 / CDNA4).
//
// bf16 values travel as raw 16-bit patterns packed two per 32-bit word
// (element 2i in the low half, 2i+1 in the high half, little endian), eight
// per 16-byte vector.  Widening bf16 -> fp32 is exact (a 16-bit shift);
// narrowing fp32 -> bf16 uses the hardware round-to-nearest-even conversion
// (v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> one word of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// FP8 E4M3 (the OCP "fn" encoding: bias 7, max 448, no infinities), four
// values per 32-bit word, byte k holding element k.  gfx950's conversions use
// this encoding and round to nearest even; narrowing would give NaN from
// +-464 up, so finite values are clamped to +-448 first (saturation).
// Widening to fp32 (and from there to bf16) is exact.
__device__ __forceinline__ f32x2 fp8_lo2(uint32_t w) {  // elements 0, 1
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}
__device__ __forceinline__ f32x2 fp8_hi2(uint32_t w) {  // elements 2, 3
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
}
// Saturation to +-448 with gfx950's NaN-propagating minimum / maximum
// (v_minimum3_f32, v_maximum3_f32): a NaN stays NaN and converts to an E4M3
// NaN code (S.1111.111), where the plain clamp (v_med3_f32) would turn it
// into -448.  One instruction more per value than that clamp, no branch.
__device__ __forceinline__ float sat_e4m3(float x) {
  return __builtin_elementwise_maximum(__builtin_elementwise_minimum(x, 448.0f), -448.0f);
}
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
}
// The two halves of pack_fp8x4 on their own (elements 0-1 into a fresh word,
// elements 2-3 into the high half of w): the same bits, in two steps.
__device__ __forceinline__ uint32_t pack_fp8x2_lo(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
}
__device__ __forceinline__ uint32_t pack_fp8x2_hi(uint32_t w, float c, float d) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), (int)w, true);
}
// Eight E4M3 values (two words) -> the same eight values as bf16 (exact).
// gfx950's scaled OCP conversion with scale 1.0 widens a pair straight to
// bf16: one instruction per pair, bitwise what widening to fp32 and packing
// gives (checked on MI355X for all 65536 byte pairs, both word halves).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  const bf16x2 v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 w) {
  return u32x4{fp8x2_to_bf16x2(w[0], false), fp8x2_to_bf16x2(w[0], true),
               fp8x2_to_bf16x2(w[1], false), fp8x2_to_bf16x2(w[1], true)};
}

// The E4M3 post/res mix of one row at n = 4 on the matrix core:
// out_i[c] = sum_j H_res[i][j] x_j[c] + H_post[i] f[c] for each lane's own
// channel c, as v_mfma_f32_4x4x4bf16_1k (16 independent 4x4x4 blocks; lane
// 4b+j supplies column j of block b's B operand and receives column j of its
// D, lane 4b+i supplies row i of A -- checked on MI355X).  The column of a
// lane is its channel's four streams (E4M3, widened exactly to bf16); A is
// row (lane & 3) of H_res split into a bf16 high part and a bf16 low part
// (H = hi + lo to 2^-17 relative, the difference h - hi being exact in fp32),
// and H_post[lane & 3] as (hi, lo) against (f, f).  Products of bf16 values
// are exact in fp32.
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct Mix4A {
  s16x4 res_hi, res_lo, post;
};
__device__ __forceinline__ Mix4A mix4_a(float r0, float r1, float r2, float r3, float hpost) {
  const uint32_t h01 = pack_bf16x2(r0, r1), h23 = pack_bf16x2(r2, r3);
  const uint32_t l01 = pack_bf16x2(r0 - bf16_lo(h01), r1 - bf16_hi(h01));
  const uint32_t l23 = pack_bf16x2(r2 - bf16_lo(h23), r3 - bf16_hi(h23));
  const float ph = bf16_lo(pack_bf16x2(hpost, 0.f));
  const uint32_t pp = pack_bf16x2(ph, hpost - ph);
  Mix4A a;
  a.res_hi = __builtin_bit_cast(s16x4, u32x2{h01, h23});
  a.res_lo = __builtin_bit_cast(s16x4, u32x2{l01, l23});
  a.post = __builtin_bit_cast(s16x4, u32x2{pp, 0u});
  return a;
}
// Channels c, c+1 (bytes b, b+1 of each stream's word, b = 0 or 2) of four
// E4M3 stream words and the F word -> the two channels' mixed outputs
// (d[i] = stream i).
__device__ __forceinline__ void mix4_pair(const Mix4A &a, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                          uint32_t f, int b, f32x4 &d0, f32x4 &d1) {
  // v_perm_b32: selector bytes 0-3 pick the second source's bytes, 4-7 the first's.
  const uint32_t sel = (uint32_t)b | ((uint32_t)(4 + b) << 8) | ((uint32_t)(b + 1) << 16) | ((uint32_t)(5 + b) << 24);
  const uint32_t self = (uint32_t)b | ((uint32_t)b << 8) | ((uint32_t)(b + 1) << 16) | ((uint32_t)(b + 1) << 24);
  const uint32_t p01 = __builtin_amdgcn_perm(x1, x0, sel);  // x0[c] x1[c] x0[c+1] x1[c+1]
  const uint32_t p23 = __builtin_amdgcn_perm(x3, x2, sel);
  const uint32_t pf = __builtin_amdgcn_perm(f, f, self);    // f[c] f[c] f[c+1] f[c+1]
  const s16x4 b0 = __builtin_bit_cast(s16x4, u32x2{fp8x2_to_bf16x2(p01, false), fp8x2_to_bf16x2(p23, false)});
  const s16x4 b1 = __builtin_bit_cast(s16x4, u32x2{fp8x2_to_bf16x2(p01, true), fp8x2_to_bf16x2(p23, true)});
  const s16x4 g0 = __builtin_bit_cast(s16x4, u32x2{fp8x2_to_bf16x2(pf, false), 0u});
  const s16x4 g1 = __builtin_bit_cast(s16x4, u32x2{fp8x2_to_bf16x2(pf, true), 0u});
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a.res_hi, b0, z, 0, 0, 0);
  d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a.res_hi, b1, z, 0, 0, 0);
  d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a.res_lo, b0, d0, 0, 0, 0);
  d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a.res_lo, b1, d1, 0, 0, 0);
  d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a.post, g0, d0, 0, 0, 0);
  d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a.post, g1, d1, 0, 0, 0);
}

// 16-byte global load / store.  Streaming data is touched once, so stores
// carry the non-temporal hint.
__device__ __forceinline__ u32x4 load16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void store16_nt(void *p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void store16_plain(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

// Wave-uniform value (lets the compiler keep row-derived addresses in SGPRs
// and read per-row coefficients with scalar loads).
__device__ __forceinline__ int64_t uniform(int64_t v) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace mhc
