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
