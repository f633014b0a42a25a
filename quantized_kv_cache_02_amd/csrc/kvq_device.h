// kvq_device.h -- gfx950 device helpers: bf16 handling, wave reductions,
// MFMA wrappers and the in-register code -> fp16 unpackers used by the decode
// kernel.  GPU code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_params.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 for finite inputs.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Butterflies across the 4 lane groups (lanes n, n+16, n+32, n+48) with the
// gfx950 row-swap permutes: each swap hands a lane its xor-16 / xor-32 partner
// in one of the two results, so max/sum of the pair is the butterfly step.  The
// two operands of every sum are in the same order on both lanes of a pair.
__device__ __forceinline__ float group_max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Byte permute of the 8 bytes {hi:lo}: selector byte k picks output byte k
// (0..3 = bytes of lo, 4..7 = bytes of hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Packed fp16 add (v_pk_add_f16).  16-bit packed math only; no packed fp32.
__device__ __forceinline__ uint32_t pk_add_h(uint32_t a, half2_t b) {
  return as_u32(as_h2(a) + b);
}

// ---------------------------------------------------------------------------
// Code -> fp16 unpacking.  The integer grids use one identity: the fp16 with
// bit pattern 0x64XY equals 1024 + 0xXY exactly (fp16 spacing at 1024 is 1).
//   int8: XY = c ^ 0x80 = c + 128, so 0x64XY - 1152 = c.
//   int4: XY = (n ^ 8) << 4 = 16 (n + 8), so 0x64XY - 1152 = 16 n; the factor 16
//         is folded into the scales by the caller.
// fp8 E4M3FN uses the hardware converter, exact for every finite code.
// ---------------------------------------------------------------------------

constexpr uint32_t kMagic = 0x64646464u;

// int8: one dword of 4 codes (c0..c3, low byte first) -> two packed fp16
// dwords (c0, c1), (c2, c3).
__device__ __forceinline__ void int8x4_to_h(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  uint32_t x = w ^ 0x80808080u;
  lo = pk_add_h(perm(kMagic, x, 0x04010400u), bias);
  hi = pk_add_h(perm(kMagic, x, 0x04030402u), bias);
}

// int4: one dword of 8 nibbles n0..n7 (n0 = low nibble of byte 0) -> four
// packed fp16 dwords holding 16*n in the order (n0,n2) (n4,n6) (n1,n3) (n5,n7).
__device__ __forceinline__ void int4x8_to_h(uint32_t w, uint32_t out[4]) {
  const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  uint32_t x = w ^ 0x88888888u;
  uint32_t ev = (x << 4) & 0xF0F0F0F0u;  // 16*(n_even+8) in each byte
  uint32_t od = x & 0xF0F0F0F0u;         // 16*(n_odd+8)
  out[0] = pk_add_h(perm(kMagic, ev, 0x04010400u), bias);
  out[1] = pk_add_h(perm(kMagic, ev, 0x04030402u), bias);
  out[2] = pk_add_h(perm(kMagic, od, 0x04010400u), bias);
  out[3] = pk_add_h(perm(kMagic, od, 0x04030402u), bias);
}

// fp8: one dword of 4 codes -> (c0, c1), (c2, c3) as packed fp16.
__device__ __forceinline__ void fp8x4_to_h(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  hi = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// ---------------------------------------------------------------------------
// MFMA wrappers (lane layouts checked on gfx950):
//   16x16x16 f16: A lane l = row l%16, k 4(l/16)+e;  B lane l = col l%16,
//                 k 4(l/16)+e;  C lane l = rows 4(l/16)+e, col l%16.
//   16x16x32 f16: as above with k 8(l/16)+e for A and B.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// bf16 MFMAs (same lane layouts as the fp16 ones above).  The operands travel
// as bit containers of the same width and are reinterpreted here.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4_t mfma32_bf16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16_bf16(u32x2_t a, u32x2_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                   __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
}

// Integer MFMA 16x16x64 i8: each lane holds 16 bytes of A (row l%16) and of B
// (column l%16); within a lane group l/16 the A and B bytes at the same
// position meet the same k (checked on gfx950), and C has the f32 layout.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t mfma64_i8(i32x4_t a, i32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Folded query of the integer caches: a row x (q times the per-channel K scale)
// with |x| < 2^ex becomes the integer vector qi = rne(x 2^(8 NSL - 2 - ex)),
// |qi| <= 2^(8 NSL - 2), written as NSL signed bytes, qi = sum_k 256^k s_k
// (balanced digits: s_0 .. s_{NSL-2} in [-128, 127], the top one in
// [-65, 64]).  Each byte is an int8 B operand; the integer dot products of the
// slices with the K codes are exact in int32 (|s| <= 128, |k| <= 127, 256
// channels) and combine into one float per logit (q_dot).  Two slices keep 15
// bits of the row's largest element, three 23: a channel 2^r below the largest
// keeps 15 - r or 23 - r bits.
//
// q_slice_bytes returns the slices as bytes 0 .. NSL-1 of one word: with the
// bias c = sum_{k < NSL-1} 128 * 256^k, u = qi + c has s_k + 128 as its byte k
// below the top (plain base-256 digits) and s_{NSL-1} as the rest, so the
// slice bytes are those of u with the bias bits flipped back.
template <int NSL>
__device__ __forceinline__ uint32_t q_slice_bytes(float x, int ex) {
  static_assert(NSL == 2 || NSL == 3, "two or three slices");
  constexpr uint32_t c = NSL == 2 ? 0x80u : 0x8080u;
  const int qi = (int)__builtin_rintf(ldexpf(x, 8 * NSL - 2 - ex));
  return ((uint32_t)qi + c) ^ c;
}

// Slice k of four consecutive values (their q_slice_bytes words w0..w3) as one
// B-operand dword: byte p is byte k of w_p.
__device__ __forceinline__ uint32_t slice_dword(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int k) {
  const uint32_t sel = (uint32_t)k | ((uint32_t)(4 + k) << 8);
  return perm(perm(w3, w2, sel), perm(w1, w0, sel), 0x05040100u);
}

// The softmax weights of a row are exp2(z - m) for a reference m that moves
// only when a logit exceeds it by more than this (log2 units): the weights stay
// below 2^8 -- exact in the fp16 (and bf16 hi + lo) P operand up to its usual
// rounding, far from fp16's 65504 -- and the accumulators are rescaled a few
// times per wavefront instead of on a large share of tiles.  Every merge
// weighs a partial by its own reference.
constexpr float kLazyHeadroom = 8.0f;

// The dot product of the folded query with the codes from the per-slice int32
// dot products (dots[k] for slice k): exact integers, one rounding to fp32 at
// the end (two slices: the sum is below 2^30 and exact in int32).
template <int NSL>
__device__ __forceinline__ float q_dot(const int (&dots)[NSL]) {
  if constexpr (NSL == 2)
    return (float)(dots[1] * 256 + dots[0]);
  else
    return (float)dots[2] * 65536.0f + (float)(dots[1] * 256 + dots[0]);
}

__device__ __forceinline__ half4_t u2_to_h4(uint32_t a, uint32_t b) {
  u32x2_t v = {a, b};
  return __builtin_bit_cast(half4_t, v);
}
__device__ __forceinline__ half8_t u4_to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(half8_t, v);
}

// Transpose 4 token rows x 4 bytes (one dword each) into MFMA B operands:
// out[q] = (token0, token1, token2, token3) of byte q, q = 0..3, as fp16.
template <int KIND>  // 0: biased magic bytes (int8 after xor, int4 nibbles), 1: fp8
__device__ __forceinline__ void v_transpose4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             half4_t out[4]) {
  const uint32_t s01lo = perm(r1, r0, 0x05010400u);  // (r0.b0, r1.b0, r0.b1, r1.b1)
  const uint32_t s01hi = perm(r1, r0, 0x07030602u);  // (r0.b2, r1.b2, r0.b3, r1.b3)
  const uint32_t s23lo = perm(r3, r2, 0x05010400u);
  const uint32_t s23hi = perm(r3, r2, 0x07030602u);
  if constexpr (KIND == 1) {
    out[0] = u2_to_h4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s01lo, 1.0f, false)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s23lo, 1.0f, false)));
    out[1] = u2_to_h4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s01lo, 1.0f, true)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s23lo, 1.0f, true)));
    out[2] = u2_to_h4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s01hi, 1.0f, false)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s23hi, 1.0f, false)));
    out[3] = u2_to_h4(as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s01hi, 1.0f, true)),
                      as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s23hi, 1.0f, true)));
  } else {
    const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    out[0] = u2_to_h4(pk_add_h(perm(kMagic, s01lo, 0x04010400u), bias),
                      pk_add_h(perm(kMagic, s23lo, 0x04010400u), bias));
    out[1] = u2_to_h4(pk_add_h(perm(kMagic, s01lo, 0x04030402u), bias),
                      pk_add_h(perm(kMagic, s23lo, 0x04030402u), bias));
    out[2] = u2_to_h4(pk_add_h(perm(kMagic, s01hi, 0x04010400u), bias),
                      pk_add_h(perm(kMagic, s23hi, 0x04010400u), bias));
    out[3] = u2_to_h4(pk_add_h(perm(kMagic, s01hi, 0x04030402u), bias),
                      pk_add_h(perm(kMagic, s23hi, 0x04030402u), bias));
  }
}

}  // namespace kvq
