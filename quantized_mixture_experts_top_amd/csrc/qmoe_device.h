// Device-side building blocks of the fused int4 MoE layer for gfx950.
//
// Operand format ("A-format"): activations that feed the MFMA contraction are
// stored as fp16, and inside every run of 8 consecutive inputs the values are
// kept in the order of input offsets {0,4,1,5,2,6,3,7}.  That is the order in
// which dq8() below produces decoded weights from one 32-bit word of packed
// codes, so an activation fragment and a weight fragment pair up element by
// element without any shuffling in the inner loop.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

// Position p of an 8-run holds input offset perm8(p) (0,4,1,5,2,6,3,7);
// input offset o sits at position inv_perm8(o) (0,2,4,6,1,3,5,7).
__host__ __device__ constexpr int perm8(int p) { return (p >> 1) | ((p & 1) << 2); }
__host__ __device__ constexpr int inv_perm8(int o) { return ((o & 3) << 1) | (o >> 2); }

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Decode 8 packed int4 codes (nibble j of v = input offset j) with one fp16
// group scale into 8 fp16 operands, in A-format order.
//
// Each nibble is OR-ed into the mantissa of the fp16 constant 1024.0 (whose
// unit in the last place is 1), giving 1024+q exactly; subtracting 1032
// leaves q-8 exactly; one packed multiply by the scale rounds (q-8)*s to
// nearest even.  Two packed fp16 operations per pair of weights, plus the
// mask/shift that extracts the nibbles.
__device__ __forceinline__ half8_t dq8(uint32_t v, uint32_t scale_bits) {
  const uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
  const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t s = as_half2(scale_bits | (scale_bits << 16));
  half2_t p0 = (as_half2((v & kMask) | kMagic) + bias) * s;          // offsets 0, 4
  half2_t p1 = (as_half2(((v >> 4) & kMask) | kMagic) + bias) * s;   // 1, 5
  half2_t p2 = (as_half2(((v >> 8) & kMask) | kMagic) + bias) * s;   // 2, 6
  half2_t p3 = (as_half2(((v >> 12) & kMask) | kMagic) + bias) * s;  // 3, 7
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// bf16 pair (one 32-bit word, element 0 in the low half) -> two floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// 8 bf16 (natural order) -> 8 fp16 in A-format order.  bf16 -> fp32 is
// exact and fp32 -> fp16 is exact for values inside the fp16 range.
__device__ __forceinline__ uint4 bf16x8_to_aformat(uint4 in) {
  float f[8];
  f[0] = bf16_lo(in.x); f[1] = bf16_hi(in.x);
  f[2] = bf16_lo(in.y); f[3] = bf16_hi(in.y);
  f[4] = bf16_lo(in.z); f[5] = bf16_hi(in.z);
  f[6] = bf16_lo(in.w); f[7] = bf16_hi(in.w);
  half2_t o0 = {(_Float16)f[0], (_Float16)f[4]};
  half2_t o1 = {(_Float16)f[1], (_Float16)f[5]};
  half2_t o2 = {(_Float16)f[2], (_Float16)f[6]};
  half2_t o3 = {(_Float16)f[3], (_Float16)f[7]};
  return make_uint4(as_u32(o0), as_u32(o1), as_u32(o2), as_u32(o3));
}

// Order-preserving map of a finite float to uint32 (-0 folded onto +0, so
// the two zeros tie and the lower expert index wins, as for equal values).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace qmoe
