// Device-side building blocks of the fused int4 MoE layer for gfx950.
//
// Operand format ("A-format"): activations that feed the MFMA contraction are
// stored as fp16 scaled per token by a power of two (each token's hidden row
// times 2^-e so that its largest |value| lies in [1, 2); its h row times
// 2^-2e), and inside every run of 8 consecutive inputs the values are
// kept in the order of input offsets {0,4,1,5,2,6,3,7}, with the values at
// odd offsets divided by 16 (exact for normal fp16 values).  That matches
// dq8() below, which produces decoded weights from one 32-bit word of packed
// codes in that order and with the odd offsets multiplied by 16, so an
// activation fragment and a weight fragment pair up element by element with
// no shuffling and the products are unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Position p of an 8-run holds input offset perm8(p) (0,4,1,5,2,6,3,7);
// input offset o sits at position inv_perm8(o) (0,2,4,6,1,3,5,7).
__host__ __device__ constexpr int perm8(int p) { return (p >> 1) | ((p & 1) << 2); }
__host__ __device__ constexpr int inv_perm8(int o) { return ((o & 3) << 1) | (o >> 2); }

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  // one VALU op; register operands (gfx9 VOP3 encodings take no literals)
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// Decode 8 packed int4 codes (nibble j of v = input offset j) with one fp16
// group scale into 8 fp16 operands, in A-format order.
//
// A nibble OR-ed into the mantissa of the fp16 constant 1024.0 gives 1024+q
// exactly (bits 0-3) or 1024+16q exactly (bits 4-7, still inside the 10-bit
// mantissa).  Subtracting 1032 (resp. 1152) leaves q-8 (resp. 16(q-8))
// exactly, and one packed multiply by the scale rounds to nearest even.  The
// odd input offsets thus carry 16*(q-8)*s, which the A-format compensates.
// Per 8 codes: 1 shift, 4 and-or, 4 packed adds, 4 packed multiplies.
// s2: the fp16 scale in both halves of a dword.
__device__ __forceinline__ half8_t dq8p(uint32_t v, uint32_t s2) {
  const uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u, kMagic = 0x64006400u;
  const half2_t b_lo = as_half2(0xE408E408u);  // (-1032, -1032)
  const half2_t b_hi = as_half2(0xE480E480u);  // (-1152, -1152)
  const half2_t s = as_half2(s2);
  const uint32_t v8 = v >> 8;
  const half2_t p0 = (as_half2(and_or(v, kLo, kMagic)) + b_lo) * s;   // offsets 0, 4
  const half2_t p1 = (as_half2(and_or(v, kHi, kMagic)) + b_hi) * s;   // 1, 5 (x16)
  const half2_t p2 = (as_half2(and_or(v8, kLo, kMagic)) + b_lo) * s;  // 2, 6
  const half2_t p3 = (as_half2(and_or(v8, kHi, kMagic)) + b_hi) * s;  // 3, 7 (x16)
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// scale_bits: one fp16 scale in the low 16 bits.
__device__ __forceinline__ half8_t dq8(uint32_t v, uint32_t scale_bits) {
  return dq8p(v, (scale_bits & 0xFFFFu) | (scale_bits << 16));
}

// Position p of an 8-run carries a value scaled by 16 when its input offset
// perm8(p) is odd, i.e. for p in {2, 3, 6, 7}.
__host__ __device__ constexpr bool x16_pos(int p) { return (p & 2) != 0; }

// bf16 pair (one 32-bit word, element 0 in the low half) -> two floats.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// 2^n as a float, for n in [-126, 127] (built from the exponent field).
__device__ __forceinline__ float pow2f(int n) { return __int_as_float((n + 127) << 23); }
// 1/p for p = 2^n, n in [-126, 126] (exact; no division).
__device__ __forceinline__ float inv_pow2f(float p) { return __int_as_float(0x7F000000 - __float_as_int(p)); }

// Tile order of the weight codes (the library's copy; rows of K2 = K/2
// bytes, K a multiple of 128): each 16-row block's codes are stored
// sub-step by sub-step (128 inputs: 64 bytes of each of its 16 rows, 1 KiB),
// and within a sub-step lane l = 16 kq + r's 16 bytes (row r, bytes
// 16 kq .. 16 kq + 15 of the sub-step) sit at 16 l: the order in which one
// wave's load instruction of an MFMA tile reads them, so that instruction
// reads 1 KiB contiguous.  Byte offset of code byte b of row n:
__host__ __device__ constexpr size_t tiled_code_offset(size_t n, size_t b, size_t K2) {
  return (n / 16) * 16 * K2 + (b / 64) * 1024 + (((b % 64) / 16) * 16 + n % 16) * 16 + b % 16;
}

// Tile order of the group scales (the layer's copy; KG = K/32 groups per
// row, a multiple of 4): each 16-row block's scales stored super-step by
// super-step (16 groups: 32 bytes of each of its rows, 512 bytes), and
// within a super-step lane l = 16 kq + r's 8 bytes (row r, groups
// 4 kq .. 4 kq + 3 of the super-step) at 8 l, so one 8-byte load per lane
// reads a block's super-step of scales as 512 contiguous bytes.  Byte
// offset of the scale of group g of row n:
__host__ __device__ constexpr size_t tiled_scale_offset(size_t n, size_t g, size_t KG) {
  return (n / 16) * 16 * KG * 2 + (g / 16) * 512 + (((g % 16) / 4) * 16 + n % 16) * 8 + (g % 4) * 2;
}

// h = SiLU(g) * u as stored: the product rounded to fp32, then to fp16.  The
// empty asm pins the fp32 value, so the compiler cannot fuse the product into
// the conversion (one rounding instead of two) in some kernels or
// instantiations and not in others: every path gives the same bits.
__device__ __forceinline__ _Float16 silu_mul_h(float gt, float up) {
  float hv = gt / (1.0f + __expf(-gt)) * up;
  asm volatile("" : "+v"(hv));
  return (_Float16)hv;
}

// Largest |value| of 8 bf16 (one 16-byte run) as a magnitude bit pattern:
// for finite values the order of the 15-bit patterns is the order of the
// magnitudes.
__device__ __forceinline__ uint32_t absmax_bf16x8(uint4 in) {
  uint32_t m = 0;
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
    m = lo > m ? lo : m;
    m = hi > m ? hi : m;
  }
  return m;
}

// Exponent e of a token row whose largest |x| has the bf16 magnitude pattern
// amax: 2^e <= amax < 2^(e+1), so the row times 2^-e has its largest value
// in [1, 2).  A row of zeros gets e = 0; e is clamped to [-kExpClamp,
// kExpClamp] so that 2^(+-2e) stays a normal float.
constexpr int kExpClamp = 60;
__device__ __forceinline__ int row_exponent(uint32_t amax) {
  if (amax == 0) return 0;
  const int field = (int)(amax >> 7);  // bf16 exponent field (8 bits)
  const int e = field == 0 ? -127 : field - 127;
  return e < -kExpClamp ? -kExpClamp : (e > kExpClamp ? kExpClamp : e);
}

// 8 bf16 (natural order) times sc (a power of two) -> 8 fp16 in A-format
// order.  bf16 -> fp32 is exact, the scaling and the division of the odd
// offsets by 16 are exact, and fp32 -> fp16 is exact for results inside the
// fp16 normal range (rounded to nearest even below it).
__device__ __forceinline__ uint4 bf16x8_to_aformat(uint4 in, float sc) {
  const float so = sc * 0.0625f;
  float f[8];
  f[0] = bf16_lo(in.x) * sc; f[1] = bf16_hi(in.x) * so;
  f[2] = bf16_lo(in.y) * sc; f[3] = bf16_hi(in.y) * so;
  f[4] = bf16_lo(in.z) * sc; f[5] = bf16_hi(in.z) * so;
  f[6] = bf16_lo(in.w) * sc; f[7] = bf16_hi(in.w) * so;
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

// Inverse of ordered_key (a -0 input comes back as +0).
__device__ __forceinline__ float from_ordered_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Maximum of a 32-bit value over the 64 lanes of a wave, returned to every
// lane.  DPP steps (quad permutes, row mirrors, row broadcasts) combine
// lanes within and across rows of 16 without going through LDS; lane 63
// ends with the maximum, which readlane broadcasts.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max_step_u32(uint32_t v) {
  const uint32_t p = __builtin_amdgcn_update_dpp(v, v, kCtrl, kRowMask, 0xF, false);
  return p > v ? p : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step_u32<0xB1, 0xF>(v);
  v = dpp_max_step_u32<0x4E, 0xF>(v);
  v = dpp_max_step_u32<0x141, 0xF>(v);
  v = dpp_max_step_u32<0x140, 0xF>(v);
  v = dpp_max_step_u32<0x142, 0xA>(v);
  v = dpp_max_step_u32<0x143, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Inclusive prefix sum over the wave's 64 lanes by DPP: shifts by 1, 2, 4
// and 8 lanes within each row of 16 (lanes shifted in from outside the row
// add 0), then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// and the total of rows 0-1 into rows 2-3 (row_bcast:31).  Rows a step does
// not write keep `old` = 0 and add nothing.
template <int kCtrl, int kRowMask, bool kBound>
__device__ __forceinline__ int dpp_add_step(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xF, kBound);
}
__device__ __forceinline__ int wave_incl_scan_add(int v) {
  v = dpp_add_step<0x111, 0xF, true>(v);   // row_shr:1
  v = dpp_add_step<0x112, 0xF, true>(v);   // row_shr:2
  v = dpp_add_step<0x114, 0xF, true>(v);   // row_shr:4
  v = dpp_add_step<0x118, 0xF, true>(v);   // row_shr:8
  v = dpp_add_step<0x142, 0xA, false>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add_step<0x143, 0xC, false>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace qmoe
