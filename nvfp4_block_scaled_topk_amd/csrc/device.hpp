// device.hpp -- gfx950 device helpers shared by the kernels: element decoders,
// bf16 rounding, MFMA operand types.
//
// NVFP4 weights are decoded in registers from their stored bytes (two E2M1 codes a
// byte, one E4M3 scale per 16 elements [FP4-Local checkpoints on DGX Spark, §4
// Round 1, #489 / #517]) straight into bf16 MFMA operands. The product of an E2M1
// value (<= 2 significant bits) and an E4M3 scale (<= 4 bits) has at most 6
// significant bits and lies in [2^-10, 2688], so the decoded weight is exact in
// bf16 and the matrix cores see the stored weight without rounding.
//
// gfx950's scaled FP4/FP8 conversions apply only the exponent of their fp32 scale
// operand. The E4M3 scale is therefore split into a power of two (given to the
// conversion) and its significand scaled into [0.5, 1) (one fp32 multiply per
// element); both steps are exact.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Round-to-nearest-even of an fp32 value to bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

// An E4M3 block scale v, prepared once per block: `pow2` is 2v, whose exponent (one
// above v's own) is what the hardware conversion applies; `mant` = v / 2^(e + 1) in
// [0.5, 1) with v's sign (0 for a zero scale), so fp4 * 2^(e + 1) * mant = fp4 * v, and
// both products are exact (the significand of v has at most 4 bits).
struct E4M3Split {
  float pow2;
  float mant;
};

// the scale in byte SEL of `word`
template <int SEL>
__device__ __forceinline__ E4M3Split e4m3_split_b(uint32_t word) {
  const float v = __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);  // exact decode of the E4M3 byte
  E4M3Split s;
  s.pow2 = v + v;
  s.mant = __builtin_amdgcn_frexp_mantf(v);
  return s;
}
__device__ __forceinline__ E4M3Split e4m3_split(uint32_t code) { return e4m3_split_b<0>(code); }

// 8 E2M1 codes (one 32-bit word, element 2j in the low nibble of byte j) times one
// E4M3 scale -> 8 bf16 values as an MFMA operand, exactly.
template <int SEL>
__device__ __forceinline__ uint32_t nvfp4x2_to_bf16x2(uint32_t codes, E4M3Split s) {
  const floatx2 p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, s.pow2, SEL);
  const float lo = p.x * s.mant;
  const float hi = p.y * s.mant;
  // both products are exact bf16 values: keep their upper halves
  return __builtin_amdgcn_perm(f32_bits(hi), f32_bits(lo), 0x07060302u);
}

__device__ __forceinline__ bf16x8 nvfp4x8_to_bf16(uint32_t codes, E4M3Split s) {
  uint32_t r[4] = {nvfp4x2_to_bf16x2<0>(codes, s), nvfp4x2_to_bf16x2<1>(codes, s),
                   nvfp4x2_to_bf16x2<2>(codes, s), nvfp4x2_to_bf16x2<3>(codes, s)};
  return __builtin_bit_cast(bf16x8, r);
}

// 8 E4M3 codes (two 32-bit words) times one E8M0 scale -> 8 bf16 values, exactly
// (E4M3 has 4 significant bits; the power-of-two scale goes to the conversion).
__device__ __forceinline__ bf16x8 mxfp8x8_to_bf16(uint32_t w0, uint32_t w1, float pow2) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, pow2, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, pow2, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, pow2, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, pow2, true);
  uint32_t r[4] = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, r);
}

// E8M0 code -> the fp32 whose exponent field is that code (what the scaled
// conversions read).
__device__ __forceinline__ float e8m0_pow2(uint32_t code) { return bits_f32(code << 23); }

__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ u32x4 ldg_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Weight bytes stream through once per call: their loads carry the non-temporal hint
// (the cache-policy operand of the buffer intrinsics, nt on global loads), which
// measured faster for these streams than the default policy.
constexpr int kWeightAux = 2;  // buffer-intrinsic cache policy: nt
__device__ __forceinline__ u32x4 ldg_nt_u32x4(const void* p) {
  typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
  const u32x4n v = __builtin_nontemporal_load(reinterpret_cast<const u32x4n*>(p));
  return u32x4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word_of(const u32x4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

}  // namespace moe
