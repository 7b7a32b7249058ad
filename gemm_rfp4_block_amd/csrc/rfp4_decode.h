// Device-side decode of ROCmFP4 blocks for gfx950.
//
// Format ("Feasibility Report: Porting ROCmFP4 to Atlas", "What is ROCmFP4?"):
//   * "Block Layout": 16 bytes qs of 4-bit indices, then e[2] (dual) or e (fast).
//     Index t (0..15) is the low nibble of qs[t], index t+16 its high nibble, so the
//     low nibbles form the first 16-weight half and the high nibbles the second.
//   * "Codebook10 Value Table": index bit 3 is the sign, bits 0..2 select a magnitude
//     in {0, 1, 2, 3, 4, 6, 8, 10}.
//   * "Scale Format": unsigned E4M3 scale byte, decoded to half of its E4M3 value.
//
// Decode strategy. A 32-bit word of qs holds eight indices: the low nibbles of its
// four bytes (four consecutive weights of the first half) and the high nibbles
// (four weights of the second half). One v_perm_b32 maps four 3-bit magnitudes at
// once through an 8-entry byte table holding the E4M3 encodings of the magnitudes;
// the sign bit of each index is then moved to bit 7 of its byte. The result is four
// E4M3 bytes in weight order, which gfx950's v_cvt_scalef32_pk_{f16,bf16,f32}_fp8
// turns into pairs of f16/bf16/f32 values exactly (every codebook value is an E4M3
// value). Those conversions apply only the exponent of their fp32 scale operand, so
// the decoded scale is applied separately, as an fp32 multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// E4M3 encodings of the magnitudes 0, 1, 2, 3 (low word, byte 0 first) and
// 4, 6, 8, 10 (high word): 0x00, 0x38, 0x40, 0x44 | 0x48, 0x4C, 0x50, 0x52.
constexpr uint32_t kMagE4m3Lo = 0x44403800u;
constexpr uint32_t kMagE4m3Hi = 0x52504C48u;

// E4M3 encodings of half the magnitudes: 0, 0.5, 1, 1.5 (low word) and 2, 3, 4, 5
// (high word). With these codes a weight is the product of its code and the full E4M3
// value of the scale byte (the decoded scale is half of it).
constexpr uint32_t kHalfE4m3Lo = 0x3C383000u;
constexpr uint32_t kHalfE4m3Hi = 0x4A484440u;

// Four E4M3 codes of half-weights (byte i = low nibble of byte i of q).
__device__ __forceinline__ uint32_t half_codes_low(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kHalfE4m3Hi, kHalfE4m3Lo, q & 0x07070707u);
  return mag | ((q << 4) & 0x80808080u);
}

// Four E4M3 codes of half-weights (byte i = high nibble of byte i of q).
__device__ __forceinline__ uint32_t half_codes_high(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kHalfE4m3Hi, kHalfE4m3Lo, (q >> 4) & 0x07070707u);
  return mag | (q & 0x80808080u);
}

// Four E4M3 codes (byte i = weight of the low nibble of byte i of q).
__device__ __forceinline__ uint32_t codes_low(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kMagE4m3Hi, kMagE4m3Lo, q & 0x07070707u);
  return mag | ((q << 4) & 0x80808080u);
}

// Four E4M3 codes (byte i = weight of the high nibble of byte i of q).
__device__ __forceinline__ uint32_t codes_high(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kMagE4m3Hi, kMagE4m3Lo, (q >> 4) & 0x07070707u);
  return mag | (q & 0x80808080u);
}

// Exact variants for bit-exact dequantization: index 8 is the integer 0 of the
// codebook, so its product with a scale is +0.0, not -0.0. The sign bit is kept
// only in bytes whose magnitude is non-zero (magnitude bytes are <= 0x52, so adding
// 0x7F sets bit 7 exactly when the byte is non-zero, with no carry between bytes).
__device__ __forceinline__ uint32_t keep_nonzero_sign(uint32_t mag, uint32_t sign) {
  return mag | (sign & (mag + 0x7F7F7F7Fu) & 0x80808080u);
}

__device__ __forceinline__ uint32_t codes_low_exact(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kMagE4m3Hi, kMagE4m3Lo, q & 0x07070707u);
  return keep_nonzero_sign(mag, q << 4);
}

__device__ __forceinline__ uint32_t codes_high_exact(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kMagE4m3Hi, kMagE4m3Lo, (q >> 4) & 0x07070707u);
  return keep_nonzero_sign(mag, q);
}

// Decoded scale S(b) = E4M3(b & 0x7F) / 2 computed with integer operations only, so
// that every byte (including exponent field 0 and 0x7F) follows the bit formula:
//   exponent field e >= 1: 2^(e-8) * (1 + m/8)    (fp32 exponent field e + 119)
//   exponent field e == 0: m * 2^-10
__device__ __forceinline__ float scale_exact(uint32_t b) {
  const uint32_t u = b & 0x7Fu;
  const uint32_t e = u >> 3;
  const float normal = __uint_as_float((u << 20) + (119u << 23));
  const float sub = static_cast<float>(u & 7u) * 0x1p-10f;
  return e != 0 ? normal : sub;
}

// E4M3 value of the low seven bits of byte `sel` of `word`, via the hardware FP8
// converter (twice the decoded scale). Only valid for finite bytes: rows must have
// passed validation, as the format requires.
template <int SEL>
__device__ __forceinline__ float e4m3_hw(uint32_t word_masked) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word_masked), SEL);
}

__device__ __forceinline__ f16x2 pair_f16(uint32_t codes, bool hi_word) {
  return hi_word ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false);
}

__device__ __forceinline__ bf16x2 pair_bf16(uint32_t codes, bool hi_word) {
  return hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
}

__device__ __forceinline__ f32x2 pair_f32(uint32_t codes, bool hi_word) {
  return hi_word ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, 1.0f, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, 1.0f, false);
}

// Unaligned loads (gfx950 runs in unaligned access mode for global memory).
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  uint4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}

__device__ __forceinline__ uint32_t load4(const uint8_t* p) {
  uint32_t v;
  __builtin_memcpy(&v, p, 4);
  return v;
}

}  // namespace rfp4
