// Device-side building blocks shared by the gfx950 kernels of libmla: vector types, the in-register
// dequantisation of record chunks, and a few wave-level helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 512;
constexpr int kFp8Rec = 528;      // 512 e4m3 + 16 e8m0
constexpr int kFp4Rec = 288;      // 256 packed e2m1 + 32 e4m3
constexpr int kFp8Chunks = 33;    // 16-byte chunks per fp8 record (32 data + 1 scale chunk)
constexpr int kFp4Chunks = 18;    // 16 data chunks + 2 scale chunks
constexpr int kUnitTokens = 64;   // scheduling unit
constexpr int kSubTokens = 32;    // kernel tile: tokens per sub-tile

__device__ __forceinline__ bf16x8 cat4(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 e4m3 values (the words w0, w1: element i in byte i) -> bf16 with one e8m0 scale. gfx950's
// scaled convert reads only the exponent field of its f32 scale operand and applies it as
// 2^(e - 127), so placing the e8m0 byte in that field gives exactly x * 2^(byte - 127) rounded once
// to bf16 (exact whenever the product is representable, NaN for the e8m0 NaN byte 0xFF). Both
// decode kernels and the dequant probe run this routine.
__device__ __forceinline__ bf16x8 dequant_fp8_8(uint32_t w0, uint32_t w1, uint32_t scale_byte) {
  const float s = __builtin_bit_cast(float, scale_byte << 23);
  return cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true));
}

// fp8 chunk -> bf16: `raw` holds 16 consecutive e4m3 values of one record, all sharing the e8m0
// scale `scale_byte` (two dequant_fp8_8 halves).
__device__ __forceinline__ void dequant_fp8_16(u32x4 raw, uint32_t scale_byte, bf16x8& lo,
                                               bf16x8& hi) {
  lo = dequant_fp8_8(raw[0], raw[1], scale_byte);
  hi = dequant_fp8_8(raw[2], raw[3], scale_byte);
}

// e4m3 byte (low 8 bits of `b`) -> f32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b & 0xFFu, 1.0f, false)[0];
}

// Two e2m1 values of byte `B` of `w` -> bf16 pair times an e4m3 scale value. The scaled convert
// only honours power-of-two scales, so the e4m3 scale is applied as an f32 multiply; e2m1 * e4m3
// has at most 6 significant bits, so the product and its bf16 rounding are exact.
template <int B>
__device__ __forceinline__ bf16x2 fp4_byte(uint32_t w, float scale) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  bf16x2 r;
  r[0] = (__bf16)(v[0] * scale);
  r[1] = (__bf16)(v[1] * scale);
  return r;
}

// fp4 half-chunk -> bf16: `w0`,`w1` hold 8 bytes = 16 e2m1 values (element 2k in the low nibble of
// byte k), all sharing the e4m3 scale value `scale`.
__device__ __forceinline__ void dequant_fp4_16(uint32_t w0, uint32_t w1, float scale, bf16x8& lo,
                                               bf16x8& hi) {
  lo = cat4(fp4_byte<0>(w0, scale), fp4_byte<1>(w0, scale), fp4_byte<2>(w0, scale),
            fp4_byte<3>(w0, scale));
  hi = cat4(fp4_byte<0>(w1, scale), fp4_byte<1>(w1, scale), fp4_byte<2>(w1, scale),
            fp4_byte<3>(w1, scale));
}

// Nearest e4m3 code of a finite f32 (ties to even), saturating at +-448, sign kept.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {
    // below 2^-6, the subnormal grid m * 2^-9 (m = 8 is the smallest normal, code 0x08)
    code = (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
  } else {
    // drop 20 of the 23 mantissa bits, rounding to nearest with ties to even (a carry moves into
    // the exponent field), then rebias the exponent from 127 to 7
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return sign | code;
}

// Four f32 values / 2^k -> four e4m3 codes (value i in byte i), with gfx950's scaled conversion:
// it divides by its scale operand and rounds to nearest, ties to even, keeping subnormals and the
// sign, exactly as e4m3_code does for results within +-448 (checked over every e4m3 value, every
// midpoint and its neighbours, and random values). The caller guarantees |v / 2^k| <= 448 (beyond,
// the conversion gives NaN rather than saturating). k = -127 has no normal f32 scale: the values
// are doubled (exact) and divided by 2^-126.
__device__ __forceinline__ uint32_t e4m3_codes4(float v0, float v1, float v2, float v3, int k) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  if (k < -126) {
    v0 *= 2.0f; v1 *= 2.0f; v2 *= 2.0f; v3 *= 2.0f;
    k = -126;
  }
  const float sc = __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
  v2s r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v0, v1, sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v2, v3, sc, true);
  return __builtin_bit_cast(uint32_t, r);
}

// k = ceil(log2(a / 448)) for a finite a >= 0, clipped to [-127, 127]; 0 for a = 0. With
// a = M * 2^E, M in [1, 2): k = E - 8 if M <= 1.75, else E - 7 (448 = 1.75 * 2^8). fp32 subnormals
// (a < 2^-126) give k <= -134, clipped to -127.
__device__ __forceinline__ int fp8_block_exponent(float a) {
  const uint32_t u = __builtin_bit_cast(uint32_t, a);
  if (u == 0) return 0;
  const int e_field = (int)(u >> 23);
  if (e_field == 0) return -127;
  const int k = e_field - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return k < -127 ? -127 : k;
}

// Pairwise reduction with the lane 32 apart (lane l <-> l ^ 32) via v_permlane32_swap.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

}  // namespace mla
