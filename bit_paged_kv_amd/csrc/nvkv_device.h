// Device-side helpers shared by the libnvkv kernels (gfx950 / CDNA4 only).
//
// Format (SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "The Core of the Ledger" paragraphs 1-2;
// SOAR Notes 05, "02 NVFP4 KV Cache"): 4-bit E2M1 codes two per byte, one OCP E4M3 scale per 16
// channels, one fp32 scale per tensor; dequantized value = e2m1 * e4m3 * g.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvkv {

constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kNvfp4DataBytes = 1024;   // one (page, head) block of packed E2M1 codes
constexpr int kNvfp4ScaleBytes = 128;   // one (page, head) block of E4M3 block scales
constexpr int kFp8Bytes = 2048;         // one (page, head) block of FP8 values

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------------
// Encoders (quantize-on-write).  Round to nearest, ties to the even mantissa, saturating to the
// largest finite magnitude; computed with exact power-of-two scalings and v_rndne_f32.
// ---------------------------------------------------------------------------------------------

// OCP E4M3 (bias 7, max 448, subnormal step 2^-9) byte of x, sign copied from x.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7Eu;            // saturate (448 and above)
  if (a < 0.015625f) {                               // below 2^-6: subnormal grid, step 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8; 8 is the smallest normal 0x08
  }
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6 .. 8
  const uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8 .. 16
  uint32_t code = ((uint32_t)(e + 7) << 3) + (m - 8u);   // m == 16 carries into the next binade
  code = code > 0x7Eu ? 0x7Eu : code;
  return sign | code;
}

// E4M3 bytes of fp32(x[i] / s) for four values (byte i of the result), bit-identical to
// e4m3_encode(x[i] / s) for every input; r = fp32(1 / s).
//  * q = x * r lies within 3 ulp of fp32(x / s).  The two can round to different E4M3 values only
//    next to a rounding midpoint of the normal range (fraction bits 19..0 near 0x80000), in the
//    subnormal range (0 < |q| < 2^-6, where the rounding position moves with the exponent), or when
//    x * r is NaN (x NaN, or 0 * inf for a tiny s).  A lane in any of these cases divides.
//  * gfx950's v_cvt_scalef32_pk_fp8_f32 with scale 1.0 rounds exactly like e4m3_encode for every
//    input of magnitude below 448 (compared on all 2^32 fp32 patterns); it does not saturate, so the
//    magnitude is clamped to 448 first, and fmin(NaN, 448) = 448 with the sign kept reproduces the
//    encoder's NaN -> signed maximum.
__device__ __forceinline__ uint32_t e4m3x4_div(const float* x, float s, float r) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  float q[4];
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[i] = x[i] * r;
    const float aq = fabsf(q[i]);
    const uint32_t key = (__float_as_uint(q[i]) & 0xFFFFFu) - (0x80000u - 4u);
    slow |= key <= 8u || (aq < 0.015625f && aq != 0.0f) || !(aq == aq);
  }
  if (slow) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = x[i] / s;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = __builtin_copysignf(fminf(fabsf(q[i]), 448.0f), q[i]);
  v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s){0, 0}, q[0], q[1], 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, q[2], q[3], 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

// Value of a non-negative E4M3 byte (0x00..0x7E) as fp32, exactly.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  return e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf((float)(8u + m), (int)e - 10);
}

// 3-bit E2M1 magnitude code of |y| (grid 0, .5, 1, 1.5 | 2, 3 | 4, 6), saturating at 6.
__device__ __forceinline__ uint32_t e2m1_encode_mag(float a) {
  if (a < 2.0f) return (uint32_t)__builtin_rintf(a * 2.0f);          // 0..4 (4 = value 2)
  if (a < 4.0f) return (uint32_t)__builtin_rintf(a) + 2u;            // 2,3,4 -> codes 4,5,6
  if (a < 6.0f) return (uint32_t)__builtin_rintf(a * 0.5f) + 4u;     // 2,3 -> codes 6,7
  return 7u;
}

// Block scale of a 16-value block with absolute maximum `amax`: returns the E4M3 byte of
// fp32(amax / fp32(6 g)) and the fp32 divisor fp32(s * g) of its elements (0 when the scale rounds
// to zero).  The quotient is taken as amax * rcp(6 g) (v_rcp_f32: within 1 ulp), within 3 ulps of
// the correctly rounded one; as in e4m3x4_div, the two can give different E4M3 bytes only next to
// a rounding midpoint of the normal range or in the subnormal range, and there (or for 6 g outside
// [2^-100, 2^100], or a NaN quotient) the lane divides.  The byte comes from the pack convert,
// after the clamp to 448 that gives the encoder's saturation (and NaN -> 0x7E).
__device__ __forceinline__ uint32_t nvfp4_block_scale(float amax, float g, float* den) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const float six_g = 6.0f * g;
  float u = amax * __builtin_amdgcn_rcpf(six_g);
  const uint32_t key = (__float_as_uint(u) & 0xFFFFFu) - (0x80000u - 8u);
  if (key <= 16u || (u < 0.015625f && u != 0.0f) || !(u == u) || !(six_g >= 0x1p-100f && six_g <= 0x1p100f))
    u = amax / six_g;                              // correctly rounded fp32 division
  const v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s){0, 0}, fminf(u, 448.0f), 0.0f, 1.0f, false);
  const uint32_t sc = __builtin_bit_cast(uint32_t, w) & 0xFFu;   // u >= 0: sign bit clear
  *den = e4m3_value(sc) * g;
  return sc;
}

// 4-bit code of one value given its block's divisor (sign in bit 3; signed zero when den == 0).
__device__ __forceinline__ uint32_t nvfp4_code(float x, float den) {
  const uint32_t sgn = (__float_as_uint(x) >> 28) & 8u;
  return sgn | (den == 0.0f ? 0u : e2m1_encode_mag(fabsf(x / den)));
}

// Quantize 16 fp32 values of one block.  Returns the E4M3 scale byte; the 4-bit E2M1 codes (sign
// in bit 3) come packed, element i in bits 4 (i % 8) of word i / 8 (lo: 0..7, hi: 8..15).  g is the
// tensor's global scale (> 0).
//
// The codes are those of the correctly rounded quotients fp32(x / den), without dividing per value:
//  * gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds an fp32 value to E2M1 exactly like the
//    encoder above (nearest, ties to the even code, saturating, sign kept; checked on the device for
//    every non-NaN fp32 bit pattern);
//  * for den in [2^-100, 2^100], q0 = x * rcp(den) (v_rcp_f32, within 1 ulp of 1 / den) is within 3
//    ulps of fp32(x / den), so the two can round to different E2M1 codes only if an E2M1 rounding
//    threshold (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) lies within 3 ulps of q0.  The test: the codes
//    of the floats 8 bit patterns below and above q0 agree (E2M1 rounding is monotonic in the
//    magnitude, and so in the pattern within one sign), so no threshold lies between them.  A
//    block where they differ for some value, or with den outside that range, takes the correctly
//    rounded division for all 16 values.  den == 0 (the block scale rounded to zero) gives signed
//    zero codes through q = x * 0.
__device__ __forceinline__ uint32_t nvfp4_quantize_block_packed(const float (&x)[16], float g, uint32_t& lo,
                                                                uint32_t& hi) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  float den;
  const uint32_t sc = nvfp4_block_scale(a, g, &den);
  float q[16];
  bool exact = den >= 0x1p-100f && den <= 0x1p100f;
  if (exact) {
    const float r = __builtin_amdgcn_rcpf(den);
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = x[i] * r;
    // codes of the patterns 8 below / 8 above each q0 (q0 = +-0 wraps to a NaN pattern below,
    // which at worst sends the block to the division)
    uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
    auto dn = [&](int i) { return __uint_as_float(__float_as_uint(q[i]) - 8u); };
    auto up = [&](int i) { return __uint_as_float(__float_as_uint(q[i]) + 8u); };
    lo0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo0, dn(0), dn(1), 1.0f, 0);
    lo0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo0, dn(2), dn(3), 1.0f, 1);
    lo0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo0, dn(4), dn(5), 1.0f, 2);
    lo0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo0, dn(6), dn(7), 1.0f, 3);
    lo1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo1, dn(8), dn(9), 1.0f, 0);
    lo1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo1, dn(10), dn(11), 1.0f, 1);
    lo1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo1, dn(12), dn(13), 1.0f, 2);
    lo1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo1, dn(14), dn(15), 1.0f, 3);
    hi0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi0, up(0), up(1), 1.0f, 0);
    hi0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi0, up(2), up(3), 1.0f, 1);
    hi0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi0, up(4), up(5), 1.0f, 2);
    hi0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi0, up(6), up(7), 1.0f, 3);
    hi1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi1, up(8), up(9), 1.0f, 0);
    hi1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi1, up(10), up(11), 1.0f, 1);
    hi1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi1, up(12), up(13), 1.0f, 2);
    hi1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi1, up(14), up(15), 1.0f, 3);
    exact = lo0 == hi0 && lo1 == hi1;
  }
  if (!exact) {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = den == 0.0f ? x[i] * 0.0f : x[i] / den;
  }
  uint32_t w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[0], q[1], 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[2], q[3], 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[4], q[5], 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[6], q[7], 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[8], q[9], 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[10], q[11], 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[12], q[13], 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[14], q[15], 1.0f, 3);
  lo = w0;
  hi = w1;
  return sc;
}

// ---------------------------------------------------------------------------------------------
// Input loaders
// ---------------------------------------------------------------------------------------------
// 8 bf16 values packed in a uint4 -> fp32 (exact)
__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------------------------------------
// gfx950 hardware converts used by the decode kernels.  With a scale operand of 1.0 they are exact
// decodes (checked exhaustively on the device): an E2M1 pair (one byte, low nibble first) or an
// E4M3 pair (one 16-bit half of a dword, low byte first) to two fp16 values.
// ---------------------------------------------------------------------------------------------
template <int BYTE>
__device__ __forceinline__ h2 fp4x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, BYTE);
}
template <bool HIGH>
__device__ __forceinline__ h2 fp8x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH);
}

__device__ __forceinline__ h8 cat4(h2 a, h2 b, h2 c, h2 d) {
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Wave-wide (64 lanes) butterfly maximum over the lanes that differ in the given xor bits.
__device__ __forceinline__ float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }

}  // namespace nvkv
