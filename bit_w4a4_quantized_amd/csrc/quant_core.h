// Device-side quantizer core for gfx950: absmax group scales, round-half-even
// codes, E4M3 / E2M1 encoders and nibble packing.
//
// The group quantization rule is the per-group symmetric quantization of the
// practice page "sota-314", section "Do this" (INT4 group 64 with 16-bit
// scales, NVFP4 group 16 with FP8 scales).  The exact arithmetic:
//   INT  : s16 = fp16_rne(fp32(absmax) / qmax); code = clamp(rint(fp32(v) / s), +-qmax)
//   FP4  : s8  = e4m3_rne_sat(fp32(absmax) / 6); code = nearest E2M1 (even-mantissa ties)
// Divisions are IEEE fp32 (correctly rounded: the HIP default without
// fast-math); rintf is round-half-even; fp32 -> fp16 conversion is RNE with
// subnormals kept.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace svdq {

// fp16 scale for an INT group: returns the fp16 bits and the scale as float.
__device__ __forceinline__ float int_scale(float amax, float qmax, uint16_t* bits) {
  __half h = __float2half_rn(amax / qmax);
  *bits = __half_as_ushort(h);
  return __half2float(h);
}

// Code of one value against a stored scale s (s == 0 -> 0).
__device__ __forceinline__ int int_code(float v, float s, float qmax) {
  if (s == 0.0f) return 0;
  float t = rintf(v / s);
  t = fminf(fmaxf(t, -qmax), qmax);
  return (int)t;
}

// fp16 scale of an INT group whose absmax is an fp16 value, without the division:
// fp16_rne(amax * RN(1/qmax)) == fp16_rne(RN(amax / qmax)) for qmax in {7, 127}.
// The product is within one fp32 ulp of amax / qmax, and amax / qmax is never within
// 32 ulps of a point where fp16 rounding changes, a midpoint m = (2k+1) g of the fp16
// grid (spacing 2g): qmax m is an odd multiple of g and amax (at least as coarse a grid)
// an even one, so |amax / qmax - m| >= g / qmax, while an fp32 ulp at m is at most
// g 2^-12 (subnormal fp16 range included).
__device__ __forceinline__ float int_scale_f16in(float amax, float inv_qmax, uint16_t* bits) {
  __half h = __float2half_rn(amax * inv_qmax);
  *bits = __half_as_ushort(h);
  return __half2float(h);
}

// RN(x / s) for fp16 values x and s != 0 (as floats; s may also be an E4M3 value), given
// r = v_rcp_f32(s) (within one ulp of 1/s): t0 = RN(x r) is within 2^-22 of x/s
// (relative), the residual x - t0 s is formed exactly by the fma up to one rounding, and
// t = RN(t0 + (x - t0 s) r) is RN of a value within 2^-44 (relative) of x/s.  The quotient
// of two fp16 values is never a midpoint of the fp32 grid (that would need 25 significant
// bits in x) and never within 2^-36 (relative) of one (x - m s is a nonzero multiple of
// m's grid times s's), so t is the correctly rounded quotient RN(x / s) exactly.
__device__ __forceinline__ float quot_rn(float x, float s, float r) {
  const float t0 = x * r;
  return __builtin_fmaf(__builtin_fmaf(-t0, s, x), r, t0);
}

// quot_rn for an fp16 x taken as it is: t0 = RN(x r + 0) equals RN(x r) for x != 0 (and is
// +0 for x = 0, where the result is 0 either way), so the result is RN(x / s) as above; every
// use of x is an fma operand, which gfx950 reads from the fp16 half-register directly.
__device__ __forceinline__ float quot_rn_h(_Float16 xh, float s, float r) {
  const float x = (float)xh;
  const float t0 = __builtin_fmaf(x, r, 0.0f);
  return __builtin_fmaf(__builtin_fmaf(-t0, s, x), r, t0);
}

// Code of an fp16 value x (as float) against an fp16 scale s, given r = 1/s
// (fp32, correctly rounded; r = 0 when s == 0).  Equals
// clamp(rint(fp32(x) / s), -qmax, qmax) for qmax <= 127 without the division:
//   * x and s are fp16, so x/s is either exactly a half-integer n + 1/2 or at
//     least 2^-13 away from every half-integer (the difference x - (n+1/2) s is
//     a nonzero multiple of the finer of the two fp16 grids);
//   * t = x * r is within |x/s| 2^-23 (< 2^-16 while |x/s| <= 128) of x/s, and
//     the IEEE quotient is within half an fp32 ulp of it, so away from a tie both
//     round to the same integer;
//   * an exact tie shows as |t - floor(t) - 1/2| < 2^-14 and is rounded from the
//     exact half, i.e. to even, as rint does for the tied fp32 quotient.
// Past |x/s| = 128 the result is clamped whatever the rounding.
__device__ __forceinline__ float int_code_f16(float x, float r, float qmax) {
  const float t = x * r;
  const float tf = floorf(t);
  const bool tie = fabsf((t - tf) - 0.5f) < 0x1p-14f;
  const float q = rintf(tie ? tf + 0.5f : t);
  return fminf(fmaxf(q, -qmax), qmax);
}

// 6-bit E2M3 field of an INT4 code held as a float: sign<<5 | |q| (q = 0 -> 0).
__device__ __forceinline__ uint32_t e2m3_field(float q) {
  const uint32_t a = (uint32_t)fabsf(q);
  return q < 0.0f ? (a | 32u) : a;
}

// fp32 (finite, >= 0) -> E4M3FN byte, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float a) {
  if (!(a < 448.0f)) return 0x7Eu;
  if (a < 0.015625f) {                        // below the smallest normal 2^-6: spacing 2^-9
    return (uint32_t)rintf(a * 512.0f);       // 0..8 (8 == smallest normal, code 0x08)
  }
  int e;
  (void)frexpf(a, &e);                        // a = f * 2^e, f in [0.5, 1)
  e -= 1;                                     // a in [2^e, 2^(e+1)), e in [-6, 8]
  float m = rintf(ldexpf(a, 3 - e));          // 8..16, exact scaling by a power of two
  uint32_t mi = (uint32_t)m;
  uint32_t code;
  if (mi == 16u) code = (uint32_t)(e + 1 + 7) << 3;
  else code = ((uint32_t)(e + 7) << 3) | (mi - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -v : v;
}

// E4M3 scale of an FP4 group.
__device__ __forceinline__ float fp4_scale(float amax, uint32_t* byte) {
  uint32_t b = e4m3_encode_pos(amax / 6.0f);
  *byte = b;
  return e4m3_decode(b);
}

// E2M1 nibble of v against scale s: sign<<3 | magnitude index; ties to the
// even mantissa (0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4).
__device__ __forceinline__ uint32_t fp4_code(float v, float s) {
  if (s == 0.0f) return 0u;
  float t = v / s;
  float a = fabsf(t);
  uint32_t idx = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                 (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                 (uint32_t)(a > 5.0f);
  return (t < 0.0f && idx != 0u) ? (idx | 8u) : idx;
}

// E2M1 nibble of the quotient t = RN(v / s) (same rule as fp4_code).
__device__ __forceinline__ uint32_t fp4_code_q(float t) {
  float a = fabsf(t);
  uint32_t idx = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                 (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                 (uint32_t)(a > 5.0f);
  return (t < 0.0f && idx != 0u) ? (idx | 8u) : idx;
}

// MXFP4 shared exponent of a group (OCP Microscaling Formats v1.0): e = floor(log2 amax) - 2
// (2: the exponent of E2M1's largest value 6 = 1.5 * 2^2), clamped to [-127, 127]; -127 for
// amax = 0.  v_frexp_exp gives amax = m 2^x with m in [0.5, 1), subnormals included, so
// floor(log2 amax) = x - 1.  The E8M0 byte is e + 127; codes are fp4_code_q(v * 2^-e) (exact).
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return -127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Eight E2M1 codes from the hardware convert with -0 made +0: v_cvt_scalef32_pk_fp4_f32 rounds
// to the nearest E2M1 value, ties to the even mantissa, saturating at 6 (the quantizers' rule)
// but keeps the sign of a negative value that rounds to zero; clear the sign bit of every
// nibble whose magnitude is 0.
__device__ __forceinline__ uint32_t fp4_plus_zero(uint32_t w) {
  const uint32_t mag = w & 0x77777777u;
  const uint32_t nz = (mag | (mag >> 1) | (mag >> 2)) & 0x11111111u;
  return mag | (w & (nz << 3));
}

// Eight values (already divided by their scale, or to be divided by the power of two s) as
// E2M1 codes, one word, code j in bits 4j..4j+3.
__device__ __forceinline__ uint32_t fp4_codes8(const float* t, float s) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[0], t[1], s, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[2], t[3], s, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[4], t[5], s, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[6], t[7], s, 3);
  return fp4_plus_zero(w);
}

// Pack 8 4-bit codes (low nibble first) into one 32-bit word.
__device__ __forceinline__ uint32_t pack8(const int* q) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) w |= ((uint32_t)q[i] & 0xFu) << (4 * i);
  return w;
}

// 8 INT4 codes as 6-bit E2M3 fields (sign<<5 | |q|: the E2M3 subnormal of q/8),
// code i at bits [6i, 6i+6) of a 48-bit value.
__device__ __forceinline__ uint64_t pack6x8(const int* q) {
  uint64_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t f = (q[i] < 0 ? 32u : 0u) | (uint32_t)(q[i] < 0 ? -q[i] : q[i]);
    w |= (uint64_t)f << (6 * i);
  }
  return w;
}

__device__ __forceinline__ uint32_t pack4_i8(const int* q) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) w |= ((uint32_t)q[i] & 0xFFu) << (8 * i);
  return w;
}

}  // namespace svdq
