// Device codecs of the four fake-quant formats (gfx950).
//
// What is computed: quantize -> dequantize of a weight or activation with a
// scale, as the AngelSlim mcore_qad article describes for its formats nvfp4,
// fp8, w4a16 and w8a8 (sections 二.3 and 三), and the straight-through
// factors its scale-only backward needs (section 一: only scales train).
//
// Arithmetic is fp32 with round-to-nearest-even. The library is compiled
// with -ffp-contract=off so no multiply-add is fused: z = x * r and
// v = value * s are each one rounded multiply, exactly as specified.
//
// Grid rounding is bit arithmetic on the fp32 encoding (E4M3: round the
// mantissa to 3 bits, E2M1: to 1 bit; multiples of the smallest step below the
// normal range), not a table search. The hot paths round two values per
// instruction on gfx950's FP4 / FP8 converters instead (e2m1_pair, e4m3_pair);
// over every non-NaN fp32 input these give the same codes and values as the
// bit-arithmetic forms below (saturating, ties to even, sign kept,
// subnormals kept).
#pragma once

#include "common.hpp"

namespace fq {

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

// |a| <= 448 -> nearest E4M3 magnitude (ties to even mantissa); code 0..126.
// Normal range: the fp32 mantissa rounded to 3 bits; below 2^-6: multiples of
// 2^-9 (scaling by 512 is exact). Both are computed and one selected.
__device__ __forceinline__ float e4m3_round_mag(float a, uint32_t &code) {
  const float qs = rintf(a * 512.0f);  // subnormal: 0..8 (8 = 2^-6, code 0x08)
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
  const bool sub = a < 0x1p-6f;
  code = sub ? (uint32_t)qs : (((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u));
  return sub ? qs * 0x1p-9f : __uint_as_float(r);
}

__device__ __forceinline__ float e4m3_round_mag(float a) {
  const float qs = rintf(a * 512.0f) * 0x1p-9f;
  const uint32_t u = __float_as_uint(a);
  const float qn = __uint_as_float((u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u);
  return a < 0x1p-6f ? qs : qn;
}

// |a| <= 6 -> nearest E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the
// even code: multiples of 0.5 below 1, otherwise the fp32 mantissa rounded to
// one bit (RNE on bit 22).
__device__ __forceinline__ float e2m1_round_mag(float a) {
  const float lo = rintf(a * 2.0f) * 0.5f;
  const uint32_t u = __float_as_uint(a);
  const float hi = __uint_as_float((u + 0x1FFFFFu + ((u >> 22) & 1u)) & 0xFFC00000u);
  return a < 1.0f ? lo : hi;
}
// E2M1 magnitude -> 3-bit code: 2 * v below 1, else (exponent - 126) << 1 | mantissa bit
__device__ __forceinline__ uint32_t e2m1_code_of_mag(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t c_hi = (((u >> 23) - 126u) << 1) | ((u >> 22) & 1u);
  return v < 1.0f ? (uint32_t)(v * 2.0f) : c_hi;
}

// Two values z0, z1 rounded to E2M1 on the converter: values (sign of z kept,
// |z| > 6 saturates) and the packed codes, z0 in the low nibble.
// An unspecified register value, made by no instruction: the converters below
// write only the low byte / half-word of their destination and keep the rest,
// which is never read, so the kept bits need not be cleared first.
__device__ __forceinline__ uint32_t undef_u32() {
  uint32_t u;
  asm volatile("" : "=v"(u));
  return u;
}
__device__ __forceinline__ uint32_t e2m1_pair(float z0, float z1, float &v0, float &v1) {
  const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(undef_u32(), z0, z1, 1.0f, 0);
  const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  v0 = v.x;
  v1 = v.y;
  return c & 0xFFu;
}
// Two values already clamped to [-448, 448] rounded to E4M3: values and the
// packed codes, z0 in the low byte.
__device__ __forceinline__ uint32_t e4m3_pair(float z0, float z1, float &v0, float &v1) {
  const uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(z0, z1, undef_u32(), false);
  const f32x2_t v = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
  v0 = v.x;
  v1 = v.y;
  return c & 0xFFFFu;
}
__device__ __forceinline__ float clamp448(float z) { return fminf(fmaxf(z, -kE4M3Max), kE4M3Max); }

// One fake-quantized element: dequantized value, code, and STE terms.
struct FQElem {
  float v;      // dequantized fp32 value
  uint32_t code;
  bool m;       // STE mask [lo <= z <= hi]
  float dvds;   // dv/ds (nvfp4: dv/dtheta before the g*[0<=theta<=448] factor)
  float dvdzp;  // int4 only
};

// int8 symmetric
__device__ __forceinline__ FQElem fq_int8(float x, float s, float r) {
  FQElem o;
  float z = x * r;
  float q = rintf(fminf(fmaxf(z, -128.0f), 127.0f));
  int qi = (int)q;
  o.m = (z >= -128.0f) && (z <= 127.0f);
  o.v = (float)qi * s;  // int -> float gives +0.0 for a zero code
  o.code = (uint32_t)(qi & 0xFF);
  o.dvds = (float)qi - (o.m ? z : 0.0f);
  o.dvdzp = 0.0f;
  return o;
}

// int4 asymmetric, zpi = clamp(rne(zp), 0, 15)
__device__ __forceinline__ FQElem fq_int4(float x, float s, float r, float zpi) {
  FQElem o;
  float z = x * r;
  float lo = -zpi, hi = 15.0f - zpi;
  float q = rintf(fminf(fmaxf(z, lo), hi));
  int qi = (int)q;
  o.m = (z >= lo) && (z <= hi);
  o.v = (float)qi * s;
  o.code = (uint32_t)(qi + (int)zpi);
  o.dvds = (float)qi - (o.m ? z : 0.0f);
  o.dvdzp = o.m ? 0.0f : -s;
  return o;
}

// FP8 E4M3, saturating, sign of z kept
__device__ __forceinline__ FQElem fq_fp8(float x, float s, float r) {
  FQElem o;
  float z = x * r;
  uint32_t c;
  float mag = e4m3_round_mag(fminf(fabsf(z), kE4M3Max), c);
  bool neg = (__float_as_uint(z) >> 31) != 0;
  float val = neg ? -mag : mag;
  o.m = (z >= -kE4M3Max) && (z <= kE4M3Max);
  o.v = val * s;
  o.code = c | (neg ? 0x80u : 0u);
  o.dvds = val - (o.m ? z : 0.0f);
  o.dvdzp = 0.0f;
  return o;
}

// NVFP4 element with block scale s (s == 0: zero block), sign of z kept
__device__ __forceinline__ FQElem fq_e2m1(float x, float s, float r) {
  FQElem o;
  if (s == 0.0f) {
    o.v = 0.0f;
    o.code = 0;
    o.m = false;
    o.dvds = 0.0f;
    o.dvdzp = 0.0f;
    return o;
  }
  const float z = x * r;
  const float az = fabsf(z);
  const float mag = e2m1_round_mag(fminf(az, kE2M1Max));
  const bool neg = (__float_as_uint(z) >> 31) != 0;
  const float val = neg ? -mag : mag;
  o.m = az <= kE2M1Max;
  o.v = val * s;
  o.code = e2m1_code_of_mag(mag) | (neg ? 0x8u : 0u);
  o.dvds = val - (o.m ? z : 0.0f);
  o.dvdzp = 0.0f;
  return o;
}

// NVFP4 block scale from the learnable parameter theta and tensor scale g.
__device__ __forceinline__ float nvfp4_block_scale(float theta, float g) {
  float th = fminf(fmaxf(theta, 0.0f), kE4M3Max);
  return e4m3_round_mag(th) * g;
}
// dv/dtheta = g * [0 <= theta <= 448] * (value - m z)
__device__ __forceinline__ float nvfp4_theta_factor(float theta, float g) {
  return (theta >= 0.0f && theta <= kE4M3Max) ? g : 0.0f;
}

// Dynamic activation block scale from the block amax and frozen g_a:
// theta = E4M3(clamp(amax * (1/(6 g)), 0, 448)), s = theta * g.
__device__ __forceinline__ float nvfp4_dynamic_scale(float amax, float g) {
  float d = 6.0f * g;
  float rd = 1.0f / d;
  float t = fminf(amax * rd, kE4M3Max);
  return e4m3_round_mag(t) * g;
}

__device__ __forceinline__ float safe_recip(float s) { return s != 0.0f ? 1.0f / s : 0.0f; }

// Straight-through factor dv/ds = value(c) - m*z of one element, without the
// dequantized value or the code (what the dScale reduction needs). For NVFP4
// the caller applies g*[0 <= theta <= 448] per block; a zero block scale comes
// in as r = 0, which gives z = 0, value 0 and factor 0. int4 also returns
// dv/dzp = -s*(1-m).
template <int FMT>
__device__ __forceinline__ float ste_factor(float x, float s, float r, float zpi, float &dvdzp) {
  const float z = x * r;
  if (FMT == FQ_FMT_NVFP4 || FMT == FQ_FMT_FP8_E4M3) {
    const float mx = FMT == FQ_FMT_NVFP4 ? kE2M1Max : kE4M3Max;
    const float az = fabsf(z);
    const float ac = fminf(az, mx);
    const float mag = FMT == FQ_FMT_NVFP4 ? e2m1_round_mag(ac) : e4m3_round_mag(ac);
    const float val = __builtin_copysignf(mag, z);
    dvdzp = 0.0f;
    return val - (az <= mx ? z : 0.0f);
  }
  const float lo = FMT == FQ_FMT_INT4 ? -zpi : -128.0f;
  const float hi = FMT == FQ_FMT_INT4 ? 15.0f - zpi : 127.0f;
  const float zc = fminf(fmaxf(z, lo), hi);
  const bool m = zc == z;
  dvdzp = m ? 0.0f : -s;
  return rintf(zc) - (m ? z : 0.0f);
}

// ste_factor of two elements sharing a scale (FP formats round on the
// converter; the integer formats use the per-element form).
template <int FMT>
__device__ __forceinline__ void ste_factor2(float x0, float x1, float s, float r, float zpi,
                                            float &f0, float &f1, float &dz0, float &dz1) {
  if (FMT == FQ_FMT_NVFP4 || FMT == FQ_FMT_FP8_E4M3) {
    const float z0 = x0 * r, z1 = x1 * r;
    float v0, v1;
    if (FMT == FQ_FMT_NVFP4) {
      e2m1_pair(z0, z1, v0, v1);
      f0 = v0 - (fabsf(z0) <= kE2M1Max ? z0 : 0.0f);
      f1 = v1 - (fabsf(z1) <= kE2M1Max ? z1 : 0.0f);
    } else {
      e4m3_pair(clamp448(z0), clamp448(z1), v0, v1);
      f0 = v0 - (fabsf(z0) <= kE4M3Max ? z0 : 0.0f);
      f1 = v1 - (fabsf(z1) <= kE4M3Max ? z1 : 0.0f);
    }
    dz0 = dz1 = 0.0f;
  } else {
    f0 = ste_factor<FMT>(x0, s, r, zpi, dz0);
    f1 = ste_factor<FMT>(x1, s, r, zpi, dz1);
  }
}

// Generic per-element dispatch for weights (fmt known at runtime).
__device__ __forceinline__ FQElem fq_weight_elem(int fmt, float x, float s, float r, float zpi) {
  switch (fmt) {
    case FQ_FMT_INT8: return fq_int8(x, s, r);
    case FQ_FMT_INT4: return fq_int4(x, s, r, zpi);
    case FQ_FMT_FP8_E4M3: return fq_fp8(x, s, r);
    default: return fq_e2m1(x, s, r);
  }
}

}  // namespace fq
