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
// Grid rounding here is bit arithmetic (E4M3: round the fp32 mantissa to 3
// bits; E2M1: threshold comparisons at the midpoints), not a table search.
#pragma once

#include "common.hpp"

namespace fq {

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

// |a| <= 448 -> nearest E4M3 magnitude (ties to even mantissa); code 0..126.
__device__ __forceinline__ float e4m3_round_mag(float a, uint32_t &code) {
  if (a < 0x1p-6f) {
    // subnormal range: multiples of 2^-9; scaling by 512 is exact
    float q = rintf(a * 512.0f);
    code = (uint32_t)q;  // 0..8 (8 is the smallest normal, 2^-6, code 0x08)
    return q * 0x1p-9f;
  }
  uint32_t u = __float_as_uint(a);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & 0xFFF00000u;
  code = ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);
  return __uint_as_float(r);
}

__device__ __forceinline__ float e4m3_round_mag(float a) {
  uint32_t c;
  return e4m3_round_mag(a, c);
}

// |a| <= 6 -> E2M1 magnitude code 0..7 (ties to even code).
__device__ __forceinline__ uint32_t e2m1_code_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}
__device__ __forceinline__ float e2m1_value_mag(uint32_t c) {
  // 0, .5, 1, 1.5 for c < 4; then 2, 3, 4, 6
  float lo = (float)c * 0.5f;
  float hi = (c == 4u) ? 2.0f : (c == 5u) ? 3.0f : (c == 6u) ? 4.0f : 6.0f;
  return c < 4u ? lo : hi;
}

// One fake-quantized element: dequantized value, code, and STE terms.
struct FQElem {
  float v;      // dequantized fp32 value
  uint32_t code;
  bool m;       // STE mask [lo <= z <= hi]
  float dvds;   // dv/ds (nvfp4: dv/dtheta before the g*[0<=theta<=448] factor)
  float dvdzp;  // int4 only
};

// Quantizer parameters for one element (already resolved from its group).
struct ElemQ {
  float s;    // effective scale (nvfp4: s_b; 0 -> zero block)
  float r;    // 1/s
  float zp;   // int4: clamp(rne(zp), 0, 15); else 0
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
  float z = x * r;
  uint32_t c = e2m1_code_mag(fminf(fabsf(z), kE2M1Max));
  bool neg = (__float_as_uint(z) >> 31) != 0;
  float mag = e2m1_value_mag(c);
  float val = neg ? -mag : mag;
  o.m = (z >= -kE2M1Max) && (z <= kE2M1Max);
  o.v = val * s;
  o.code = c | (neg ? 0x8u : 0u);
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
