// Shared host/device helpers of libfq (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq.h"

namespace fq {

// ---------------------------------------------------------------- errors --
// Thread-local message for the last non-OK status (fq_last_error()).
void set_error(const char *fmt, ...);
fq_status hip_status(hipError_t e, const char *what);

#define FQ_CHECK_ARG(cond, ...)                          \
  do {                                                   \
    if (!(cond)) {                                       \
      ::fq::set_error(__VA_ARGS__);                      \
      return FQ_ERR_INVALID_ARGUMENT;                    \
    }                                                    \
  } while (0)

#define FQ_CHECK_SUPPORTED(cond, ...)                    \
  do {                                                   \
    if (!(cond)) {                                       \
      ::fq::set_error(__VA_ARGS__);                      \
      return FQ_ERR_UNSUPPORTED;                         \
    }                                                    \
  } while (0)

// After a batch of launches: turn a launch failure into FQ_ERR_HIP.
#define FQ_CHECK_LAUNCH(what)                                        \
  do {                                                               \
    hipError_t e_ = hipGetLastError();                               \
    if (e_ != hipSuccess) return ::fq::hip_status(e_, what);         \
  } while (0)

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ----------------------------------------------------------------- bf16 --
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
// fp32 -> bf16, round to nearest even, two at a time on the hardware
// converter (v_cvt_pk_bf16_f32: the same bits as adding 0x7FFF + lsb to the
// fp32 encoding and truncating, for every non-NaN input).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16(f, 0.0f) & 0xFFFFu; }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 in 16 bytes
struct alignas(16) bf16x8_t {
  uint32_t w[4];
};

__device__ __forceinline__ void unpack8(const bf16x8_t &v, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = lo_bf16(v.w[i]);
    f[2 * i + 1] = hi_bf16(v.w[i]);
  }
}
__device__ __forceinline__ bf16x8_t pack8(const float *f) {
  bf16x8_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
  return v;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Division of 32-bit unsigned numerators by a runtime divisor d >= 1 with a
// multiply-high and a shift (round-up method, Hacker's Delight 10-9):
// l = ceil(log2 d), M = floor(2^32 (2^l - d) / d) + 1, q = (mulhi(x, M) + x) >> l.
struct FastDiv {
  uint32_t d, m, l;
  FastDiv() : d(1), m(1), l(0) {}
  explicit FastDiv(uint32_t div) : d(div) {
    l = 0;
    while ((1ull << l) < div) ++l;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t x) const {
    uint64_t t = (uint64_t)__umulhi(x, m) + x;
    return (uint32_t)(t >> l);
  }
};

}  // namespace fq
