// Real-quantized export of a weight stack on gfx950: the quantizer parameters
// in their stored form, and the decode of stored codes back to bf16.
//
// What it is: the QAT + ZeRO-3 page's convert / save_format=real keeps each
// quantized linear's codes with its weight scale; the mcore_qad article
// (section 三) stores each format in its deployment layout. The codes come
// from the fake-quant pass (k_quantize_stacked); this file turns the learnable
// parameters into their stored bytes (NVFP4 block scale -> E4M3 byte, int4 zero
// point -> byte) and decodes codes + stored scales with the FQ pass's own
// arithmetic (v = value(code) * s, one fp32 multiply, bf16 RNE), so decoding
// an export reproduces the fake-quant values bit for bit.
//
// All passes stream: 16 elements per thread, one work item per thread.
#include "internal.hpp"

namespace fq {

namespace {

constexpr int kThreads = 256;

inline int grid_for(long work_items) {
  long b = (work_items + kThreads - 1) / kThreads;
  if (b < 1) b = 1;
  if (b > (1 << 22)) b = 1 << 22;
  return (int)b;
}

// E4M3 byte of clamp(theta, 0, 448): the rounding the forward applies to the
// block parameter, on the converter (4 per thread when the count allows).
__global__ __launch_bounds__(kThreads) void k_export_theta(const float *__restrict__ theta,
                                                           uint32_t n, uint8_t *__restrict__ out) {
  const uint32_t n4 = n / 4;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
    const float4 t = reinterpret_cast<const float4 *>(theta)[i];
    float v0, v1;
    uint32_t lo = e4m3_pair(fminf(fmaxf(t.x, 0.0f), kE4M3Max), fminf(fmaxf(t.y, 0.0f), kE4M3Max),
                            v0, v1);
    uint32_t hi = e4m3_pair(fminf(fmaxf(t.z, 0.0f), kE4M3Max), fminf(fmaxf(t.w, 0.0f), kE4M3Max),
                            v0, v1);
    reinterpret_cast<uint32_t *>(out)[i] = lo | (hi << 16);
  }
  // the last n % 4 values (one thread each)
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n - 4 * n4) {
    float v0, v1;
    const float th = fminf(fmaxf(theta[4 * n4 + t], 0.0f), kE4M3Max);
    out[4 * n4 + t] = (uint8_t)(e4m3_pair(th, 0.0f, v0, v1) & 0xFFu);
  }
}

// zero-point byte clamp(rne(zp), 0, 15)
__global__ __launch_bounds__(kThreads) void k_export_zp(const float *__restrict__ zp, uint32_t n,
                                                        uint8_t *__restrict__ out) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    out[i] = (uint8_t)fminf(fmaxf(rintf(zp[i]), 0.0f), 15.0f);
}

// 16 decoded values of one chunk, from its codes and its scale.
template <int FMT>
__device__ __forceinline__ void decode16(const uint32_t *cw, float s, float zp, float *v) {
  if (FMT == FQ_FMT_NVFP4) {
    // 8 bytes of E2M1 nibbles, even element low; the converter gives exact values
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t c = cw[w];
      f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
      f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
      f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
      f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
      float *o = v + 8 * w;
      o[0] = p0.x * s; o[1] = p0.y * s; o[2] = p1.x * s; o[3] = p1.y * s;
      o[4] = p2.x * s; o[5] = p2.y * s; o[6] = p3.x * s; o[7] = p3.y * s;
    }
  } else if (FMT == FQ_FMT_FP8_E4M3) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[w], false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[w], true);
      v[4 * w + 0] = lo.x * s;
      v[4 * w + 1] = lo.y * s;
      v[4 * w + 2] = hi.x * s;
      v[4 * w + 3] = hi.y * s;
    }
  } else if (FMT == FQ_FMT_INT8) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = (int)(int8_t)((cw[j >> 2] >> (8 * (j & 3))) & 0xFFu);
      v[j] = (float)c * s;
    }
  } else {  // int4: value = code - zero point (+0.0 for a zero value)
    const int z = (int)zp;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = (int)((cw[j >> 3] >> (4 * (j & 7))) & 0xFu);
      v[j] = (float)(c - z) * s;
    }
  }
}

// out[chunk c] = decode of 16 elements. 4-bit formats: 8 code bytes per chunk;
// 1-byte formats: 16. Scale index = c / chunks_per_group; expert = c /
// chunks_per_expert (NVFP4 tensor scale).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequantize(
    const uint8_t *__restrict__ codes, uint32_t nchunk, FastDiv chunks_per_group,
    FastDiv chunks_per_expert, const float *__restrict__ scale,
    const uint8_t *__restrict__ scale_bytes, const uint8_t *__restrict__ zp_bytes,
    const float *__restrict__ gscale, bf16x8_t *__restrict__ out) {
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += gridDim.x * blockDim.x) {
    uint32_t cw[4];
    if (FMT == FQ_FMT_NVFP4 || FMT == FQ_FMT_INT4) {
      const uint2 b = reinterpret_cast<const uint2 *>(codes)[c];
      cw[0] = b.x;
      cw[1] = b.y;
    } else {
      const uint2 b0 = reinterpret_cast<const uint2 *>(codes)[2 * c];
      const uint2 b1 = reinterpret_cast<const uint2 *>(codes)[2 * c + 1];
      cw[0] = b0.x;
      cw[1] = b0.y;
      cw[2] = b1.x;
      cw[3] = b1.y;
    }
    float s, zp = 0.0f;
    if (FMT == FQ_FMT_NVFP4) {
      // s_b = fp32(E4M3 value of the block byte * g), as the forward forms it
      const f32x2_t th = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)scale_bytes[c], false);
      s = th.x * gscale[chunks_per_expert.div(c)];
    } else {
      const uint32_t g = chunks_per_group.div(c);
      s = scale[g];
      if (FMT == FQ_FMT_INT4) zp = (float)zp_bytes[g];
    }
    float v[16];
    decode16<FMT>(cw, s, zp, v);
    out[2 * (size_t)c] = pack8(v);
    out[2 * (size_t)c + 1] = pack8(v + 8);
  }
}

}  // namespace

void launch_export_theta(const float *theta, size_t n, uint8_t *out, hipStream_t st) {
  if (!n) return;
  const long threads = (long)(n / 4) > (long)(n % 4) ? (long)(n / 4) : (long)(n % 4);
  hipLaunchKernelGGL(k_export_theta, dim3(grid_for(threads)), dim3(kThreads), 0, st, theta,
                     (uint32_t)n, out);
}

void launch_export_zp(const float *zp, size_t n, uint8_t *out, hipStream_t st) {
  if (!n) return;
  hipLaunchKernelGGL(k_export_zp, dim3(grid_for((long)n)), dim3(kThreads), 0, st, zp,
                     (uint32_t)n, out);
}

void launch_dequantize(const uint8_t *codes, fq_shape s, int fmt, int group, const float *scale,
                       const uint8_t *scale_bytes, const uint8_t *zp_bytes, const float *gscale,
                       uint16_t *out, hipStream_t st) {
  const uint32_t nchunk = (uint32_t)((size_t)s.E * s.N * s.K / 16);
  if (!nchunk) return;
  const FastDiv cpg((uint32_t)(group / 16));
  const FastDiv cpe((uint32_t)((size_t)s.N * s.K / 16));
  auto o = reinterpret_cast<bf16x8_t *>(out);
  const dim3 grid(grid_for(nchunk)), block(kThreads);
#define FQ_DQ(F)                                                                                  \
  hipLaunchKernelGGL(k_dequantize<F>, grid, block, 0, st, codes, nchunk, cpg, cpe, scale,         \
                     scale_bytes, zp_bytes, gscale, o)
  switch (fmt) {
    case FQ_FMT_INT8: FQ_DQ(FQ_FMT_INT8); break;
    case FQ_FMT_INT4: FQ_DQ(FQ_FMT_INT4); break;
    case FQ_FMT_FP8_E4M3: FQ_DQ(FQ_FMT_FP8_E4M3); break;
    default: FQ_DQ(FQ_FMT_NVFP4); break;
  }
#undef FQ_DQ
}

}  // namespace fq
