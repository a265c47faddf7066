// HBM-bound passes of libfq on gfx950: the stacked weight fake-quant, the
// observers, activation fake-quant (plain, gathered, after SwiGLU), SwiGLU
// backward, combine / unpermute (the last two optionally with the gradient of
// a learnable activation scale, summed in a fixed order).
//
// Every pass moves 16-byte vectors per lane (8 bf16), so a wavefront touches
// 1 KiB of contiguous memory per load; indexes are 32-bit with precomputed
// fast division. Launches use enough blocks to cover all 256 CUs several
// times and grid-stride beyond that.
#include "internal.hpp"

namespace fq {

namespace {

constexpr int kThreads = 256;

// Streaming kernels launch one work item per thread (a grid-stride loop only
// beyond 2^22 blocks): launched in address order, neighbouring waves stream
// neighbouring memory, which HBM serves measurably faster than a capped
// persistent grid striding over the whole array.
inline int grid_for(long work_items, int per_block = kThreads, int max_blocks = 1 << 22) {
  long b = (work_items + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > max_blocks) b = max_blocks;
  return (int)b;
}

// ------------------------------------------------------------- fill --------
__global__ void k_fill_u32(uint32_t *p, uint32_t v, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_repeat_rows(const float *__restrict__ v, uint32_t total, FastDiv n,
                              float *__restrict__ out) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x)
    out[i] = v[n.div(i)];
}

// ------------------------------------------- stacked weight fake-quant -----
// One thread-iteration handles one 8-element vector of one row. Requires
// group % 8 == 0 so a vector never straddles a scale group.
template <int FMT>
__device__ __forceinline__ void quantize_vec(const bf16x8_t v, float s, float zpi, uint32_t i,
                                             bf16x8_t *__restrict__ out,
                                             uint8_t *__restrict__ codes) {
  const float r = safe_recip(s);
  float x[8], y[8];
  unpack8(v, x);
  if (FMT == FQ_FMT_NVFP4 || FMT == FQ_FMT_FP8_E4M3) {
    uint32_t cw[2] = {0u, 0u};
    if (FMT == FQ_FMT_NVFP4 && s == 0.0f) {  // zero block: +0.0, code 0
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.0f;
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float v0, v1;
        if (FMT == FQ_FMT_NVFP4) {
          cw[0] |= e2m1_pair(x[2 * p] * r, x[2 * p + 1] * r, v0, v1) << (8 * p);
        } else {
          cw[p >> 1] |= e4m3_pair(clamp448(x[2 * p] * r), clamp448(x[2 * p + 1] * r), v0, v1)
                        << (16 * (p & 1));
        }
        y[2 * p] = v0 * s;
        y[2 * p + 1] = v1 * s;
      }
    }
    if (out) out[i] = pack8(y);
    if (codes) {
      if (FMT == FQ_FMT_NVFP4) reinterpret_cast<uint32_t *>(codes)[i] = cw[0];
      else reinterpret_cast<uint2 *>(codes)[i] = make_uint2(cw[0], cw[1]);
    }
    return;
  }
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    FQElem e = fq_weight_elem(FMT, x[j], s, r, zpi);
    y[j] = e.v;
    c[j] = e.code;
  }
  if (out) out[i] = pack8(y);
  if (codes) {
    if (FMT == FQ_FMT_INT8) {
      uint2 b;
      b.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      b.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      reinterpret_cast<uint2 *>(codes)[i] = b;
    } else {
      uint32_t b = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) b |= (c[j] & 0xFu) << (4 * j);
      reinterpret_cast<uint32_t *>(codes)[i] = b;
    }
  }
}

// kQU vectors a grid stride apart per thread and iteration, loads issued
// before any arithmetic (1 measured best, with one vector per thread).
constexpr int kQU = 1;
constexpr int kQGridCap = 1 << 22;
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_quantize_stacked(
    const bf16x8_t *__restrict__ w, uint32_t nvec, FastDiv vec_per_expert,
    FastDiv vec_per_group, const float *__restrict__ scale,
    const float *__restrict__ zero_point, const float *__restrict__ gscale,
    bf16x8_t *__restrict__ out, uint8_t *__restrict__ codes) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i0 = blockIdx.x * blockDim.x + threadIdx.x; i0 < nvec; i0 += kQU * stride) {
    bf16x8_t v[kQU];
    float sc[kQU], zp[kQU], g[kQU];
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
      const uint32_t i = i0 + u * stride;
      if (i < nvec) {
        v[u] = w[i];
        // a group never straddles a row, so the group index is i / (group / 8)
        const uint32_t gidx = vec_per_group.div(i);
        sc[u] = scale[gidx];
        zp[u] = (FMT == FQ_FMT_INT4) ? zero_point[gidx] : 0.0f;
        g[u] = (FMT == FQ_FMT_NVFP4) ? gscale[vec_per_expert.div(i)] : 1.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
      const uint32_t i = i0 + u * stride;
      if (i < nvec) {
        float s = sc[u], zpi = 0.0f;
        if (FMT == FQ_FMT_INT4) zpi = fminf(fmaxf(rintf(zp[u]), 0.0f), 15.0f);
        if (FMT == FQ_FMT_NVFP4) s = nvfp4_block_scale(s, g[u]);
        quantize_vec<FMT>(v[u], s, zpi, i, out, codes);
      }
    }
  }
}

// ------------------------------------------------------------ observer -----
// Groups that span 2..64 vectors are reduced across adjacent lanes; one
// vector per lane, vectors of a group on consecutive lanes of one wave.
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_observer_lanes(const bf16x8_t *__restrict__ w,
                                                             uint32_t nvec, int lanes_per_group,
                                                             float *__restrict__ scale,
                                                             float *__restrict__ zero_point) {
  const uint32_t stride = gridDim.x * blockDim.x;
  // uniform trip count so every lane takes part in the shuffles
  for (uint32_t base = blockIdx.x * blockDim.x; base < nvec; base += stride) {
    uint32_t i = base + threadIdx.x;
    bool ok = i < nvec;
    float x[8];
    bf16x8_t v = ok ? w[i] : bf16x8_t{{0, 0, 0, 0}};
    unpack8(v, x);
    float amax = 0.0f, mn = 0.0f, mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      amax = fmaxf(amax, fabsf(x[j]));
      mn = fminf(mn, x[j]);
      mx = fmaxf(mx, x[j]);
    }
    for (int o = 1; o < lanes_per_group; o <<= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      mn = fminf(mn, __shfl_xor(mn, o, 64));
      mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    }
    if (ok && (threadIdx.x & (lanes_per_group - 1)) == 0) {
      uint32_t gi = i / (uint32_t)lanes_per_group;
      if (FMT == FQ_FMT_INT8 || FMT == FQ_FMT_FP8_E4M3) {
        float s = amax / (FMT == FQ_FMT_INT8 ? 127.0f : kE4M3Max);
        scale[gi] = s == 0.0f ? 1.0f : s;
      } else if (FMT == FQ_FMT_INT4) {
        float s = (mx - mn) / 15.0f;  // mn <= 0 <= mx
        s = s == 0.0f ? 1.0f : s;
        float r = 1.0f / s;
        scale[gi] = s;
        zero_point[gi] = fminf(fmaxf(rintf(-mn * r), 0.0f), 15.0f);
      } else {  // nvfp4: block amax now, theta after the expert amax is known
        scale[gi] = amax;
      }
    }
  }
}

// Groups longer than 64 vectors (per-channel scales): one block per group.
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_observer_block(const bf16x8_t *__restrict__ w,
                                                             int vec_per_group,
                                                             float *__restrict__ scale,
                                                             float *__restrict__ zero_point) {
  const bf16x8_t *p = w + (size_t)blockIdx.x * vec_per_group;
  float amax = 0.0f, mn = 0.0f, mx = 0.0f;
  for (int i = threadIdx.x; i < vec_per_group; i += blockDim.x) {
    float x[8];
    unpack8(p[i], x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      amax = fmaxf(amax, fabsf(x[j]));
      mn = fminf(mn, x[j]);
      mx = fmaxf(mx, x[j]);
    }
  }
  __shared__ float red[3][kThreads / 64];
  amax = warp_max(amax);
  mx = warp_max(mx);
  mn = -warp_max(-mn);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = amax;
    red[1][threadIdx.x >> 6] = mn;
    red[2][threadIdx.x >> 6] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k) {
      amax = fmaxf(amax, red[0][k]);
      mn = fminf(mn, red[1][k]);
      mx = fmaxf(mx, red[2][k]);
    }
    if (FMT == FQ_FMT_INT8 || FMT == FQ_FMT_FP8_E4M3) {
      float s = amax / (FMT == FQ_FMT_INT8 ? 127.0f : kE4M3Max);
      scale[blockIdx.x] = s == 0.0f ? 1.0f : s;
    } else {  // int4
      float s = (mx - mn) / 15.0f;
      s = s == 0.0f ? 1.0f : s;
      float r = 1.0f / s;
      scale[blockIdx.x] = s;
      zero_point[blockIdx.x] = fminf(fmaxf(rintf(-mn * r), 0.0f), 15.0f);
    }
  }
}

// Per-expert amax from the block amaxes (one block per expert, no atomics):
// out_bits[e] = bits of max over blocks [e*nb, (e+1)*nb).
__global__ __launch_bounds__(kThreads) void k_expert_amax(const float *__restrict__ block_amax,
                                                          uint32_t nb, uint32_t *__restrict__ out_bits) {
  const float *p = block_amax + (size_t)blockIdx.x * nb;
  float m = 0.0f;
  for (uint32_t i = threadIdx.x; i < nb; i += blockDim.x) m = fmaxf(m, p[i]);
  m = warp_max(m);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k) m = fmaxf(m, red[k]);
    out_bits[blockIdx.x] = __float_as_uint(m);
  }
}

// theta_b = E4M3(clamp(amax_b * (1/(6 g)), 0, 448)), g = amax_e / 2688 (1 if 0)
__global__ void k_nvfp4_theta(float *__restrict__ theta, uint32_t n, FastDiv blocks_per_expert,
                              const uint32_t *__restrict__ expert_amax) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    float ae = __uint_as_float(expert_amax[blocks_per_expert.div(i)]);
    float g = ae / (kE2M1Max * kE4M3Max);
    g = g == 0.0f ? 1.0f : g;
    float d = 6.0f * g;
    float rd = 1.0f / d;
    float t = fminf(theta[i] * rd, kE4M3Max);
    theta[i] = e4m3_round_mag(t);
  }
}

__global__ void k_nvfp4_global(uint32_t *__restrict__ g_bits, int E) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) {
    float g = __uint_as_float(g_bits[e]) / (kE2M1Max * kE4M3Max);
    reinterpret_cast<float *>(g_bits)[e] = g == 0.0f ? 1.0f : g;
  }
}

// per-tensor absmax into out_bits[0] (zeroed before)
__global__ __launch_bounds__(kThreads) void k_absmax_tensor(const bf16x8_t *__restrict__ x,
                                                            uint32_t nvec,
                                                            uint32_t *__restrict__ out_bits) {
  float amax = 0.0f;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += gridDim.x * blockDim.x) {
    float f[8];
    unpack8(x[i], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
  }
  amax = warp_max(amax);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k) amax = fmaxf(amax, red[k]);
    atomicMax(out_bits, __float_as_uint(amax));  // max is order independent
  }
}

__global__ void k_act_scale_finalize(uint32_t *bits, float div) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    float s = __uint_as_float(bits[0]) / div;
    reinterpret_cast<float *>(bits)[0] = s == 0.0f ? 1.0f : s;
  }
}

// ------------------------------------------------ activation fake-quant -----
// Per-tensor frozen activation quantizer, resolved once per thread.
struct ActQ {
  int fmt;
  float s;  // s_a (fp8 / int8) or g_a (nvfp4)
  float r;  // 1/s_a
};

__device__ __forceinline__ ActQ load_actq(int fmt, const float *scale) {
  ActQ q;
  q.fmt = fmt;
  q.s = (fmt == FQ_FMT_NONE) ? 1.0f : scale[0];
  q.r = (fmt == FQ_FMT_NONE) ? 1.0f : 1.0f / q.s;
  return q;
}

// 16 consecutive elements along K (one NVFP4 block): values in place, mask bits out.
__device__ __forceinline__ uint32_t act_fq16(const ActQ &q, float *x) {
  uint32_t mask = 0;
  if (q.fmt == FQ_FMT_NONE) return 0xFFFFu;
  if (q.fmt == FQ_FMT_NVFP4 || q.fmt == FQ_FMT_FP8_E4M3) {
    float s = q.s, r = q.r;
    const float mx = q.fmt == FQ_FMT_NVFP4 ? kE2M1Max : kE4M3Max;
    if (q.fmt == FQ_FMT_NVFP4) {
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(x[j]));
      s = nvfp4_dynamic_scale(amax, q.s);
      if (s == 0.0f) {  // zero block: +0.0, mask 0
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = 0.0f;
        return 0u;
      }
      r = 1.0f / s;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float z0 = x[2 * p] * r, z1 = x[2 * p + 1] * r;
      float v0, v1;
      if (q.fmt == FQ_FMT_NVFP4) e2m1_pair(z0, z1, v0, v1);
      else e4m3_pair(clamp448(z0), clamp448(z1), v0, v1);
      mask |= (uint32_t)(fabsf(z0) <= mx) << (2 * p);
      mask |= (uint32_t)(fabsf(z1) <= mx) << (2 * p + 1);
      x[2 * p] = v0 * s;
      x[2 * p + 1] = v1 * s;
    }
    return mask;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    FQElem e = fq_int8(x[j], q.s, q.r);
    x[j] = e.v;
    mask |= (uint32_t)e.m << j;
  }
  return mask;
}

// 8 consecutive elements along K, one half of a 16-element block; the other
// half is on lane ^ 1, which must run the same call (NVFP4 takes the block
// amax over both halves, so the result equals act_fq16 on the whole block).
// Values in place, 8 mask bits out.
__device__ __forceinline__ uint32_t act_fq8_pair(const ActQ &q, float *x) {
  uint32_t mask = 0;
  if (q.fmt == FQ_FMT_NONE) return 0xFFu;
  if (q.fmt == FQ_FMT_NVFP4 || q.fmt == FQ_FMT_FP8_E4M3) {
    float s = q.s, r = q.r;
    const float mx = q.fmt == FQ_FMT_NVFP4 ? kE2M1Max : kE4M3Max;
    if (q.fmt == FQ_FMT_NVFP4) {
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      s = nvfp4_dynamic_scale(amax, q.s);
      if (s == 0.0f) {  // zero block: +0.0, mask 0
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 0.0f;
        return 0u;
      }
      r = 1.0f / s;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float z0 = x[2 * p] * r, z1 = x[2 * p + 1] * r;
      float v0, v1;
      if (q.fmt == FQ_FMT_NVFP4) e2m1_pair(z0, z1, v0, v1);
      else e4m3_pair(clamp448(z0), clamp448(z1), v0, v1);
      mask |= (uint32_t)(fabsf(z0) <= mx) << (2 * p);
      mask |= (uint32_t)(fabsf(z1) <= mx) << (2 * p + 1);
      x[2 * p] = v0 * s;
      x[2 * p + 1] = v1 * s;
    }
    return mask;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    FQElem e = fq_int8(x[j], q.s, q.r);
    x[j] = e.v;
    mask |= (uint32_t)e.m << j;
  }
  return mask;
}

__device__ __forceinline__ void load16(const bf16x8_t *p, float *x) {
  bf16x8_t a = p[0], b = p[1];
  unpack8(a, x);
  unpack8(b, x + 8);
}
__device__ __forceinline__ void store16(bf16x8_t *p, const float *x) {
  p[0] = pack8(x);
  p[1] = pack8(x + 8);
}

// FP8 / INT8 activation fake-quant of 16 elements that also yields each
// element's straight-through factor dv/ds_a = value(c) - m*z (the factor of a
// learnable per-tensor scale, the same as a weight scale's). Values in place,
// factors to dvds, mask bits returned.
__device__ __forceinline__ uint32_t act_fq16_ds(const ActQ &q, float *x, float *dvds) {
  uint32_t mask = 0;
  if (q.fmt == FQ_FMT_FP8_E4M3) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float z0 = x[2 * p] * q.r, z1 = x[2 * p + 1] * q.r;
      float v0, v1;
      e4m3_pair(clamp448(z0), clamp448(z1), v0, v1);
      const bool m0 = fabsf(z0) <= kE4M3Max, m1 = fabsf(z1) <= kE4M3Max;
      mask |= ((uint32_t)m0 << (2 * p)) | ((uint32_t)m1 << (2 * p + 1));
      dvds[2 * p] = v0 - (m0 ? z0 : 0.0f);
      dvds[2 * p + 1] = v1 - (m1 ? z1 : 0.0f);
      x[2 * p] = v0 * q.s;
      x[2 * p + 1] = v1 * q.s;
    }
    return mask;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    FQElem e = fq_int8(x[j], q.s, q.r);
    x[j] = e.v;
    dvds[j] = e.dvds;
    mask |= (uint32_t)e.m << j;
  }
  return mask;
}

// Sum of v over the block, the same in every thread and bitwise reproducible:
// a butterfly inside each wave (both partners of a step add the same two
// values, so every lane ends with the same sum), then the waves in index order.
template <int NT>
__device__ __forceinline__ float block_sum_fixed(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __shared__ float red[NT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) s += red[k];
  return s;
}

// out[row] = sum of in[row, 0:n], one block per row, fixed order.
__global__ __launch_bounds__(kThreads) void k_sum_rows(const float *__restrict__ in, uint32_t n,
                                                       float *__restrict__ out) {
  const float *p = in + (size_t)blockIdx.x * n;
  float v = 0.0f;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) v += p[i];
  v = block_sum_fixed<kThreads>(v);
  if (threadIdx.x == 0) out[blockIdx.x] = v;
}

// out[0] = sum of the n block partials (one block, fixed order).
constexpr int kSumThreads = 1024;
__global__ __launch_bounds__(kSumThreads) void k_sum_partials(const float *__restrict__ part,
                                                              uint32_t n, float *__restrict__ out) {
  float v = 0.0f;
  for (uint32_t i = threadIdx.x; i < n; i += kSumThreads) v += part[i];
  v = block_sum_fixed<kSumThreads>(v);
  if (threadIdx.x == 0) out[0] = v;
}

// number of 16-element chunks to process: all of them, or only the first
// n_rows[0] rows (rows past the routed count are left untouched)
__device__ __forceinline__ uint32_t live_chunks(uint32_t max_chunks, const int32_t *n_rows,
                                                uint32_t chunks_per_row) {
  return n_rows ? min((uint32_t)n_rows[0] * chunks_per_row, max_chunks) : max_chunks;
}

// x [M, K] -> xq [M, K]. One 16-byte vector (8 elements) per lane, so each
// wave load and store covers 1 KiB; a 16-block spans the lane pair
// (2m, 2m + 1). The grid stride and the vector count are even, so both lanes
// of a pair run every iteration together.
__global__ __launch_bounds__(kThreads) void k_act_fq(const bf16x8_t *__restrict__ x, uint32_t max_vec,
                                                     const int32_t *__restrict__ n_rows, uint32_t vpr,
                                                     int afmt, const float *__restrict__ ascale,
                                                     bf16x8_t *__restrict__ xq) {
  ActQ q = load_actq(afmt, ascale);
  const uint32_t nvec = live_chunks(max_vec, n_rows, vpr);
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nvec; c += gridDim.x * blockDim.x) {
    float f[8];
    unpack8(x[c], f);
    act_fq8_pair(q, f);
    xq[c] = pack8(f);
  }
}

// dx[M, K] *= mask(FQ_a(x))   (in place)
__global__ __launch_bounds__(kThreads) void k_act_mask(bf16x8_t *__restrict__ dx,
                                                       const bf16x8_t *__restrict__ x,
                                                       uint32_t max_chunks,
                                                       const int32_t *__restrict__ n_rows,
                                                       uint32_t cpr, int afmt,
                                                       const float *__restrict__ ascale) {
  ActQ q = load_actq(afmt, ascale);
  const uint32_t nchunk = live_chunks(max_chunks, n_rows, cpr);
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += gridDim.x * blockDim.x) {
    float f[16], d[16];
    load16(x + 2 * (size_t)c, f);
    uint32_t m = act_fq16(q, f);
    load16(dx + 2 * (size_t)c, d);
#pragma unroll
    for (int j = 0; j < 16; ++j) d[j] = ((m >> j) & 1u) ? d[j] : 0.0f;
    store16(dx + 2 * (size_t)c, d);
  }
}

// xq[r] = FQ_a(x[perm[r] / topk]) for r < n_rows[0]
// Per token: x[t] is read and fake-quantized once, then stored to each of its
// routed rows xq[row_of[t, j]] (j ascending; -1 = not routed here). One
// 16-byte vector per lane, so every store instruction of a wave covers 1 KiB
// of one routed row (32-byte pieces per lane scatter ~9 % slower); a 16-block
// spans the lane pair (2m, 2m + 1). The grid stride and the vector count are
// even, so both lanes of a pair run every iteration together.
__global__ __launch_bounds__(kThreads) void k_gather_actfq(
    const bf16x8_t *__restrict__ x, const int32_t *__restrict__ row_of, int topk,
    FastDiv vec_per_row, uint32_t nvec, int afmt, const float *__restrict__ ascale,
    bf16x8_t *__restrict__ xq) {
  ActQ q = load_actq(afmt, ascale);
  const uint32_t vpr = vec_per_row.d;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nvec; c += gridDim.x * blockDim.x) {
    const uint32_t t = vec_per_row.div(c);
    const uint32_t cc = c - t * vpr;
    float f[8];
    unpack8(x[c], f);
    act_fq8_pair(q, f);
    const bf16x8_t v = pack8(f);
    for (int j = 0; j < topk; ++j) {
      const int r = row_of[t * topk + j];
      if (r >= 0) xq[(size_t)r * vpr + cc] = v;
    }
  }
}

// sigmoid(g) = 1 / (1 + exp(-g)) on the hardware exp and reciprocal (a few
// ulp; 0 and 1 at the extremes). The forward and the backward both call it,
// so the backward sees exactly the forward's A.
__device__ __forceinline__ float sigmoid_hw(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
// SwiGLU value of 16 elements in fp32, silu(g) = g * sigmoid(g), rounded to
// bf16 (the stored A); sig receives sigmoid(g).
__device__ __forceinline__ void swiglu16(const float *g, const float *u, float *a, float *sig) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sig[j] = sigmoid_hw(g[j]);
    a[j] = bf16_to_f32(f32_to_bf16((g[j] * sig[j]) * u[j]));
  }
}

// h [R, 2F] -> a [R, F] (optional), aq [R, F]. One 16-byte vector of each
// output per lane (1 KiB per wave store); a 16-block spans a lane pair, as in
// the gather.
__global__ __launch_bounds__(kThreads) void k_swiglu_actfq(
    const bf16x8_t *__restrict__ h, FastDiv vec_per_row, uint32_t max_vec,
    const int32_t *__restrict__ n_rows, int afmt, const float *__restrict__ ascale,
    bf16x8_t *__restrict__ a_out, bf16x8_t *__restrict__ aq_out) {
  ActQ q = load_actq(afmt, ascale);
  const uint32_t vpr = vec_per_row.d;  // F / 8
  const uint32_t nvec = min((uint32_t)n_rows[0] * vpr, max_vec);
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nvec; c += gridDim.x * blockDim.x) {
    const uint32_t r = vec_per_row.div(c);
    const uint32_t cc = c - r * vpr;
    const bf16x8_t *hr = h + (size_t)r * 2 * vpr;
    float g[8], u[8], a[8];
    unpack8(hr[cc], g);
    unpack8(hr[vpr + cc], u);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      a[j] = bf16_to_f32(f32_to_bf16((g[j] * sigmoid_hw(g[j])) * u[j]));
    if (a_out) a_out[c] = pack8(a);
    act_fq8_pair(q, a);
    aq_out[c] = pack8(a);
  }
}

// dh = SwiGLU'(h) applied to da = m_a * daq. DS: also the block's share of
// dS_a = sum daq * dv/ds_a(A) into ds_part[blockIdx.x] (A recomputed as in the
// forward, so its FQ factors are the forward's).
template <bool DS>
__global__ __launch_bounds__(kThreads) void k_swiglu_bwd(
    const bf16x8_t *__restrict__ daq, const bf16x8_t *__restrict__ h, FastDiv chunks_per_row,
    uint32_t max_chunks, const int32_t *__restrict__ n_rows, int afmt,
    const float *__restrict__ ascale, bf16x8_t *__restrict__ dh, float *__restrict__ ds_part) {
  ActQ q = load_actq(afmt, ascale);
  const uint32_t cpr = chunks_per_row.d;
  const uint32_t nchunk = min((uint32_t)n_rows[0] * cpr, max_chunks);
  float part = 0.0f;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += gridDim.x * blockDim.x) {
    uint32_t r = chunks_per_row.div(c);
    uint32_t cc = c - r * cpr;
    const bf16x8_t *hr = h + 2 * ((size_t)r * 2 * cpr);
    float g[16], u[16], a[16], sg[16], d[16], dg[16], du[16];
    load16(hr + 2 * cc, g);
    load16(hr + 2 * (cpr + cc), u);
    swiglu16(g, u, a, sg);
    uint32_t m;
    if (DS) {
      float dv[16];
      m = act_fq16_ds(q, a, dv);
      load16(daq + 2 * (size_t)c, d);
#pragma unroll
      for (int j = 0; j < 16; ++j) part = fmaf(d[j], dv[j], part);
    } else {
      m = act_fq16(q, a);
      load16(daq + 2 * (size_t)c, d);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float da = ((m >> j) & 1u) ? d[j] : 0.0f;
      const float s = sg[j];
      dg[j] = da * u[j] * s * (1.0f + g[j] * (1.0f - s));
      du[j] = da * g[j] * s;
    }
    bf16x8_t *dr = dh + 2 * ((size_t)r * 2 * cpr);
    store16(dr + 2 * cc, dg);
    store16(dr + 2 * (cpr + cc), du);
  }
  if (DS) {
    part = block_sum_fixed<kThreads>(part);
    if (threadIdx.x == 0) ds_part[blockIdx.x] = part;
  }
}

// out[t] = bf16(sum_j p[t,j] * o[row_of[t,j]]), j ascending, local slots only
__global__ __launch_bounds__(kThreads) void k_combine(const bf16x8_t *__restrict__ o,
                                                      const float *__restrict__ probs,
                                                      const int32_t *__restrict__ row_of, int topk,
                                                      FastDiv chunks_per_row, uint32_t nchunk,
                                                      bf16x8_t *__restrict__ out) {
  const uint32_t cpr = chunks_per_row.d;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += gridDim.x * blockDim.x) {
    uint32_t t = chunks_per_row.div(c);
    uint32_t cc = c - t * cpr;
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
    for (int j = 0; j < topk; ++j) {
      int r = row_of[t * topk + j];
      if (r < 0) continue;
      float p = probs[t * topk + j];
      float f[16];
      load16(o + 2 * ((size_t)r * cpr + cc), f);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc[i] + p * f[i];
    }
    store16(out + 2 * (size_t)c, acc);
  }
}

// do[r] = bf16(p[t,j] * dout[t]), f = perm[r]
// Per token: dout[t] is read once and dO[row_of[t, j]] = bf16(p[t,j] * dout[t])
// stored for each routed slot j; one 16-byte vector per lane (1 KiB of one
// routed row per wave store).
__global__ __launch_bounds__(kThreads) void k_combine_bwd(
    const bf16x8_t *__restrict__ dout, const float *__restrict__ probs,
    const int32_t *__restrict__ row_of, int topk, FastDiv vec_per_row, uint32_t nvec,
    bf16x8_t *__restrict__ dO) {
  const uint32_t vpr = vec_per_row.d;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nvec; c += gridDim.x * blockDim.x) {
    const uint32_t t = vec_per_row.div(c);
    const uint32_t cc = c - t * vpr;
    float d[8];
    unpack8(dout[c], d);
    for (int j = 0; j < topk; ++j) {
      const int r = row_of[t * topk + j];
      if (r < 0) continue;
      const float p = probs[t * topk + j];
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = p * d[i];
      dO[(size_t)r * vpr + cc] = pack8(o);
    }
  }
}

// dx[t] = bf16(m_a(x[t]) * sum_j dxq[row_of[t,j]]). DS: also the block's
// share of dS_a = sum over (t, h) of (sum_j dxq[row_of[t,j], h]) * dv/ds_a(x[t, h])
// into ds_part[blockIdx.x].
template <bool DS>
__global__ __launch_bounds__(kThreads) void k_unpermute_reduce(
    const bf16x8_t *__restrict__ dxq, const int32_t *__restrict__ row_of,
    const bf16x8_t *__restrict__ x, int topk, FastDiv chunks_per_row, uint32_t nchunk, int afmt,
    const float *__restrict__ ascale, bf16x8_t *__restrict__ dx, float *__restrict__ ds_part) {
  ActQ q = load_actq(afmt, ascale);
  const uint32_t cpr = chunks_per_row.d;
  float part = 0.0f;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += gridDim.x * blockDim.x) {
    uint32_t t = chunks_per_row.div(c);
    uint32_t cc = c - t * cpr;
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
    for (int j = 0; j < topk; ++j) {
      int r = row_of[t * topk + j];
      if (r < 0) continue;
      float f[16];
      load16(dxq + 2 * ((size_t)r * cpr + cc), f);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc[i] + f[i];
    }
    uint32_t m = 0xFFFFu;
    if (DS) {
      float xf[16], dv[16];
      load16(x + 2 * (size_t)c, xf);
      m = act_fq16_ds(q, xf, dv);
#pragma unroll
      for (int j = 0; j < 16; ++j) part = fmaf(acc[j], dv[j], part);
    } else if (afmt != FQ_FMT_NONE) {
      float xf[16];
      load16(x + 2 * (size_t)c, xf);
      m = act_fq16(q, xf);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = ((m >> j) & 1u) ? acc[j] : 0.0f;
    store16(dx + 2 * (size_t)c, acc);
  }
  if (DS) {
    part = block_sum_fixed<kThreads>(part);
    if (threadIdx.x == 0) ds_part[blockIdx.x] = part;
  }
}

}  // namespace

// ========================================================= launchers =======
// dst[e][r][c] = src[e][r][c] inside src's [rows_s, cols_s], else `fill`, for
// dst of [E, rows_d, cols_d]: zero-pads (rows_d >= rows_s, cols_d >= cols_s) or
// crops (<=) a stack of row-major matrices. n_rows (device, may be NULL): only
// the dst rows below n_rows[0] are written (routed-row tensors).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_reshape_copy(const T *__restrict__ src, int rows_s,
                                                           int cols_s, T *__restrict__ dst,
                                                           size_t n, int rows_d, int cols_d,
                                                           T fill, const int32_t *n_rows) {
  const int limit = n_rows ? *n_rows : rows_d;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t er = i / (size_t)cols_d;
    const int c = (int)(i - er * (size_t)cols_d);
    const size_t e = er / (size_t)rows_d;
    const int r = (int)(er - e * (size_t)rows_d);
    if (r >= limit) continue;
    dst[i] = (r < rows_s && c < cols_s) ? src[(e * rows_s + r) * (size_t)cols_s + c] : fill;
  }
}

void launch_reshape_u16(const uint16_t *src, int E, int rows_s, int cols_s, uint16_t *dst,
                        int rows_d, int cols_d, const int32_t *n_rows, hipStream_t st) {
  const size_t n = (size_t)E * rows_d * cols_d;
  if (!n) return;
  hipLaunchKernelGGL(k_reshape_copy<uint16_t>, dim3(grid_for((long)n, kThreads, 1 << 16)),
                     dim3(kThreads), 0, st, src, rows_s, cols_s, dst, n, rows_d, cols_d,
                     (uint16_t)0, n_rows);
}

void launch_reshape_f32(const float *src, int E, int rows_s, int cols_s, float *dst, int rows_d,
                        int cols_d, float fill, hipStream_t st) {
  const size_t n = (size_t)E * rows_d * cols_d;
  if (!n) return;
  hipLaunchKernelGGL(k_reshape_copy<float>, dim3(grid_for((long)n, kThreads, 1 << 16)),
                     dim3(kThreads), 0, st, src, rows_s, cols_s, dst, n, rows_d, cols_d, fill,
                     (const int32_t *)nullptr);
}

void launch_fill_u32(uint32_t *p, uint32_t v, long n, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n)), dim3(kThreads), 0, st, p, v, n);
}

void launch_repeat_rows(const float *v, int rows, int n, float *out, hipStream_t st) {
  const uint32_t total = (uint32_t)((size_t)rows * n);
  if (!total) return;
  hipLaunchKernelGGL(k_repeat_rows, dim3(grid_for(total)), dim3(kThreads), 0, st, v, total,
                     FastDiv((uint32_t)n), out);
}

void launch_sum_rows(const float *in, int rows, int n, float *out, hipStream_t st) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_sum_rows, dim3(rows), dim3(kThreads), 0, st, in, (uint32_t)n, out);
}

void launch_quantize_stacked(const uint16_t *w, fq_shape s, const fq_weight_q &q, uint16_t *out,
                             uint8_t *codes, hipStream_t st) {
  uint32_t nvec = (uint32_t)((size_t)s.E * s.N * s.K / 8);
  FastDiv vpe((uint32_t)((size_t)s.N * s.K / 8)), vpg(q.group / 8);
  dim3 grid(grid_for(ceil_div((long)nvec, kQU), kThreads, kQGridCap)), block(kThreads);
  auto wv = reinterpret_cast<const bf16x8_t *>(w);
  auto ov = reinterpret_cast<bf16x8_t *>(out);
#define FQ_QS(F)                                                                        \
  hipLaunchKernelGGL(k_quantize_stacked<F>, grid, block, 0, st, wv, nvec, vpe, vpg, q.scale, \
                     q.zero_point, q.global_scale, ov, codes)
  switch (q.fmt) {
    case FQ_FMT_INT8: FQ_QS(FQ_FMT_INT8); break;
    case FQ_FMT_INT4: FQ_QS(FQ_FMT_INT4); break;
    case FQ_FMT_FP8_E4M3: FQ_QS(FQ_FMT_FP8_E4M3); break;
    default: FQ_QS(FQ_FMT_NVFP4); break;
  }
#undef FQ_QS
}

void launch_observer_weight(const uint16_t *w, fq_shape s, int fmt, int group, float *scale,
                            float *zero_point, float *gscale, hipStream_t st) {
  auto wv = reinterpret_cast<const bf16x8_t *>(w);
  uint32_t nvec = (uint32_t)((size_t)s.E * s.N * s.K / 8);
  int vpg = group / 8;
  if (fmt == FQ_FMT_NVFP4) {
    auto gbits = reinterpret_cast<uint32_t *>(gscale);
    hipLaunchKernelGGL(k_observer_lanes<FQ_FMT_NVFP4>, dim3(grid_for(nvec)), dim3(kThreads), 0, st,
                       wv, nvec, vpg, scale, zero_point);
    uint32_t nb = (uint32_t)((size_t)s.E * s.N * (s.K / group));
    hipLaunchKernelGGL(k_expert_amax, dim3(s.E), dim3(kThreads), 0, st, scale,
                       (uint32_t)((size_t)s.N * (s.K / group)), gbits);
    FastDiv bpe((uint32_t)((size_t)s.N * (s.K / group)));
    hipLaunchKernelGGL(k_nvfp4_theta, dim3(grid_for(nb)), dim3(kThreads), 0, st, scale, nb, bpe,
                       gbits);
    hipLaunchKernelGGL(k_nvfp4_global, dim3(ceil_div(s.E, kThreads)), dim3(kThreads), 0, st, gbits,
                       s.E);
    return;
  }
  bool lanes = vpg <= 64 && (vpg & (vpg - 1)) == 0;
  if (lanes) {
#define FQ_OBL(F)                                                                               \
  hipLaunchKernelGGL(k_observer_lanes<F>, dim3(grid_for(nvec)), dim3(kThreads), 0, st, wv, nvec, \
                     vpg, scale, zero_point)
    switch (fmt) {
      case FQ_FMT_INT8: FQ_OBL(FQ_FMT_INT8); break;
      case FQ_FMT_INT4: FQ_OBL(FQ_FMT_INT4); break;
      default: FQ_OBL(FQ_FMT_FP8_E4M3); break;
    }
#undef FQ_OBL
  } else {
    uint32_t ngroups = nvec / vpg;
#define FQ_OBB(F) \
  hipLaunchKernelGGL(k_observer_block<F>, dim3(ngroups), dim3(kThreads), 0, st, wv, vpg, scale, zero_point)
    switch (fmt) {
      case FQ_FMT_INT8: FQ_OBB(FQ_FMT_INT8); break;
      case FQ_FMT_INT4: FQ_OBB(FQ_FMT_INT4); break;
      default: FQ_OBB(FQ_FMT_FP8_E4M3); break;
    }
#undef FQ_OBB
  }
}

void launch_observer_tensor(const uint16_t *x, size_t n, int fmt, float *scale, hipStream_t st) {
  auto bits = reinterpret_cast<uint32_t *>(scale);
  launch_fill_u32(bits, 0u, 1, st);
  uint32_t nvec = (uint32_t)(n / 8);
  if (nvec)
    hipLaunchKernelGGL(k_absmax_tensor, dim3(grid_for(nvec, kThreads, 2048)), dim3(kThreads), 0, st,
                       reinterpret_cast<const bf16x8_t *>(x), nvec, bits);
  float div = fmt == FQ_FMT_FP8_E4M3 ? kE4M3Max : fmt == FQ_FMT_NVFP4 ? kE2M1Max * kE4M3Max : 127.0f;
  hipLaunchKernelGGL(k_act_scale_finalize, dim3(1), dim3(64), 0, st, bits, div);
}

void launch_act_fq(const uint16_t *x, size_t M, int K, const int32_t *n_rows, int afmt,
                   const float *ascale, uint16_t *xq, hipStream_t st) {
  uint32_t nvec = (uint32_t)(M * K / 8);
  if (!nvec) return;
  hipLaunchKernelGGL(k_act_fq, dim3(grid_for(nvec)), dim3(kThreads), 0, st,
                     reinterpret_cast<const bf16x8_t *>(x), nvec, n_rows, (uint32_t)(K / 8), afmt,
                     ascale, reinterpret_cast<bf16x8_t *>(xq));
}

void launch_act_mask(uint16_t *dx, const uint16_t *x, size_t M, int K, const int32_t *n_rows,
                     int afmt, const float *ascale, hipStream_t st) {
  uint32_t nchunk = (uint32_t)(M * K / 16);
  if (!nchunk) return;
  hipLaunchKernelGGL(k_act_mask, dim3(grid_for(nchunk)), dim3(kThreads), 0, st,
                     reinterpret_cast<bf16x8_t *>(dx), reinterpret_cast<const bf16x8_t *>(x), nchunk,
                     n_rows, (uint32_t)(K / 16), afmt, ascale);
}

void launch_gather_actfq(const uint16_t *x, int T, int H, const int32_t *row_of, int topk,
                         int afmt, const float *ascale, uint16_t *xq, hipStream_t st) {
  const uint32_t nvec = (uint32_t)((size_t)T * H / 8);
  if (!nvec) return;
  hipLaunchKernelGGL(k_gather_actfq, dim3(grid_for(nvec)), dim3(kThreads), 0, st,
                     reinterpret_cast<const bf16x8_t *>(x), row_of, topk, FastDiv(H / 8), nvec,
                     afmt, ascale, reinterpret_cast<bf16x8_t *>(xq));
}

void launch_swiglu_actfq(const uint16_t *h, int R_max, const int32_t *n_rows, int F, int afmt,
                         const float *ascale, uint16_t *a, uint16_t *aq, hipStream_t st) {
  const uint32_t maxv = (uint32_t)((size_t)R_max * F / 8);
  if (!maxv) return;
  hipLaunchKernelGGL(k_swiglu_actfq, dim3(grid_for(maxv)), dim3(kThreads), 0, st,
                     reinterpret_cast<const bf16x8_t *>(h), FastDiv(F / 8), maxv, n_rows, afmt, ascale,
                     reinterpret_cast<bf16x8_t *>(a), reinterpret_cast<bf16x8_t *>(aq));
}

long act_grad_partials(long rows, int cols) { return grid_for(rows * cols / 16); }

void launch_swiglu_bwd(const uint16_t *daq, const uint16_t *h, int R_max, const int32_t *n_rows,
                       int F, int afmt, const float *ascale, uint16_t *dh, float *dscale_a,
                       float *part, hipStream_t st) {
  uint32_t maxc = (uint32_t)((size_t)R_max * F / 16);
  const int grid = grid_for(maxc);
  auto dq = reinterpret_cast<const bf16x8_t *>(daq);
  auto hv = reinterpret_cast<const bf16x8_t *>(h);
  auto dv = reinterpret_cast<bf16x8_t *>(dh);
  if (!dscale_a) {
    if (!maxc) return;
    hipLaunchKernelGGL(k_swiglu_bwd<false>, dim3(grid), dim3(kThreads), 0, st, dq, hv,
                       FastDiv(F / 16), maxc, n_rows, afmt, ascale, dv, nullptr);
    return;
  }
  if (maxc)
    hipLaunchKernelGGL(k_swiglu_bwd<true>, dim3(grid), dim3(kThreads), 0, st, dq, hv,
                       FastDiv(F / 16), maxc, n_rows, afmt, ascale, dv, part);
  hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(kSumThreads), 0, st, part,
                     maxc ? (uint32_t)grid : 0u, dscale_a);
}

void launch_combine(const uint16_t *o, const float *probs, const int32_t *row_of, int T, int topk,
                    int H, uint16_t *out, hipStream_t st) {
  uint32_t nchunk = (uint32_t)((size_t)T * H / 16);
  if (!nchunk) return;
  hipLaunchKernelGGL(k_combine, dim3(grid_for(nchunk)), dim3(kThreads), 0, st,
                     reinterpret_cast<const bf16x8_t *>(o), probs, row_of, topk, FastDiv(H / 16),
                     nchunk, reinterpret_cast<bf16x8_t *>(out));
}

void launch_combine_bwd(const uint16_t *dout, const float *probs, const int32_t *row_of, int T,
                        int topk, int H, uint16_t *dO, hipStream_t st) {
  const uint32_t nvec = (uint32_t)((size_t)T * H / 8);
  if (!nvec) return;
  hipLaunchKernelGGL(k_combine_bwd, dim3(grid_for(nvec)), dim3(kThreads), 0, st,
                     reinterpret_cast<const bf16x8_t *>(dout), probs, row_of, topk, FastDiv(H / 8),
                     nvec, reinterpret_cast<bf16x8_t *>(dO));
}

void launch_unpermute_reduce(const uint16_t *dxq, const int32_t *row_of, const uint16_t *x, int T,
                             int topk, int H, int afmt, const float *ascale, uint16_t *dx,
                             float *dscale_a, float *part, hipStream_t st) {
  uint32_t nchunk = (uint32_t)((size_t)T * H / 16);
  const int grid = grid_for(nchunk);
  auto dq = reinterpret_cast<const bf16x8_t *>(dxq);
  auto xv = reinterpret_cast<const bf16x8_t *>(x);
  auto dv = reinterpret_cast<bf16x8_t *>(dx);
  if (!dscale_a) {
    if (!nchunk) return;
    hipLaunchKernelGGL(k_unpermute_reduce<false>, dim3(grid), dim3(kThreads), 0, st, dq, row_of,
                       xv, topk, FastDiv(H / 16), nchunk, afmt, ascale, dv, nullptr);
    return;
  }
  if (nchunk)
    hipLaunchKernelGGL(k_unpermute_reduce<true>, dim3(grid), dim3(kThreads), 0, st, dq, row_of,
                       xv, topk, FastDiv(H / 16), nchunk, afmt, ascale, dv, part);
  hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(kSumThreads), 0, st, part,
                     nchunk ? (uint32_t)grid : 0u, dscale_a);
}

}  // namespace fq
