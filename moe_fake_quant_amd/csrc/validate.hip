// Checks of the device-data preconditions that the release entry points
// assume and do not check (the host cannot see device data without a sync):
// routing ids in range, segment offsets that start at 0, never decrease and
// stay within the row buffers, and finite, positive quantizer scales (an
// NVFP4 block parameter may be 0: such a block quantizes to +0.0). The
// kernels only read their inputs and OR one bit per failed condition into a
// status word; they never trap, so a bad input is reported, not faulted on.
#include "internal.hpp"

namespace fq {

namespace {

constexpr int kThreads = 256;

// one flagged lane per wave posts the bit (a divergent vector atomic)
__device__ __forceinline__ void post(bool bad, uint32_t bit, uint32_t *status) {
  const unsigned long long any = __ballot(bad);
  if (any && (threadIdx.x & 63) == (uint32_t)__builtin_ctzll(any)) atomicOr(status, bit);
}

__global__ __launch_bounds__(kThreads) void k_check_ids(const int32_t *__restrict__ ids, long n,
                                                        int n_experts, uint32_t *status) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i - threadIdx.x < n;
       i += (long)gridDim.x * blockDim.x) {
    bool bad = false;
    if (i < n) {
      const int v = ids[i];
      bad = v < 0 || v >= n_experts;
    }
    post(bad, FQ_BAD_EXPERT_ID, status);
  }
}

__global__ __launch_bounds__(kThreads) void k_check_seg(const int32_t *__restrict__ seg, int E,
                                                        int R_max, uint32_t *status) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i - (int)threadIdx.x <= E;
       i += gridDim.x * blockDim.x) {
    bool start = false, order = false, end = false;
    if (i <= E) {
      const int v = seg[i];
      if (i == 0) start = v != 0;
      if (i < E) order = seg[i + 1] < v;
      if (i == E) end = v > R_max || v < 0;
    }
    post(start, FQ_BAD_SEG_START, status);
    post(order, FQ_BAD_SEG_ORDER, status);
    post(end, FQ_BAD_SEG_END, status);
  }
}

// mode 0: finite and > 0; 1: finite and >= 0; 2: finite
__global__ __launch_bounds__(kThreads) void k_check_f32(const float *__restrict__ v, long n, int mode,
                                                        uint32_t bit, uint32_t *status) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i - threadIdx.x < n;
       i += (long)gridDim.x * blockDim.x) {
    bool bad = false;
    if (i < n) {
      const float x = v[i];
      const bool fin = (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u;
      bad = !fin || (mode == 0 && !(x > 0.0f)) || (mode == 1 && !(x >= 0.0f));
    }
    post(bad, bit, status);
  }
}

int grid_of(long n) {
  const long b = (n + kThreads - 1) / kThreads;
  return (int)(b < 1 ? 1 : b > 4096 ? 4096 : b);
}

}  // namespace

void launch_validate(const int32_t *ids, long n_ids, int n_experts, const int32_t *seg, int E,
                     int R_max, const float *scale, long n_scale, int scale_mode,
                     const float *zero_point, const float *gscale, int n_g, const float *act_scale,
                     uint32_t *status, hipStream_t st) {
  launch_fill_u32(status, 0u, 1, st);
  if (ids && n_ids > 0)
    hipLaunchKernelGGL(k_check_ids, dim3(grid_of(n_ids)), dim3(kThreads), 0, st, ids, n_ids,
                       n_experts, status);
  if (seg)
    hipLaunchKernelGGL(k_check_seg, dim3(grid_of((long)E + 1)), dim3(kThreads), 0, st, seg, E,
                       R_max, status);
  if (scale && n_scale > 0)
    hipLaunchKernelGGL(k_check_f32, dim3(grid_of(n_scale)), dim3(kThreads), 0, st, scale, n_scale,
                       scale_mode, (uint32_t)FQ_BAD_SCALE, status);
  if (zero_point && n_scale > 0)
    hipLaunchKernelGGL(k_check_f32, dim3(grid_of(n_scale)), dim3(kThreads), 0, st, zero_point,
                       n_scale, 2, (uint32_t)FQ_BAD_ZERO_POINT, status);
  if (gscale && n_g > 0)
    hipLaunchKernelGGL(k_check_f32, dim3(1), dim3(kThreads), 0, st, gscale, (long)n_g, 0,
                       (uint32_t)FQ_BAD_GLOBAL_SCALE, status);
  if (act_scale)
    hipLaunchKernelGGL(k_check_f32, dim3(1), dim3(kThreads), 0, st, act_scale, 1l, 0,
                       (uint32_t)FQ_BAD_ACT_SCALE, status);
}

}  // namespace fq
