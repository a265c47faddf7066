// Measured peaks of the part, for the benchmark's roofline context (not part
// of the fake-quant path): a register-only chain of bf16 MFMAs and a plain
// device copy. C ABI, launched on the caller's stream; the caller times them.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8v;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 operand pair: varied values around 0.1 .. 1 with random signs
// (random_data != 0), or all 1.0. The MFMA clock under load depends on the
// operand bits, so both are reported.
__device__ __forceinline__ uint32_t operand_word(uint32_t i, int random_data) {
  if (!random_data) return 0x3f803f80u;
  const uint32_t h = mix(i * 2654435761u + 12345u);
  const uint32_t lo = (0x3dc0u + (h & 0x1ffu)) | (((h >> 18) & 1u) << 15);
  const uint32_t hi = (0x3dc0u + ((h >> 9) & 0x1ffu)) | (((h >> 19) & 1u) << 15);
  return lo | (hi << 16);
}

// 8 independent accumulators per wave, `iters` rounds of 8 MFMA 32x32x16
__global__ __launch_bounds__(256) void k_mfma_chain(float *out, int iters, int random_data) {
  uint32_t wa[4], wb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wa[i] = operand_word(threadIdx.x * 8u + i + blockIdx.x * 4096u, random_data);
    wb[i] = operand_word(threadIdx.x * 8u + 4u + i + blockIdx.x * 4096u + 777u, random_data);
  }
  bf16x8v a, b;
  __builtin_memcpy(&a, wa, 16);
  __builtin_memcpy(&b, wb, 16);
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// one 16-byte vector per thread
__global__ __launch_bounds__(256) void k_copy16(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                size_t n16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

// out[t] = XOR over the routed rows r = row_of[t, j] (j < topk, r >= 0) of
// rows[r]: the access pattern of the per-token reductions over routed rows
// (topk scattered row reads per row written), 16 bytes per thread, with no
// arithmetic to speak of.
__global__ __launch_bounds__(256) void k_scattered_rows(const uint4 *__restrict__ rows,
                                                        const int32_t *__restrict__ row_of, int T,
                                                        int topk, int cpr, uint4 *__restrict__ out) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * cpr) return;
  const int t = (int)(i / cpr), c = (int)(i - (size_t)t * cpr);
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int j = 0; j < topk; ++j) {
    const int r = row_of[(size_t)t * topk + j];
    if (r < 0) continue;
    const uint4 v = rows[(size_t)r * cpr + c];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  out[i] = acc;
}

// rows[r] = src[t] for the routed rows r = row_of[t, j] (j < topk, r >= 0):
// the mirror pattern (one token row read, topk scattered row writes), as
// the combine backward moves its rows.
__global__ __launch_bounds__(256) void k_scattered_rows_w(const uint4 *__restrict__ src,
                                                          const int32_t *__restrict__ row_of, int T,
                                                          int topk, int cpr,
                                                          uint4 *__restrict__ rows) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)T * cpr) return;
  const int t = (int)(i / cpr), c = (int)(i - (size_t)t * cpr);
  const uint4 v = src[i];
  for (int j = 0; j < topk; ++j) {
    const int r = row_of[(size_t)t * topk + j];
    if (r >= 0) rows[(size_t)r * cpr + c] = v;
  }
}

// The memory pattern of the top-K KL kernel with none of its selection or
// softmax work. One workgroup per token: the teacher row is read once
// (coalesced, 16 bytes per lane, four loads in flight) and folded into x;
// then student[t, idx[t, k]] is read for k < K (K scattered 2-byte reads);
// the outputs are 8K + 4 bytes per token like the KL kernel's (an index and
// an fp32 value per entry, one fp32 per token). V is a multiple of 8.
__global__ __launch_bounds__(512) void k_stream_gather(const uint4 *__restrict__ teacher,
                                                       const uint16_t *__restrict__ student,
                                                       const int32_t *__restrict__ idx, int V, int K,
                                                       int32_t *__restrict__ out_i,
                                                       float *__restrict__ out_f,
                                                       uint32_t *__restrict__ out_l) {
  __shared__ uint32_t red[8];
  const int t = blockIdx.x;
  const int n16 = V / 8;
  const uint4 *row = teacher + (size_t)t * n16;
  uint32_t x = 0;
  int i = threadIdx.x;
  for (; i + 3 * 512 < n16; i += 4 * 512) {
    const uint4 a = row[i], b = row[i + 512], c = row[i + 1024], d = row[i + 1536];
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += 512) {
    const uint4 a = row[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = red[0] ^ red[1] ^ red[2] ^ red[3] ^ red[4] ^ red[5] ^ red[6] ^ red[7];
  const uint16_t *srow = student + (size_t)t * V;
  for (int k = threadIdx.x; k < K; k += 512) {
    const int j = idx[(size_t)t * K + k];
    out_i[(size_t)t * K + k] = j ^ (int)(x & 1u);
    out_f[(size_t)t * K + k] = __uint_as_float((uint32_t)srow[j] << 16);
  }
  if (threadIdx.x == 0) out_l[t] = x;
}

// 16 bytes per lane from global memory into LDS (lds_wave_base + 16 * lane),
// the lane reading base + off, base uniform in scalar registers; the asm
// starts with the wait states a base register or M0 written just before need.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, char *lds_wave_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "{m0}"(m0v)
               : "memory");
}

constexpr size_t kStreamPanel = (size_t)256 * 4096;  // 256 rows of 4 KiB

// The forward grouped GEMM's operand stream alone, with its ring and its
// panel sharing: per 64-deep stage each 8-wave block moves 256 rows x 128 B
// of an X panel and of a W panel (4 KiB rows, as at hidden 2048) into a
// two-stage LDS ring with global_load_lds, waits for the stage, and issues
// the next; no MFMAs. A tile is 32 stages. On each XCD (blocks b % 8) the X
// panel of a tile is shared by 6 consecutive blocks and its W panel by every
// 6th, as the forward's (row tile, i tile) list shares them.
__global__ __launch_bounds__(512) void k_operand_stream(const char *xs, const char *ws, int npx,
                                                       int npw, int ntiles) {
  __shared__ __attribute__((aligned(1024))) char ring[2 * 65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nst = ntiles * 32;
  auto issue = [&](int t) {
    const int tile = t >> 5, kt = t & 31;
    const int px = ((tile * 8 + xcd) * 6 + slot / 6) % npx;
    const int pw = ((tile * 8 + xcd) * 6 + slot % 6) % npw;
    char *st = ring + (t & 1) * 65536;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const uint32_t off =
          (uint32_t)(((wave * 4 + ii) * 8 + (lane >> 3)) * 4096 + kt * 128 + (lane & 7) * 16);
      dma16(xs + (size_t)px * kStreamPanel, off, st + (wave * 4 + ii) * 1024);
      dma16(ws + (size_t)pw * kStreamPanel, off, st + 32768 + (wave * 4 + ii) * 1024);
    }
  };
  issue(0);
  for (int t = 0; t < nst; ++t) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of stage t
    asm volatile("s_barrier" ::: "memory");
    if (t + 1 < nst) issue(t + 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace

extern "C" {

// xs, ws: device buffers of at least panels * 1 MiB each (panels >= 1);
// blocks a multiple of 8. Moves blocks * ntiles * 32 * 64 KiB.
int fqp_operand_stream(const void *xs, const void *ws, int panels, int blocks, int ntiles,
                       void *stream) {
  if (!xs || !ws || panels <= 0 || blocks <= 0 || blocks % 8 != 0 || ntiles <= 0) return 1;
  hipLaunchKernelGGL(k_operand_stream, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                     (const char *)xs, (const char *)ws, panels, panels, ntiles);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// flops = 32*32*16*2 * 8 * iters * blocks * 4 waves. out: blocks * 256 floats.
int fqp_mfma_chain(float *out, int blocks, int iters, int random_data, void *stream) {
  if (!out || blocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(k_mfma_chain, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters,
                     random_data);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// bytes: a multiple of 16; src and dst 16-byte aligned device buffers
int fqp_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes % 16 != 0) return 1;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  const size_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(k_copy16, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4 *)src, (uint4 *)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// rows: [R, row_bytes] with R > every row_of entry; out: [T, row_bytes];
// row_bytes a multiple of 16
int fqp_scattered_rows(const void *rows, const int32_t *row_of, int T, int topk, int row_bytes,
                       void *out, void *stream) {
  if (!rows || !row_of || !out || T < 0 || topk <= 0 || row_bytes <= 0 || row_bytes % 16 != 0)
    return 1;
  const int cpr = row_bytes / 16;
  const size_t n = (size_t)T * cpr;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_scattered_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, (const uint4 *)rows, row_of, T, topk, cpr, (uint4 *)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}


// src: [T, row_bytes]; rows: [R, row_bytes] with R > every row_of entry;
// row_bytes a multiple of 16
int fqp_scattered_rows_w(const void *src, const int32_t *row_of, int T, int topk, int row_bytes,
                         void *rows, void *stream) {
  if (!src || !row_of || !rows || T < 0 || topk <= 0 || row_bytes <= 0 || row_bytes % 16 != 0)
    return 1;
  const int cpr = row_bytes / 16;
  const size_t n = (size_t)T * cpr;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_scattered_rows_w, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, (const uint4 *)src, row_of, T, topk, cpr, (uint4 *)rows);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// teacher, student: [T, V] bf16, V a multiple of 8, rows 16-byte aligned;
// idx: [T, K] int32, every entry in [0, V) (the caller checks); out_i, out_f:
// [T, K]; out_l: [T]
int fqp_stream_gather(const void *teacher, const uint16_t *student, const int32_t *idx, int T,
                      int V, int K, int32_t *out_i, float *out_f, uint32_t *out_l, void *stream) {
  if (!teacher || !student || !idx || !out_i || !out_f || !out_l || T < 0 || V <= 0 || V % 8 != 0 ||
      K <= 0 || K > V)
    return 1;
  if (T == 0) return 0;
  hipLaunchKernelGGL(k_stream_gather, dim3((unsigned)T), dim3(512), 0, (hipStream_t)stream,
                     (const uint4 *)teacher, student, idx, V, K, out_i, out_f, out_l);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
