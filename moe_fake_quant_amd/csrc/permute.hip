// Routed-token permutation on gfx950: a stable counting sort of the
// (token, slot) pairs by local expert, so that one grouped GEMM sees each
// expert's rows contiguous (AngelSlim mcore_qad article, section 二.4).
//
//   pass 1  per 256-pair chunk: per-expert counts (LDS histogram)
//   pass 2  per expert: exclusive scan of its chunk counts (one block each)
//   pass 3  one block: exclusive scan of the expert totals -> seg_offsets
//   pass 4  per chunk: stable rank of each pair among the chunk's pairs of
//           the same expert, position = seg + chunk offset + rank
// No atomics decide an order, so the result is unique and deterministic.
#include <mutex>

#include "internal.hpp"

namespace fq {

namespace {

constexpr int kChunk = 256;

__global__ __launch_bounds__(kChunk) void k_perm_count(const int32_t *__restrict__ ids, int P,
                                                       int ebegin, int E, int nchunk,
                                                       int32_t *__restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  int f = blockIdx.x * kChunk + threadIdx.x;
  if (f < P) {
    int e = ids[f] - ebegin;
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)e * nchunk + blockIdx.x] = hist[e];
}

// block-wide exclusive scan of one value per thread; returns the block total
__device__ int block_exclusive_scan(int v, int &excl) {
  __shared__ int wsum[kChunk / 64];
  int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int k = 0; k < kChunk / 64; ++k) {
    if (k < w) before += wsum[k];
    total += wsum[k];
  }
  __syncthreads();
  excl = before + x - v;
  return total;
}

__global__ __launch_bounds__(kChunk) void k_perm_scan_chunks(int32_t *__restrict__ counts, int nchunk,
                                                             int32_t *__restrict__ totals) {
  int32_t *c = counts + (size_t)blockIdx.x * nchunk;
  int running = 0;
  for (int base = 0; base < nchunk; base += kChunk) {
    int i = base + threadIdx.x;
    int v = i < nchunk ? c[i] : 0;
    int excl;
    int tot = block_exclusive_scan(v, excl);
    if (i < nchunk) c[i] = running + excl;
    running += tot;
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = running;
}

__global__ __launch_bounds__(kChunk) void k_perm_scan_experts(const int32_t *__restrict__ totals, int E,
                                                              int32_t *__restrict__ seg) {
  int running = 0;
  for (int base = 0; base < E; base += kChunk) {
    int i = base + threadIdx.x;
    int v = i < E ? totals[i] : 0;
    int excl;
    int tot = block_exclusive_scan(v, excl);
    if (i < E) seg[i] = running + excl;
    running += tot;
  }
  if (threadIdx.x == 0) seg[E] = running;
}

__global__ __launch_bounds__(kChunk) void k_perm_scatter(const int32_t *__restrict__ ids, int P,
                                                         int ebegin, int E, int nchunk,
                                                         const int32_t *__restrict__ chunk_off,
                                                         const int32_t *__restrict__ seg,
                                                         int32_t *__restrict__ perm,
                                                         int32_t *__restrict__ row_of) {
  __shared__ int32_t le[kChunk];
  int f = blockIdx.x * kChunk + threadIdx.x;
  int e = -1;
  if (f < P) {
    e = ids[f] - ebegin;
    if (e < 0 || e >= E) e = -1;
  }
  le[threadIdx.x] = e;
  __syncthreads();
  if (f >= P) return;
  if (e < 0) {
    row_of[f] = -1;
    return;
  }
  int rank = 0;
  for (int j = 0; j < (int)threadIdx.x; ++j) rank += (le[j] == e);
  int pos = seg[e] + chunk_off[(size_t)e * nchunk + blockIdx.x] + rank;
  perm[pos] = f;
  row_of[f] = pos;
}

}  // namespace

// Scratch of the allocation-free permute entry point: the per-chunk counts
// and expert totals live in this array instead of a caller workspace. Each
// GPU the library runs on holds its own copy until the process ends. Every
// entry of the counts and totals a call uses is written before it is read,
// so nothing needs clearing between calls; calls that overlap on one GPU
// share the array and race.
static __device__ __align__(256) int32_t scratch[kPermuteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_dev[kMaxDevices] = {};
}  // namespace

fq_status permute_scratch(int32_t **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "permute scratch: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("permute scratch: device %d outside 0..%d", dev, kMaxDevices - 1);
    return FQ_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    // the array's device address on the current device (the host-side name
    // is only a stand-in, never passed to a kernel)
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "permute scratch: hipGetSymbolAddress");
    g_scratch_dev[dev] = static_cast<int32_t *>(p);
  }
  *out = g_scratch_dev[dev];
  return FQ_OK;
}

size_t permute_workspace_bytes(int E, long P) {
  long nchunk = (P + kChunk - 1) / kChunk;
  if (nchunk < 1) nchunk = 1;
  return sizeof(int32_t) * ((size_t)E * nchunk + (size_t)E);
}

void launch_permute(const int32_t *ids, int T, int topk, int ebegin, int E, int32_t *perm,
                    int32_t *row_of, int32_t *seg, void *ws, hipStream_t st) {
  int P = T * topk;
  int nchunk = (P + kChunk - 1) / kChunk;
  if (nchunk < 1) nchunk = 1;
  int32_t *counts = static_cast<int32_t *>(ws);
  int32_t *totals = counts + (size_t)E * nchunk;
  hipLaunchKernelGGL(k_perm_count, dim3(nchunk), dim3(kChunk), E * sizeof(int32_t), st, ids, P, ebegin,
                     E, nchunk, counts);
  hipLaunchKernelGGL(k_perm_scan_chunks, dim3(E), dim3(kChunk), 0, st, counts, nchunk, totals);
  hipLaunchKernelGGL(k_perm_scan_experts, dim3(1), dim3(kChunk), 0, st, totals, E, seg);
  if (P > 0)
    hipLaunchKernelGGL(k_perm_scatter, dim3(nchunk), dim3(kChunk), 0, st, ids, P, ebegin, E, nchunk,
                       counts, seg, perm, row_of);
}

}  // namespace fq
