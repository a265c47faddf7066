// Top-K KL distillation on gfx950: the loss between the student's and the
// (quantization-off) teacher's logits over the teacher's K most likely tokens
// per position, and its gradient on the student logits, without forming the
// [tokens, vocab] probabilities (AngelSlim mcore_qad article, section 二.5;
// the forward / reverse top-K variants of the QAT + ZeRO-3 page's loss table).
//
// One workgroup per token row. The K-th largest teacher logit is found
// exactly with two 256-bin histogram passes over an order-preserving 16-bit
// key of the bf16 logits (high byte, then low byte inside the chosen high
// bin); a third pass compacts the selected entries in vocabulary order into
// LDS (equal logits at the threshold: the lower indices first) and stops as
// soon as K are found. The student logits are gathered at those K indices;
// both restricted softmaxes, the loss and the gradient come from LDS.
#include "internal.hpp"

namespace fq {

namespace {

constexpr int kKT = 1024;          // threads per row
constexpr int kKW = kKT / 64;      // waves per row

struct KLShared {
  uint32_t hist[kKW][256];         // per-wave histograms
  uint32_t scan[kKW];
  float red[kKW];
  uint32_t sel_bin, sel_above;
  int32_t idx[kTopKMax];
  float tv[kTopKMax];
  float sv[kTopKMax];
};

// bf16 bits -> 16-bit key whose unsigned order is the value order (-0 and +0
// get one key: they are equal logits)
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over the block in thread order; total to every thread.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total, KLShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == 63) sh.scan[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kKW; ++w) {
    const uint32_t x = sh.scan[w];
    before += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();  // scan[] is reused by the next call
  total = tot;
  return before + incl - v;
}

// Block sum / max in a fixed order (butterfly in each wave, then the waves in
// index order); the result in every thread.
__device__ __forceinline__ float block_sum(float v, KLShared &sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = sh.red[0];
#pragma unroll
  for (int w = 1; w < kKW; ++w) s += sh.red[w];
  __syncthreads();
  return s;
}
__device__ __forceinline__ float block_max(float v, KLShared &sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = sh.red[0];
#pragma unroll
  for (int w = 1; w < kKW; ++w) s = fmaxf(s, sh.red[w]);
  __syncthreads();
  return s;
}

__device__ __forceinline__ void zero_hist(KLShared &sh) {
  uint32_t *h = &sh.hist[0][0];
  for (int i = threadIdx.x; i < kKW * 256; i += kKT) h[i] = 0u;
  __syncthreads();
}

// Sum the per-wave histograms into hist[0], then find the bin b (scanning
// from 255 down) with above(b) < need <= above(b) + count(b), where above(b)
// counts the entries of the higher bins. Requires need <= total.
__device__ __forceinline__ void find_bin(KLShared &sh, uint32_t need) {
  if (threadIdx.x < 256) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kKW; ++w) s += sh.hist[w][threadIdx.x];
    sh.hist[0][threadIdx.x] = s;  // only this thread touches bin threadIdx.x
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = sh.hist[0][255 - 4 * lane - j];
      sum += c[j];
    }
    uint32_t acc = wave_incl_scan(sum, lane) - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (acc < need && acc + c[j] >= need) {
        sh.sel_bin = 255u - 4u * lane - j;
        sh.sel_above = acc;
      }
      acc += c[j];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void k_count_valid(const uint8_t *__restrict__ valid, int T,
                                                     float *__restrict__ inv_n) {
  __shared__ uint32_t red[4];
  uint32_t n = 0;
  for (int i = threadIdx.x; i < T; i += 256) n += valid ? (valid[i] != 0) : 1u;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t tot = red[0] + red[1] + red[2] + red[3];
    inv_n[0] = 1.0f / (float)(tot > 0 ? tot : 1u);
  }
}

template <bool REVERSE>
__global__ __launch_bounds__(kKT) void k_topk_kl(const uint16_t *__restrict__ student,
                                                 const uint16_t *__restrict__ teacher, int V, int K,
                                                 const uint8_t *__restrict__ valid,
                                                 const float *__restrict__ inv_n,
                                                 int32_t *__restrict__ out_idx,
                                                 float *__restrict__ out_grad,
                                                 float *__restrict__ loss_tok) {
  __shared__ KLShared sh;
  const int t = threadIdx.x, wave = t >> 6;
  const size_t row = blockIdx.x;
  const uint4 *trow = reinterpret_cast<const uint4 *>(teacher + row * (size_t)V);
  const uint32_t nvec = (uint32_t)V / 8u;

  // pass 1: histogram of the key's high byte
  zero_hist(sh);
  for (uint32_t v = t; v < nvec; v += kKT) {
    const uint4 q = trow[v];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t key = order_key((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
      atomicAdd(&sh.hist[wave][key >> 8], 1u);
    }
  }
  __syncthreads();
  find_bin(sh, (uint32_t)K);
  const uint32_t hi = sh.sel_bin, above_hi = sh.sel_above;

  // pass 2: histogram of the low byte inside the chosen high byte
  zero_hist(sh);
  for (uint32_t v = t; v < nvec; v += kKT) {
    const uint4 q = trow[v];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t key = order_key((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
      if ((key >> 8) == hi) atomicAdd(&sh.hist[wave][key & 0xFFu], 1u);
    }
  }
  __syncthreads();
  find_bin(sh, (uint32_t)K - above_hi);
  const uint32_t tau = (hi << 8) | sh.sel_bin;            // key of the K-th largest
  const uint32_t need_ties = (uint32_t)K - above_hi - sh.sel_above;

  // pass 3: keys above tau, then the first need_ties keys equal to tau, in
  // vocabulary order, compacted into LDS; stops once K are in
  uint32_t taken = 0, ties_taken = 0;
  for (uint32_t base = 0; base < nvec && taken < (uint32_t)K; base += kKT) {
    const uint32_t v = base + t;
    uint32_t key[8], raw[8];
    uint32_t n_gt = 0, n_eq = 0;
    if (v < nvec) {
      const uint4 q = trow[v];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        raw[h] = (w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
        key[h] = order_key(raw[h]);
        n_gt += key[h] > tau;
        n_eq += key[h] == tau;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 8; ++h) key[h] = raw[h] = 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((n_gt << 16) | n_eq, tot, sh);
    const uint32_t r = need_ties - ties_taken;              // ties still to take
    const uint32_t ex_eq = ex & 0xFFFFu;
    uint32_t pos = taken + (ex >> 16) + min(ex_eq, r);
    uint32_t tie_rank = ex_eq;
    if (v < nvec) {
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        bool take = key[h] > tau;
        if (key[h] == tau) {
          take = tie_rank < r;
          ++tie_rank;
        }
        if (take) {
          sh.idx[pos] = (int32_t)(8u * v + h);
          sh.tv[pos] = bf16_to_f32(raw[h]);
          ++pos;
        }
      }
    }
    const uint32_t took_ties = min(tot & 0xFFFFu, r);
    taken += (tot >> 16) + took_ties;
    ties_taken += took_ties;
  }
  __syncthreads();

  // the student's logits at the selected entries; both restricted softmaxes
  const uint16_t *srow = student + row * (size_t)V;
  float mt = -INFINITY, ms = -INFINITY;
  for (int i = t; i < K; i += kKT) {
    // (the clamp only guards the address; every index is in [0, V) by construction)
    const float zs = bf16_to_f32(srow[min(max(sh.idx[i], 0), V - 1)]);
    sh.sv[i] = zs;
    mt = fmaxf(mt, sh.tv[i]);
    ms = fmaxf(ms, zs);
  }
  mt = block_max(mt, sh);
  ms = block_max(ms, sh);
  float et = 0.0f, es = 0.0f;
  for (int i = t; i < K; i += kKT) {
    et += __expf(sh.tv[i] - mt);
    es += __expf(sh.sv[i] - ms);
  }
  et = block_sum(et, sh);
  es = block_sum(es, sh);
  const float lse_t = mt + __logf(et), lse_s = ms + __logf(es);
  float l = 0.0f;
  for (int i = t; i < K; i += kKT) {
    const float lt = sh.tv[i] - lse_t, ls = sh.sv[i] - lse_s;
    l += REVERSE ? __expf(ls) * (ls - lt) : __expf(lt) * (lt - ls);
  }
  const float loss = block_sum(l, sh);
  const bool ok = valid ? valid[row] != 0 : true;
  const float scale = ok ? inv_n[0] : 0.0f;
  for (int i = t; i < K; i += kKT) {
    const float lt = sh.tv[i] - lse_t, ls = sh.sv[i] - lse_s;
    const float ps = __expf(ls);
    const float g = REVERSE ? ps * ((ls - lt) - loss) : ps - __expf(lt);
    out_idx[row * (size_t)K + i] = sh.idx[i];
    out_grad[row * (size_t)K + i] = g * scale;
  }
  if (t == 0) loss_tok[row] = ok ? loss : 0.0f;
}

// loss_mean = (sum over tokens of loss_tok, fixed order) * inv_n
__global__ __launch_bounds__(1024) void k_kl_mean(const float *__restrict__ loss_tok, int T,
                                                  const float *__restrict__ inv_n,
                                                  float *__restrict__ loss_mean) {
  __shared__ float red[16];
  float s = 0.0f;
  for (int i = threadIdx.x; i < T; i += 1024) s += loss_tok[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = red[0];
    for (int w = 1; w < 16; ++w) tot += red[w];
    loss_mean[0] = tot * inv_n[0];
  }
}

}  // namespace

void launch_topk_kl(const uint16_t *student, const uint16_t *teacher, int T, int V, int K,
                    bool reverse, const uint8_t *valid, int32_t *idx, float *grad, float *loss_tok,
                    float *loss_mean, float *inv_n, hipStream_t st) {
  hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(256), 0, st, valid, T, inv_n);
  if (T > 0) {
    if (reverse)
      hipLaunchKernelGGL(k_topk_kl<true>, dim3(T), dim3(kKT), 0, st, student, teacher, V, K, valid,
                         inv_n, idx, grad, loss_tok);
    else
      hipLaunchKernelGGL(k_topk_kl<false>, dim3(T), dim3(kKT), 0, st, student, teacher, V, K,
                         valid, inv_n, idx, grad, loss_tok);
  }
  hipLaunchKernelGGL(k_kl_mean, dim3(1), dim3(1024), 0, st, loss_tok, T, inv_n, loss_mean);
}

}  // namespace fq
