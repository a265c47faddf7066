// Top-K KL distillation on gfx950: the loss between the student's and the
// (quantization-off) teacher's logits over the teacher's K most likely tokens
// per position, and its gradient on the student logits, without forming the
// [tokens, vocab] probabilities (AngelSlim mcore_qad article, section 二.5;
// the forward / reverse top-K variants of the QAT + ZeRO-3 page's loss table).
//
// One workgroup per token row; the teacher row is streamed once. A sample
// spread over the row bounds the K-th largest logit from below; the stream keeps the
// (few) entries above that bound, in vocabulary order, and the exact K-th
// largest, the ties (lower index first) and the selection come from them
// (k_topk_kl). Rows where the bound fails are selected exactly by histograms
// over an order-preserving 16-bit key of the bf16 logits (select_hist). The
// student logits are gathered at the K selected indices; both restricted
// softmaxes, the loss and the gradient come from LDS.
#include <type_traits>

#include "internal.hpp"

namespace fq {

namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int kKT = 512;           // threads per row
constexpr int kKW = kKT / 64;      // waves per row

// Reduction scratch.
struct KLShared {
  uint32_t scan[kKW];
  uint32_t cnt[2][kKW];
  float red2[2][kKW][2];
};
// The selected entries of a row (K <= KM).
template <int KM>
struct KLSel {
  int32_t idx[KM];
  float tv[KM];
  float sv[KM];
};
// Histograms of the histogram selection.
struct KLHist {
  uint32_t hist[kKW][256];         // per-wave histograms
  uint32_t sel_bin, sel_above;
};
constexpr int kCandMax = 8192;     // candidates of the sampled selection
constexpr int kWaveCand = kCandMax / kKW;   // one part per wave
constexpr int kHistBins = 4096;    // key-value counters of the threshold search
// The big LDS arrays share one region: candidates (or histograms) while the
// row is selected, then the selected entries. Sized for K <= KM: the smaller
// instance (K <= 1024) leaves room for four rows' workgroups per CU.
template <int KM>
union KLBig {
  uint32_t cand[kCandMax];             // vocabulary indices
  KLHist hs;
  KLSel<KM> sel;
};

// bf16 bits -> 16-bit key whose unsigned order is the value order (-0 and +0
// get one key: they are equal logits)
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// inverse of order_key (key 0x8000 -> +0)
__device__ __forceinline__ uint32_t raw_of_key(uint32_t k) {
  return (k & 0x8000u) ? (k ^ 0x8000u) : (~k & 0xFFFFu);
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
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total, KLShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == 63) sh.scan[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t x = sh.scan[w];
    before += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();  // scan[] is reused by the next call
  total = tot;
  return before + incl - v;
}

// Two block reductions (max if MAX, else sum) at once, in a fixed order, with
// one barrier (alternating scratch rows, `par` flips).
template <int NT, bool MAX>
__device__ __forceinline__ void block_reduce2(float &a, float &b, KLShared &sh, int &par) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float x = __shfl_xor(a, o, 64), y = __shfl_xor(b, o, 64);
    a = MAX ? fmaxf(a, x) : a + x;
    b = MAX ? fmaxf(b, y) : b + y;
  }
  if ((threadIdx.x & 63) == 0) {
    sh.red2[par][threadIdx.x >> 6][0] = a;
    sh.red2[par][threadIdx.x >> 6][1] = b;
  }
  __syncthreads();
  a = sh.red2[par][0][0];
  b = sh.red2[par][0][1];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    a = MAX ? fmaxf(a, sh.red2[par][w][0]) : a + sh.red2[par][w][0];
    b = MAX ? fmaxf(b, sh.red2[par][w][1]) : b + sh.red2[par][w][1];
  }
  par ^= 1;
}

__device__ __forceinline__ void zero_hist(KLHist &sh) {
  uint32_t *h = &sh.hist[0][0];
  for (int i = threadIdx.x; i < kKW * 256; i += kKT) h[i] = 0u;
  __syncthreads();
}

// Sum the per-wave histograms into hist[0], then find the bin b (scanning
// from 255 down) with above(b) < need <= above(b) + count(b), where above(b)
// counts the entries of the higher bins. Requires need <= total.
__device__ __forceinline__ void find_bin(KLHist &sh, uint32_t need) {
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

// The K selected entries (se.idx, se.tv) of one row -> the student's logits
// there, both restricted softmaxes, the loss and the scaled gradient.
template <int NT, bool REVERSE, int KM>
__device__ __forceinline__ void kl_tail(KLShared &sh, KLSel<KM> &se,
                                        const uint16_t *__restrict__ student,
                                        size_t row, int V, int K,
                                        const uint8_t *__restrict__ valid,
                                        const float *__restrict__ inv_n,
                                        int32_t *__restrict__ out_idx,
                                        float *__restrict__ out_grad,
                                        float *__restrict__ loss_tok) {
  const int t = threadIdx.x;
  // the student's logits at the selected entries; both restricted softmaxes
  const uint16_t *srow = student + row * (size_t)V;
  float mt = -INFINITY, ms = -INFINITY;
  for (int i = t; i < K; i += NT) {
    // (the clamp only guards the address; every index is in [0, V) by construction)
    const float zs = bf16_to_f32(srow[min(max(se.idx[i], 0), V - 1)]);
    se.sv[i] = zs;
    mt = fmaxf(mt, se.tv[i]);
    ms = fmaxf(ms, zs);
  }
  int par = 0;
  block_reduce2<NT, true>(mt, ms, sh, par);
  float et = 0.0f, es = 0.0f;
  for (int i = t; i < K; i += NT) {
    et += __expf(se.tv[i] - mt);
    es += __expf(se.sv[i] - ms);
  }
  block_reduce2<NT, false>(et, es, sh, par);
  const float lse_t = mt + __logf(et), lse_s = ms + __logf(es);
  float l = 0.0f, unused = 0.0f;
  for (int i = t; i < K; i += NT) {
    const float lt = se.tv[i] - lse_t, ls = se.sv[i] - lse_s;
    l += REVERSE ? __expf(ls) * (ls - lt) : __expf(lt) * (lt - ls);
  }
  block_reduce2<NT, false>(l, unused, sh, par);
  const float loss = l;
  const bool ok = valid ? valid[row] != 0 : true;
  const float scale = ok ? inv_n[0] : 0.0f;
  for (int i = t; i < K; i += NT) {
    const float lt = se.tv[i] - lse_t, ls = se.sv[i] - lse_s;
    const float ps = __expf(ls);
    const float g = REVERSE ? ps * ((ls - lt) - loss) : ps - __expf(lt);
    out_idx[row * (size_t)K + i] = se.idx[i];
    out_grad[row * (size_t)K + i] = g * scale;
  }
  if (t == 0) loss_tok[row] = ok ? loss : 0.0f;
}


// Exact selection by histograms: two 256-bin passes over the key's high and
// low byte find the K-th largest key; a third pass compacts the selection in
// vocabulary order (per-chunk block scans) and stops once K are in. Reads the
// row three times; used when the sampled bracket does not hold.
template <int KM>
__device__ __forceinline__ void select_hist(KLShared &sh, KLBig<KM> &big,
                                            const uint4 *__restrict__ trow, uint32_t nvec, int K) {
  KLHist &hs = big.hs;
  KLSel<KM> &se = big.sel;   // written only after the histograms are done with
  const int t = threadIdx.x, wave = t >> 6;
  // pass 1: histogram of the key's high byte
  zero_hist(hs);
  for (uint32_t v = t; v < nvec; v += kKT) {
    const uint4 q = trow[v];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t key = order_key((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
      atomicAdd(&hs.hist[wave][key >> 8], 1u);
    }
  }
  __syncthreads();
  find_bin(hs, (uint32_t)K);
  const uint32_t hi = hs.sel_bin, above_hi = hs.sel_above;

  // pass 2: histogram of the low byte inside the chosen high byte
  zero_hist(hs);
  for (uint32_t v = t; v < nvec; v += kKT) {
    const uint4 q = trow[v];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t key = order_key((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
      if ((key >> 8) == hi) atomicAdd(&hs.hist[wave][key & 0xFFu], 1u);
    }
  }
  __syncthreads();
  find_bin(hs, (uint32_t)K - above_hi);
  const uint32_t tau = (hi << 8) | hs.sel_bin;            // key of the K-th largest
  const uint32_t need_ties = (uint32_t)K - above_hi - hs.sel_above;

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
    const uint32_t ex = block_excl_scan<kKT>((n_gt << 16) | n_eq, tot, sh);
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
          se.idx[pos] = (int32_t)(8u * v + h);
          se.tv[pos] = bf16_to_f32(raw[h]);
          ++pos;
        }
      }
    }
    const uint32_t took_ties = min(tot & 0xFFFFu, r);
    taken += (tot >> 16) + took_ties;
    ties_taken += took_ties;
  }
  __syncthreads();

}

// Inclusive prefix sum over the 64 lanes on DPP moves (rows of 16 lanes
// shifted 1, 2, 4, 8, then the row broadcasts of lanes 15 and 31). Every lane
// must be active.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Block total of per-lane booleans, counted with ballots (one barrier;
// alternating scratch rows).
__device__ __forceinline__ uint32_t wave_count(bool f) {
  return (uint32_t)__popcll(__ballot(f));
}

// One token row per workgroup, the row streamed once. A sample spread over
// the row (one 8-logit vector per thread) gives a key L a little below the
// sample's share of the top K. The stream appends the vocabulary index of
// every entry with key >= L to an LDS list in vocabulary order (a block-wide
// prefix sum per step of 4 vectors per thread). When the list holds at least
// K entries and fits (the usual case) it alone decides the exact K-th largest
// key, the ties (lower index first) and the ordered selection. Otherwise the
// row is selected again by histograms (select_hist). Exact either way.
template <bool REVERSE, int KM>
__global__ __launch_bounds__(kKT) __attribute__((amdgpu_waves_per_eu(KM <= 1024 ? 8 : 6))) void k_topk_kl(const uint16_t *__restrict__ student,
                                                 const uint16_t *__restrict__ teacher, int V,
                                                 int K, const uint8_t *__restrict__ valid,
                                                 const float *__restrict__ inv_n,
                                                 int32_t *__restrict__ out_idx,
                                                 float *__restrict__ out_grad,
                                                 float *__restrict__ loss_tok) {
  __shared__ KLShared sh;
  __shared__ KLBig<KM> xs;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const size_t row = blockIdx.x;
  const uint4 *trow = reinterpret_cast<const uint4 *>(teacher + row * (size_t)V);
  const uint32_t nvec = (uint32_t)V / 8u;
  int par = 0;
  // block total of a per-thread count (wave sums on DPP, one barrier)
  auto bsum = [&](uint32_t c) {
    c = __builtin_amdgcn_readlane(wave_scan_dpp(c), 63);
    if (lane == 0) sh.cnt[par][wave] = c;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kKW; ++w) s += sh.cnt[par][w];
    par ^= 1;
    return s;
  };

  // sample: one vector per thread. KM <= 1024: the eight threads of a group
  // read one whole 128-byte line (8 consecutive vectors), the 64 lines spread
  // over the row (a line starts at a multiple of 8 vectors, at most nvec -
  // nvec / 64 <= nvec - 8 when nvec >= 512, so the group stays in the row);
  // 4-5 % faster at K = 1000 than one scattered vector per thread. The larger
  // selection (three rows per CU instead of four) keeps the scattered
  // vectors (the line sample measured 6 % slower there): their lines are
  // already cached when the stream reaches them.
  const uint32_t vs =
      nvec < (uint32_t)kKT ? (uint32_t)t
      : KM <= 1024
          ? ((uint32_t)(((unsigned long long)(t >> 3) * nvec) / (kKT / 8)) & ~7u) + (uint32_t)(t & 7)
          : (uint32_t)(((unsigned long long)t * nvec) / kKT);
  const bool has_s = vs < nvec;
  uint32_t sk[8];
  {
    const uint4 q = trow[min(vs, nvec - 1u)];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int h = 0; h < 8; ++h)
      sk[h] = has_s ? order_key((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu) : 0u;
  }
  const uint32_t n_smp = bsum(has_s ? 8u : 0u);
  // k' = the sample's expected share mu of the top K plus six standard
  // deviations and 4 (so count(key >= L) >= K all but never fails, and the
  // list stays near K + 6 sqrt(K V / n_smp)); at most n_smp, and the sample
  // holds n_smp >= 8 keys >= 1, so lo = 1 satisfies count >= k'
  const float mu = (float)K * (float)n_smp / (float)V;
  const uint32_t kq = min(n_smp, (uint32_t)ceilf(mu + 6.0f * sqrtf(mu) + 4.0f));
  uint32_t lo = 1, hi = 65536;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    uint32_t c = 0;
#pragma unroll
    for (int h = 0; h < 8; ++h) c += wave_count(sk[h] >= mid);
    if (lane == 0) sh.cnt[par][wave] = c;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kKW; ++w) tot += sh.cnt[par][w];
    par ^= 1;
    if (tot >= kq) lo = mid;
    else hi = mid;
  }
  const uint32_t L = lo;

  // the stream: wave w owns the contiguous vectors [w * nv_w, (w + 1) * nv_w)
  // and appends the indices of its entries with key >= L, in vocabulary
  // order, to its own part of the list (wave-level prefix sums only)
  const uint32_t nv_w = (nvec + kKW - 1) / kKW;
  const uint32_t wv0 = min(nvec, (uint32_t)wave * nv_w), wv1 = min(nvec, wv0 + nv_w);
  uint32_t wn = 0;                                           // this wave's count (wave-uniform)
  uint32_t *wl = xs.cand + wave * kWaveCand;
  // A bound above +0 (the usual case: the top of a logit row) is tested on
  // the raw bits: for such a bound, key >= L holds exactly when the bf16
  // pattern, read as a signed 16-bit integer, is >= the bound's pattern b
  // (negative values and -0 read as negative integers). Per 32-bit word, one
  // packed saturating subtract (b - 1) - x gives both halves' answers in
  // their sign bits; v_perm's sign-replicating selectors gather the eight
  // signs of a vector into bytes in element order, and two byte dot
  // products with one bit per byte pack them into the 8-bit flag mask.
  // list entries: the vocabulary index, or (when every wave's stretch of the
  // row has at most 65536 entries) the index within the stretch << 16 | key,
  // so that the keys need not be read again
  const bool packed = nv_w * 8u <= 65536u;
  const bool pos_bound = L > 0x8000u;
  const uint32_t bm1 = (raw_of_key(L) - 1u) & 0xFFFFu;
  const s16x2 bm1x2 = __builtin_bit_cast(s16x2, bm1 | (bm1 << 16));
  for (uint32_t v0 = wv0; v0 < wv1; v0 += 4u * 64u) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = trow[min(v0 + (uint32_t)u * 64u + lane, wv1 - 1u)];
    uint32_t f[4] = {0u, 0u, 0u, 0u};
    if (pos_bound) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = v0 + (uint32_t)u * 64u + lane < wv1;
        const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          d[p] = __builtin_bit_cast(
              uint32_t, __builtin_elementwise_sub_sat(bm1x2, __builtin_bit_cast(s16x2, w[p])));
        const uint32_t lo = __builtin_amdgcn_perm(d[1], d[0], 0x0B0A0908u) & 0x08040201u;
        const uint32_t hi = __builtin_amdgcn_perm(d[3], d[2], 0x0B0A0908u) & 0x80402010u;
        const uint32_t fu =
            __builtin_amdgcn_udot4(hi, 0x01010101u, __builtin_amdgcn_udot4(lo, 0x01010101u, 0u, false), false);
        f[u] = in ? fu : 0u;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool in = v0 + (uint32_t)u * 64u + lane < wv1;
        const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t k = order_key((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
          f[u] |= (uint32_t)(in && k >= L) << h;
        }
      }
    }
    // counts of the 4 steps, two 16-bit fields per word (at most 8 * 64 each)
    const uint32_t c01 = __popc(f[0]) | (__popc(f[1]) << 16);
    const uint32_t c23 = __popc(f[2]) | (__popc(f[3]) << 16);
    const uint32_t i01 = wave_scan_dpp(c01), i23 = wave_scan_dpp(c23);
    const uint32_t t01 = __builtin_amdgcn_readlane(i01, 63);
    const uint32_t t23 = __builtin_amdgcn_readlane(i23, 63);
    const uint32_t e01 = i01 - c01, e23 = i23 - c23;
    const uint32_t tot0 = t01 & 0xFFFFu, tot1 = t01 >> 16, tot2 = t23 & 0xFFFFu;
    const uint32_t pos0[4] = {wn + (e01 & 0xFFFFu), wn + tot0 + (e01 >> 16),
                              wn + tot0 + tot1 + (e23 & 0xFFFFu),
                              wn + tot0 + tot1 + tot2 + (e23 >> 16)};
    wn += tot0 + tot1 + tot2 + (t23 >> 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t m = f[u], p = pos0[u];
      const uint32_t vb = 8u * (v0 + (uint32_t)u * 64u + lane);
      while (m) {
        const uint32_t h = __builtin_ctz(m);
        m &= m - 1u;
        uint32_t e = vb + h;
        if (packed) {
          const uint32_t word = h < 4 ? (h < 2 ? q[u].x : q[u].y) : (h < 6 ? q[u].z : q[u].w);
          e = ((e - 8u * wv0) << 16) | order_key((word >> (16u * (h & 1u))) & 0xFFFFu);
        }
        if (p < (uint32_t)kWaveCand) wl[p] = e;
        ++p;
      }
    }
  }
  if (lane == 0) sh.cnt[par][wave] = wn;
  __syncthreads();
  uint32_t wbase[kKW + 1];
  wbase[0] = 0;
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < kKW; ++w) {
    const uint32_t c = sh.cnt[par][w];
    wbase[w + 1] = wbase[w] + c;
    overflow |= c > (uint32_t)kWaveCand;
  }
  par ^= 1;
  const uint32_t n = wbase[kKW];
  // list entry i lives at wave w's part, offset i - wbase[w]: its vocabulary
  // index and, for packed entries, its key (else 0)
  auto list_at = [&](uint32_t i, uint32_t &key) {
    uint32_t w = 0;
#pragma unroll
    for (int x = 1; x < kKW; ++x) w += i >= wbase[x];
    const uint32_t e = xs.cand[w * kWaveCand + (i - wbase[w])];
    if (!packed) {
      key = 0u;
      return e;
    }
    key = e & 0xFFFFu;
    return 8u * min(nvec, w * nv_w) + (e >> 16);
  };

  // the sampled selection with kPer list entries per thread (8 when the list
  // fits, else 16)
  auto fast = [&](auto kper_tag) {
    constexpr int kPer = decltype(kper_tag)::value;
    // this thread's contiguous slice of the list and its keys (packed in the
    // list, else re-read from the teacher row: a few entries per thread)
    const uint32_t per = (n + kKT - 1) / kKT;
    const uint32_t c0 = min(n, (uint32_t)t * per), c1 = min(n, c0 + per);
    const uint16_t *trow16 = teacher + row * (size_t)V;
    uint32_t ci[kPer], ck[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) ci[u] = (c0 + u < c1) ? list_at(c0 + u, ck[u]) : 0u;
    if (!packed) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) ck[u] = trow16[ci[u]];
#pragma unroll
      for (int u = 0; u < kPer; ++u) ck[u] = order_key(ck[u]);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) ck[u] = (c0 + u < c1) ? ck[u] : 0u;
    // the K-th largest key among the list (every key >= it is listed: the
    // list holds all keys >= L, at least K of them): a count per key value
    // from L up (the list is in registers now, its memory is free)
    uint32_t kmax = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) kmax = max(kmax, ck[u]);
    for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    if (lane == 0) sh.cnt[par][wave] = kmax;
    __syncthreads();
    kmax = 0;
#pragma unroll
    for (int w = 0; w < kKW; ++w) kmax = max(kmax, sh.cnt[par][w]);
    par ^= 1;
    uint32_t tau;
    if (kmax - L < (uint32_t)kHistBins) {
      uint32_t *hb = xs.cand;                                // kHistBins counters
      for (int i = t; i < kHistBins; i += kKT) hb[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (ck[u] >= L) atomicAdd(&hb[ck[u] - L], 1u);
      __syncthreads();
      // thread t sums bins from the top: its kHistBins / kKT bins, highest first
      constexpr int kB = kHistBins / kKT;
      const uint32_t top = kHistBins - 1 - t * kB;           // this thread's highest bin
      uint32_t bc[kB], sum = 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        bc[j] = hb[top - j];
        sum += bc[j];
      }
      uint32_t total;
      uint32_t acc = block_excl_scan<kKT>(sum, total, sh);    // entries in higher bins
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (acc < (uint32_t)K && acc + bc[j] >= (uint32_t)K) sh.cnt[par][0] = L + top - j;
        acc += bc[j];
      }
      __syncthreads();
      tau = sh.cnt[par][0];
      par ^= 1;
    } else {
      uint32_t lo2 = L, hi2 = 65536;
      while (hi2 - lo2 > 1) {
        const uint32_t mid = (lo2 + hi2) >> 1;
        uint32_t c = 0;
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if ((uint32_t)u < per) c += wave_count(ck[u] >= mid);   // (block-uniform test)
        if (lane == 0) sh.cnt[par][wave] = c;
        __syncthreads();
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < kKW; ++w) tot += sh.cnt[par][w];
        par ^= 1;
        if (tot >= (uint32_t)K) lo2 = mid;
        else hi2 = mid;
      }
      tau = lo2;
    }
    // ordered selection: keys above tau, then the first ties
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      n_gt += ck[u] > tau;
      n_eq += ck[u] == tau;     // (keys past the slice are 0, never equal to tau >= 1)
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kKT>((n_gt << 16) | n_eq, tot, sh);
    const uint32_t need_ties = (uint32_t)K - (tot >> 16);
    uint32_t p = (ex >> 16) + min(ex & 0xFFFFu, need_ties);
    uint32_t tie_rank = ex & 0xFFFFu;
    uint32_t npick = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      bool take = ck[u] > tau;
      if (ck[u] == tau) {
        take = tie_rank < need_ties;
        ++tie_rank;
      }
      npick |= (uint32_t)take << u;
    }
    __syncthreads();   // the selected entries overwrite the list's memory
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if ((npick >> u) & 1u) {
        xs.sel.idx[p] = (int32_t)ci[u];
        xs.sel.tv[p] = bf16_to_f32(raw_of_key(ck[u]));
        ++p;
      }
  };
  if (n >= (uint32_t)K && !overflow && n <= (uint32_t)kCandMax) {
    if (n <= 8u * kKT) fast(std::integral_constant<int, 8>{});
    else fast(std::integral_constant<int, kCandMax / kKT>{});
  } else {
    select_hist(sh, xs, trow, nvec, K);
  }
  __syncthreads();
  kl_tail<kKT, REVERSE, KM>(sh, xs.sel, student, row, V, K, valid, inv_n, out_idx, out_grad,
                        loss_tok);
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
    auto k = reverse ? (K <= 1024 ? k_topk_kl<true, 1024> : k_topk_kl<true, kTopKMax>)
                     : (K <= 1024 ? k_topk_kl<false, 1024> : k_topk_kl<false, kTopKMax>);
    hipLaunchKernelGGL(k, dim3(T), dim3(kKT), 0, st, student, teacher, V, K, valid, inv_n, idx,
                       grad, loss_tok);
  }
  hipLaunchKernelGGL(k_kl_mean, dim3(1), dim3(1024), 0, st, loss_tok, T, inv_n, loss_mean);
}

}  // namespace fq
