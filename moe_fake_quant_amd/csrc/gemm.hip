// Grouped GEMM over routed rows on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation: all experts of a stack in one launch (AngelSlim mcore_qad
// article, section 二.4), forward and the scale-only backward (section 一).
//
// One kernel computes C[i][j] = sum_c P[i][c] * Q[j][c] on a 256 x 256 tile
// with a 64-deep contraction step; four waves, each 128 x 128 (4 x 4 MFMA
// 32x32 sub-tiles). Operands are staged global -> registers -> LDS (double
// buffered), LDS rows are 128 B with a 16-byte-slot XOR swizzle so that both
// the staging writes and the MFMA fragment reads are bank-conflict free.
//
//   mode   P (row operand, i)          Q (column operand, j)     contraction
//   FWD    W_fq[e] rows n   (K-contig) X rows r of segment e      k
//   DGRAD  W_fq[e] as [n][k] -> i = k  dY rows r (N-contig)       n
//          (transposed on the way into LDS)
//   WGRAD  X rows -> i = k (transposed) dY rows -> j = n (transp.) routed rows r
//
// A "transposed" operand is read as 8 contraction rows x 8 contiguous
// columns per lane (eight 16-byte loads) and turned into eight 8-long
// contraction vectors with v_perm_b32 before its LDS write.
//
// FWD / DGRAD store bf16 rows; WGRAD never stores dW: its epilogue
// multiplies each dWq element by the straight-through factor dv/ds
// (recomputed from the raw weight and its scale) and reduces over the
// quantization group (dScale), deterministically.
//
// Scheduling: FWD / DGRAD tiles are (expert, row tile, i tile); the number of
// row tiles of each expert comes from seg_offsets on the device (a block-wide
// scan in LDS), so empty experts cost nothing and no host sync is needed.
// Block ids are remapped so that consecutive tiles land on the same XCD (the
// hardware deals blocks round-robin over the 8 XCDs), keeping an expert's
// weights and rows in one XCD's L2.
#include "internal.hpp"

namespace fq {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8v;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int BI = 256;   // tile rows (i)
constexpr int BJ = 256;   // tile cols (j)
constexpr int BK = 64;    // contraction step
constexpr int NT = 512;   // threads per block (8 waves, 2 per SIMD)
constexpr int WJ_TILE = 64;  // j extent of one wave (waves: 2 along i x 4 along j)
constexpr int kTileBytes = 256 * BK * 2;  // one operand tile in LDS (32 KiB)

enum Mode { FWD = 0, DGRAD = 1, WGRAD = 2 };

// byte offset of 16-byte slot kc (0..7) of LDS row idx (0..255)
__device__ __forceinline__ uint32_t lds_off(uint32_t idx, uint32_t kc) {
  uint32_t swz = (idx ^ (idx >> 3)) & 7u;
  return idx * 128u + ((kc ^ swz) << 4);
}

__device__ __forceinline__ bf16x8_t ldg16(const char *base, uint32_t byte_off) {
  return *reinterpret_cast<const bf16x8_t *>(base + byte_off);
}

// ---- normal operand: 256 rows of a row-major matrix, 64 contiguous contraction
// elements each. Thread t: rows u*32 + t/8 (u = 0..7), 16-byte slot t%8.
// The per-thread row byte offsets are fixed for a tile; the contraction step
// adds c0*2 bytes. Offsets are 32-bit from a block-uniform base pointer.
struct NormalRows {
  uint32_t off[4];
  __device__ __forceinline__ void init(size_t ld, int row0, int row_last) {
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int r = min(row0 + u * 64 + (t >> 3), row_last);
      off[u] = (uint32_t)(((size_t)r * ld + (t & 7) * 8) * 2);
    }
  }
  __device__ __forceinline__ void load(bf16x8_t (&v)[4], const char *base, int c0) const {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ldg16(base, off[u] + c0 * 2);
  }
};
__device__ __forceinline__ void store_normal(char *lds, const bf16x8_t (&v)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    *reinterpret_cast<bf16x8_t *>(lds + lds_off(u * 64 + (t >> 3), t & 7)) = v[u];
}

// ---- transposed operand: element (c, idx) at base[c * ld + idx]; the tile is
// contraction rows c0..c0+63 x idx idx0..idx0+255. Thread t: idx block t%32
// (8 columns), contraction block t/32 (4 rows). Rows c >= c_end read as 0.
__device__ __forceinline__ void load_trans(bf16x8_t (&v)[4], const char *base, uint32_t ld, int c0,
                                           int c_end, int idx0) {
  const int t = threadIdx.x;
  const uint32_t col = idx0 + (t & 31) * 8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int c = c0 + (t >> 5) * 4 + q;
    bool ok = c < c_end;
    int cc = ok ? c : c0;  // c0 < c_end whenever this tile is loaded
    bf16x8_t x = ldg16(base, ((uint32_t)cc * ld + col) * 2);
    v[q].w[0] = ok ? x.w[0] : 0u;
    v[q].w[1] = ok ? x.w[1] : 0u;
    v[q].w[2] = ok ? x.w[2] : 0u;
    v[q].w[3] = ok ? x.w[3] : 0u;
  }
}
// 4 contraction rows x 8 columns -> 8 columns x 4 contraction values (8 bytes
// each, half of a 16-byte LDS slot)
__device__ __forceinline__ void store_trans(char *lds, const bf16x8_t (&v)[4]) {
  const int t = threadIdx.x;
  const uint32_t idxb = (t & 31) * 8, cb = t >> 5, kc = cb >> 1, half = (cb & 1) * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint2 lo, hi;  // columns 2p and 2p+1
    lo.x = __builtin_amdgcn_perm(v[1].w[p], v[0].w[p], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(v[3].w[p], v[2].w[p], 0x05040100u);
    hi.x = __builtin_amdgcn_perm(v[1].w[p], v[0].w[p], 0x07060302u);
    hi.y = __builtin_amdgcn_perm(v[3].w[p], v[2].w[p], 0x07060302u);
    *reinterpret_cast<uint2 *>(lds + lds_off(idxb + 2 * p, kc) + half) = lo;
    *reinterpret_cast<uint2 *>(lds + lds_off(idxb + 2 * p + 1, kc) + half) = hi;
  }
}

struct GemmArgs {
  const uint16_t *p;   // FWD/DGRAD: W_fq [E,N,K]; WGRAD: Xq [R_max, K]
  const uint16_t *q;   // FWD: Xq [R_max, K]; DGRAD/WGRAD: dY [R_max, N]
  const int32_t *seg;  // [E+1]
  int E, N, K;
  int n_it;            // i tiles
  int n_jt;            // WGRAD: j tiles
  // FWD/DGRAD output [R_max, ldo]
  uint16_t *out;
  // WGRAD epilogue
  const uint16_t *w;   // raw weights [E,N,K]
  int wfmt, group;
  const float *scale, *zero_point, *gscale;
  float *dscale, *dzp;     // final outputs (group <= 128), or NULL
  float *pscale, *pzp;     // partials per 128-chunk of K (group > 128), or NULL
};

// Expert and first row of this block's row tile: block-wide scan of per-expert
// row-tile counts (E <= 256 per pass, looped). Returns false when the block
// has no tile.
__device__ bool find_row_tile(const int32_t *seg, int E, int tile, int &e_out, int &row0,
                              int &row_end) {
  __shared__ int s_found[3];
  __shared__ int s_wsum[NT / 64];
  if (threadIdx.x == 0) s_found[0] = -1;
  __syncthreads();
  int base_tiles = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    int e = e0 + threadIdx.x;
    int lo = 0, hi = 0, nt = 0;
    if (e < E) {
      lo = seg[e];
      hi = seg[e + 1];
      nt = (hi - lo + BJ - 1) / BJ;
    }
    // inclusive scan of nt
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wsum[w] = x;
    __syncthreads();
    int before = base_tiles, total = base_tiles;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
      if (k < w) before += s_wsum[k];
      total += s_wsum[k];
    }
    int start = before + x - nt;
    if (e < E && tile >= start && tile < start + nt) {
      s_found[0] = e;
      s_found[1] = lo + (tile - start) * BJ;
      s_found[2] = hi;
    }
    __syncthreads();
    base_tiles = total;
  }
  e_out = s_found[0];
  row0 = s_found[1];
  row_end = s_found[2];
  return e_out >= 0;
}

// dS of the 128 (k) x 32 (n) slab of dWq that column sub-tile U (0..1) of one wave
// holds: lane n = n0 + lane%32, k = k0 + 32s + 8q + 4(lane/32) + v for
// acc[s][U][4q + v]. Each dWq element is weighted by its straight-through
// factor and summed over its quantization group in a fixed order.
template <int WFMT, int U>
__device__ __forceinline__ void wgrad_epilogue(const GemmArgs &a, const f32x16 (&acc)[4][2], int e,
                                               int k0, int n0, int lane) {
  const int n = n0 + (lane & 31);
  const int h = lane >> 5;
  const int G = a.K / a.group;
  const float g_e = (WFMT == FQ_FMT_NVFP4) ? a.gscale[e] : 1.0f;
  const uint16_t *wrow = a.w + ((size_t)e * a.N + n) * a.K;
  const size_t srow = ((size_t)e * a.N + n) * G;
  // this lane's raw weights of the slab: k = k0 + 32s + 8q + 4h + v
  uint2 wv[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wv[s][q] = *reinterpret_cast<const uint2 *>(wrow + k0 + s * 32 + 8 * q + 4 * h);
  float part_s[4], part_z[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float ps16[2], pz16[2];  // the sub-tile's two 16-blocks
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // every group is a multiple of 16 long: one scale per 16-block
      const int gi = (k0 + s * 32 + 16 * b) / a.group;
      float sc = a.scale[srow + gi];
      float zpi = 0.0f, fac = 1.0f;
      if (WFMT == FQ_FMT_INT4) zpi = fminf(fmaxf(rintf(a.zero_point[srow + gi]), 0.0f), 15.0f);
      if (WFMT == FQ_FMT_NVFP4) {
        fac = nvfp4_theta_factor(sc, g_e);
        sc = nvfp4_block_scale(sc, g_e);
      }
      const float r = safe_recip(sc);
      float accs = 0.0f, accz = 0.0f;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = 2 * b + qq;
        const float x4[4] = {lo_bf16(wv[s][q].x), hi_bf16(wv[s][q].x), lo_bf16(wv[s][q].y),
                             hi_bf16(wv[s][q].y)};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float dzp;
          const float phi = ste_factor<WFMT>(x4[v], sc, r, zpi, dzp);
          const float d = acc[s][U][4 * q + v];
          accs += d * phi;
          if (WFMT == FQ_FMT_INT4) accz += d * dzp;
        }
      }
      ps16[b] = (WFMT == FQ_FMT_NVFP4) ? accs * fac : accs;
      pz16[b] = accz;
    }
    // a 16-block is split between this lane (k%8 < 4 or >= 4) and lane ^ 32
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      ps16[b2] += __shfl_xor(ps16[b2], 32, 64);
      if (WFMT == FQ_FMT_INT4) pz16[b2] += __shfl_xor(pz16[b2], 32, 64);
    }
    if (a.group == 16 && lane < 32) {
      const int kb = (k0 + s * 32) / 16;
      a.dscale[srow + kb] = ps16[0];
      a.dscale[srow + kb + 1] = ps16[1];
      if (WFMT == FQ_FMT_INT4 && a.dzp) {
        a.dzp[srow + kb] = pz16[0];
        a.dzp[srow + kb + 1] = pz16[1];
      }
    }
    part_s[s] = ps16[0] + ps16[1];
    part_z[s] = pz16[0] + pz16[1];
  }
  if (lane < 32 && a.group != 16) {
    if (a.group == 32) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kb = (k0 + s * 32) / 32;
        a.dscale[srow + kb] = part_s[s];
        if (WFMT == FQ_FMT_INT4 && a.dzp) a.dzp[srow + kb] = part_z[s];
      }
    } else if (a.group == 64) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int kb = (k0 + h2 * 64) / 64;
        a.dscale[srow + kb] = part_s[2 * h2] + part_s[2 * h2 + 1];
        if (WFMT == FQ_FMT_INT4 && a.dzp) a.dzp[srow + kb] = part_z[2 * h2] + part_z[2 * h2 + 1];
      }
    } else {
      const float s128 = (part_s[0] + part_s[1]) + (part_s[2] + part_s[3]);
      const float z128 = (part_z[0] + part_z[1]) + (part_z[2] + part_z[3]);
      const int kb = k0 / 128;
      if (a.group == 128) {
        a.dscale[srow + kb] = s128;
        if (WFMT == FQ_FMT_INT4 && a.dzp) a.dzp[srow + kb] = z128;
      } else {
        const size_t prow = ((size_t)e * a.N + n) * (a.K / 128);
        a.pscale[prow + kb] = s128;
        if (WFMT == FQ_FMT_INT4 && a.pzp) a.pzp[prow + kb] = z128;
      }
    }
  }
}

template <int MODE, int WFMT>
__global__ __launch_bounds__(NT) void k_grouped_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];  // P0 Q0 P1 Q1 = 128 KiB
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wi = wave & 1, wj = wave >> 1;  // 2 x 4 waves: 128 (i) x 64 (j) each

  // XCD-aware remap of the block id
  const uint32_t nb = gridDim.x, b = blockIdx.x;
  const uint32_t wid = (b & 7u) * (nb >> 3) + (b >> 3);

  int e, it, j0 = 0, j_end = 0, i0;
  int c_total;  // contraction length
  if (MODE == WGRAD) {
    const int per_e = a.n_it * a.n_jt;
    e = wid / per_e;
    if (e >= a.E) return;
    int rem = wid - e * per_e;
    int jt = rem / a.n_it;
    it = rem - jt * a.n_it;
    j0 = jt * BJ;
    i0 = it * BI;
  } else {
    int tile = wid / a.n_it;
    it = wid - tile * a.n_it;
    i0 = it * BI;
    if (!find_row_tile(a.seg, a.E, tile, e, j0, j_end)) return;
  }
  const int seg_lo = a.seg[e], seg_hi = a.seg[e + 1];
  if (MODE == WGRAD) c_total = seg_hi - seg_lo;
  else c_total = (MODE == FWD) ? a.K : a.N;

  // operand base pointers (block-uniform) and leading dimensions
  const size_t NK = (size_t)a.N * a.K;
  const char *pbase, *qbase;
  if (MODE == FWD) {
    pbase = reinterpret_cast<const char *>(a.p + e * NK);   // W_fq[e] [N][K], rows i = n
    qbase = reinterpret_cast<const char *>(a.q);            // Xq rows (absolute)
  } else if (MODE == DGRAD) {
    pbase = reinterpret_cast<const char *>(a.p + e * NK);   // W_fq[e] as (c = n, idx = k)
    qbase = reinterpret_cast<const char *>(a.q);            // dY rows (absolute)
  } else {
    pbase = reinterpret_cast<const char *>(a.p + (size_t)seg_lo * a.K);  // Xq: (c = r, idx = k)
    qbase = reinterpret_cast<const char *>(a.q + (size_t)seg_lo * a.N);  // dY: (c = r, idx = n)
  }
  NormalRows prow, qrow;
  if (MODE == FWD) prow.init(a.K, i0, a.N - 1);
  if (MODE == FWD) qrow.init(a.K, j0, j_end - 1);
  if (MODE == DGRAD) qrow.init(a.N, j0, j_end - 1);

  f32x16 acc[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[s][u][v] = 0.0f;

  const int nk = (c_total + BK - 1) / BK;
  bf16x8_t rp[4], rq[4];

  auto load_tile = [&](int kt) {
    const int c0 = kt * BK;
    if (MODE == FWD) {
      prow.load(rp, pbase, c0);
      qrow.load(rq, qbase, c0);
    } else if (MODE == DGRAD) {
      load_trans(rp, pbase, a.K, c0, c_total, i0);
      qrow.load(rq, qbase, c0);
    } else {
      load_trans(rp, pbase, a.K, c0, c_total, i0);
      load_trans(rq, qbase, a.N, c0, c_total, j0);
    }
  };
  auto store_tile = [&](int buf) {
    char *sp = smem + (2 * buf) * kTileBytes;
    char *sq = smem + (2 * buf + 1) * kTileBytes;
    if (MODE == FWD) {
      store_normal(sp, rp);
      store_normal(sq, rq);
    } else if (MODE == DGRAD) {
      store_trans(sp, rp);
      store_normal(sq, rq);
    } else {
      store_trans(sp, rp);
      store_trans(sq, rq);
    }
  };
  // MFMA fragments of one 16-deep step: [0..3] P sub-tiles, [4..5] Q sub-tiles
  auto read_frags = [&](int buf, int ks, bf16x8v (&f)[6]) {
    const char *sp = smem + (2 * buf) * kTileBytes;
    const char *sq = smem + (2 * buf + 1) * kTileBytes;
    const uint32_t kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      f[s] = *reinterpret_cast<const bf16x8v *>(sp + lds_off(wi * 128 + s * 32 + (lane & 31), kc));
#pragma unroll
    for (int u = 0; u < 2; ++u)
      f[4 + u] = *reinterpret_cast<const bf16x8v *>(sq + lds_off(wj * WJ_TILE + u * 32 + (lane & 31), kc));
  };

  // Pipeline: global loads of tile kt+1 are in flight during the MFMAs of
  // tile kt; the fragments of step ks+1 are read from LDS during the MFMAs
  // of step ks.
  bf16x8v fr[2][6];
  if (nk > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    read_frags(0, 0, fr[0]);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_tile(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) read_frags(cur, ks + 1, fr[(ks + 1) & 1]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[s][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks & 1][s], fr[ks & 1][4 + u],
                                                              acc[s][u], 0, 0, 0);
    }
    if (more) store_tile(cur ^ 1);
    __syncthreads();
    if (more) read_frags(cur ^ 1, 0, fr[0]);
  }

  // accumulator (s, u, v) of this lane: i = i0 + wi*128 + s*32 + 8*(v/4) + 4*(lane/32) + v%4,
  //                                     j = j0 + wj*64 + u*32 + lane%32
  if (MODE != WGRAD) {
    const int ldo = (MODE == FWD) ? a.N : a.K;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = j0 + wj * WJ_TILE + u * 32 + (lane & 31);
      if (j >= j_end) continue;
      uint16_t *orow = a.out + (size_t)j * ldo;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = i0 + wi * 128 + s * 32 + 8 * q + 4 * (lane >> 5);
          uint2 pk;
          pk.x = pack_bf16(acc[s][u][4 * q + 0], acc[s][u][4 * q + 1]);
          pk.y = pack_bf16(acc[s][u][4 * q + 2], acc[s][u][4 * q + 3]);
          *reinterpret_cast<uint2 *>(orow + i) = pk;
        }
    }
    return;
  }

  // ---- WGRAD epilogue: i = k, j = n of expert e. dS over groups along k.
  {
    const int k0 = i0 + wi * 128, n0 = j0 + wj * WJ_TILE;
    wgrad_epilogue<WFMT, 0>(a, acc, e, k0, n0, lane);
    wgrad_epilogue<WFMT, 1>(a, acc, e, k0, n0 + 32, lane);
  }
}

}  // namespace

// ============================================================ launchers ====
static int round8(long x) { return (int)((x + 7) / 8 * 8); }

void launch_gemm_fwd(const uint16_t *xq, int R_max, const int32_t *seg, fq_shape s,
                     const uint16_t *wfq, uint16_t *y, hipStream_t st) {
  GemmArgs a{};
  a.p = wfq;
  a.q = xq;
  a.seg = seg;
  a.E = s.E;
  a.N = s.N;
  a.K = s.K;
  a.n_it = s.N / BI;
  a.out = y;
  long tiles = (long)(R_max / BJ + s.E) * a.n_it;
  if (tiles <= 0 || R_max <= 0) return;
  hipLaunchKernelGGL((k_grouped_gemm<FWD, 0>), dim3(round8(tiles)), dim3(NT), 0, st, a);
}

void launch_gemm_dgrad(const uint16_t *dy, int R_max, const int32_t *seg, fq_shape s,
                       const uint16_t *wfq, uint16_t *dx, hipStream_t st) {
  GemmArgs a{};
  a.p = wfq;
  a.q = dy;
  a.seg = seg;
  a.E = s.E;
  a.N = s.N;
  a.K = s.K;
  a.n_it = s.K / BI;
  a.out = dx;
  long tiles = (long)(R_max / BJ + s.E) * a.n_it;
  if (tiles <= 0 || R_max <= 0) return;
  hipLaunchKernelGGL((k_grouped_gemm<DGRAD, 0>), dim3(round8(tiles)), dim3(NT), 0, st, a);
}

void launch_gemm_wgrad_dscale(const uint16_t *dy, const uint16_t *xq, const int32_t *seg, fq_shape s,
                              const uint16_t *w, const fq_weight_q &q, float *dscale, float *dzp,
                              float *pscale, float *pzp, hipStream_t st) {
  GemmArgs a{};
  a.p = xq;
  a.q = dy;
  a.seg = seg;
  a.E = s.E;
  a.N = s.N;
  a.K = s.K;
  a.n_it = s.K / BI;
  a.n_jt = s.N / BJ;
  a.w = w;
  a.wfmt = q.fmt;
  a.group = q.group;
  a.scale = q.scale;
  a.zero_point = q.zero_point;
  a.gscale = q.global_scale;
  a.dscale = dscale;
  a.dzp = dzp;
  a.pscale = pscale;
  a.pzp = pzp;
  long tiles = (long)s.E * a.n_it * a.n_jt;
  dim3 grid(round8(tiles)), block(NT);
  switch (q.fmt) {
    case FQ_FMT_INT8: hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_INT8>), grid, block, 0, st, a); break;
    case FQ_FMT_INT4: hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_INT4>), grid, block, 0, st, a); break;
    case FQ_FMT_FP8_E4M3:
      hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_FP8_E4M3>), grid, block, 0, st, a);
      break;
    default: hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_NVFP4>), grid, block, 0, st, a); break;
  }
}

}  // namespace fq
