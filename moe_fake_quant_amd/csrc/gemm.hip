// Grouped GEMM over routed rows on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation: all experts of a stack in one launch (AngelSlim mcore_qad
// article, section 二.4), forward and the scale-only backward (section 一).
//
// One kernel computes C[i][j] = sum_c P[i][c] * Q[j][c] on a 256 x 256 tile.
// Eight waves (two per SIMD), each 128 (i) x 64 (j) = 4 x 2 MFMA 32x32 tiles.
//
//   mode   P (row operand, i)            Q (column operand, j)        contraction
//   FWD    W_fq[e] rows n (K-contig)     X rows r of segment e         k
//   DGRAD  W_fq[e] [n][k]: i = k         dY rows r (N-contig)          n
//   WGRAD  X rows: i = k                 dY rows: j = n                routed rows r
//
// X can also be token-ordered (ROUTED): routed row r is then read from token
// row perm[r] / topk, in the load addresses, so no gathered copy is needed.
//
// Operands stream from global memory straight into LDS (global_load_lds,
// 16 bytes per lane, no staging registers) through a ring of two stages of
// 64 contraction elements: WGRAD loads one stage ahead with one barrier per
// stage, FWD / DGRAD two stages ahead in the ping-pong schedule described at
// run_tile. (Measured against four 32-deep stages: full 128-byte row
// segments per load and fewer barriers gain more than the deeper lookahead.) A
// contraction-contiguous operand is stored as 256 rows x 128 B and read with
// ds_read_b128; a transposed operand (contraction is its row) keeps its
// natural layout, 64 rows x 512 B, and the MFMA fragments are gathered
// with ds_read_tr16_b64 (a 4 x 16 -> 16 x 4 transpose inside each 16-lane
// group). Both layouts XOR-swizzle 16-byte chunks so the fragment reads are
// bank-conflict free.
//
// FWD / DGRAD store bf16 rows; WGRAD never stores dW: its epilogue
// multiplies each dWq element by the straight-through factor dv/ds
// (recomputed from the raw weight and its scale) and reduces over the
// quantization group (dScale), deterministically. Both epilogues move whole
// rows through the free stage buffer (the output tile out of it, the raw
// weights into it): partial-line global accesses cost far more than the LDS
// round trip.
//
// Scheduling: a persistent grid of one block per CU walks the tile list.
// FWD / DGRAD tiles are (expert, row tile, i tile); the number of row tiles of
// each expert comes from seg_offsets on the device (a block-wide scan in
// LDS), so empty experts cost nothing and no host sync is needed. Each of the
// 8 XCDs owns a contiguous eighth of the tiles, keeping the panels its blocks
// share in its own L2. A FWD / DGRAD call too small to fill the CUs runs each
// tile's contraction as several parts (the SPLIT kernels), whose fp32 sums a
// second kernel adds in part order.
#include <atomic>
#include <type_traits>

#include "internal.hpp"

namespace fq {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8v;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int BI = 256;   // tile rows (i)
constexpr int BJ = 256;   // tile cols (j)
constexpr int BK = 64;    // contraction elements per stage
constexpr int NSTAGE = 2;
constexpr int NT = 512;   // threads per block (8 waves, 2 per SIMD)
constexpr int WJ_TILE = 64;  // j extent of one wave (waves: 2 along i x 4 along j)
constexpr int kStageBytes = 256 * BK * 2;  // one operand, one stage: 32 KiB

enum Mode { FWD = 0, DGRAD = 1, WGRAD = 2 };

// The ring: one LDS object holding both stages of both operands, so that the
// stage and operand offsets of every fragment read are compile-time
// immediates on one base address.
__shared__ __attribute__((aligned(1024))) char g_ring[4 * kStageBytes];

template <int S>
__device__ __forceinline__ char *stage_p() {
  return g_ring + S * kStageBytes;
}
template <int S>
__device__ __forceinline__ char *stage_q() {
  return g_ring + (2 + S) * kStageBytes;
}

// Contraction-contiguous layout: row idx (0..255) of 8 16-byte chunks (8
// contraction elements each); chunk kc sits at kc ^ sw(idx). The swizzle
// (rows in pairs share one) was chosen by measuring the LDS bank-conflict
// counter for the fragment read pattern (32 consecutive rows, one chunk).
__device__ __forceinline__ uint32_t nrm_sw(uint32_t idx) { return (idx >> 1) & 7u; }
__device__ __forceinline__ uint32_t nrm_off(uint32_t idx, uint32_t kc) {
  return idx * 128u + ((kc ^ nrm_sw(idx)) << 4);
}
// Transposed layout: contraction row c (0..63) of 32 16-byte chunks (8 columns
// each); column chunk q sits at q ^ tr_sw(c). Within the four rows a
// ds_read_tr16_b64 group touches, the swizzle spreads their chunks over
// distinct banks.
__device__ __forceinline__ uint32_t tr_sw(uint32_t c) {
  const uint32_t r = c & 3u;
  return 4u * r + 2u * (r >> 1);
}
__device__ __forceinline__ uint32_t trn_off(uint32_t c, uint32_t chunk) {
  return c * 512u + ((chunk ^ tr_sw(c)) << 4);
}

// 16 bytes per lane from global memory into LDS at lds_wave_base + 16 * lane:
// the lane reads base + off (base uniform, held in scalar registers).
// Issued as inline asm: the compiler then does not model the LDS write and
// inserts no wait before reads of the other stages; the ring's own
// vmcnt waits and barriers order the accesses. The compiler's hazard pass
// does not look inside the asm, so it starts with the wait states the
// hardware needs when the instruction just before wrote M0 (one) or, as a
// vector instruction (v_readfirstlane), one of the base registers (five).
__device__ __forceinline__ void dma16(const char *base, uint32_t off, char *lds_wave_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  // readfirstlane returns a signed int: widen through uint32_t (no sign extension)
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "{m0}"(m0v)
               : "memory");
}

// One barrier for the whole block without a memory fence (a fence would wait
// for every outstanding load, draining the ring).
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt lgkmcnt(0) leaving the other counters alone (gfx9 encoding): this
// wave's LDS reads have returned
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
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
  float *dscale, *dzp;     // final outputs [E, N, K/group]
  // Row chunks: the contraction over an expert's rows is split into chunks of
  // at most chunk_rows rows (every expert has at least one). An expert with
  // one chunk and group <= 128 writes dScale directly; otherwise each chunk
  // writes partial sums per block of min(group, 128) along K to
  // part_s / part_z [chunk, N, K / block], summed afterwards in chunk order.
  int chunk_rows;
  FastDiv gdiv16;          // division by group / 16
  float *part_s, *part_z;
  int *chunk_start_out;    // [E+1] chunk prefix, written by block 0
  // X rows through the routing (FWD's Q, WGRAD's P): routed row r reads row
  // xperm[r] / topk of a token-indexed X; NULL = X is indexed by routed row
  const int32_t *xperm;
  FastDiv xtopk;
  // FWD / DGRAD split along the contraction (small calls that would leave CUs
  // idle): each tile's contraction runs as ksplit parts of kper stages, part
  // s writing fp32 sums to part[s, R_max, ldo], added afterwards in part order
  int ksplit, kper;
  float *part;
  int part_rows;
  // FWD / DGRAD tile order: groups of gm row tiles, each group's tiles with
  // the row tile fastest (gm = 1: i fastest)
  int gm;
};

constexpr int kMaxExperts = 1024;

// tile_start[e] = number of work units of experts 0..e-1 (e = 0..E), from
// seg_offsets on the device: a block-wide exclusive scan in LDS. Units per
// expert: ceil(rows / rows_per_unit), at least min_units.
__device__ void build_tile_prefix(const int32_t *seg, int E, int rows_per_unit, int min_units,
                                  int *tile_start) {
  __shared__ int s_wsum[NT / 64];
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int e = e0 + threadIdx.x;
    const int nt =
        e < E ? max((seg[e + 1] - seg[e] + rows_per_unit - 1) / rows_per_unit, min_units) : 0;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wsum[w] = x;
    __syncthreads();
    int before = base, total = base;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
      if (k < w) before += s_wsum[k];
      total += s_wsum[k];
    }
    if (e < E) tile_start[e] = before + x - nt;
    __syncthreads();
    base = total;
  }
  if (threadIdx.x == 0) tile_start[E] = base;
  __syncthreads();
}

// expert of row tile `tile`: the last e with tile_start[e] <= tile
__device__ __forceinline__ int expert_of_tile(const int *tile_start, int E, int tile) {
  int lo = 0, hi = E;  // tile_start[lo] <= tile < tile_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tile) lo = mid;
    else hi = mid;
  }
  return lo;
}

// dS of the 128 (k) x 32 (n) slab of dWq that column sub-tile U (0..1) of one wave
// holds: lane n = n0 + lane%32, k = k0 + 32s + 8q + 4(lane/32) + v for
// acc[s][U][4q + v]. Each dWq element is weighted by its straight-through
// factor and summed over its quantization group in a fixed order.
// this lane's raw weights of the slab: k = k0 + 32s + 8q + 4h + v
// The raw weights of the slab rows n0 .. n0+31, k0 .. k0+127 (32 x 256 bytes)
// into this wave's 8 KiB of LDS with whole-row DMA, row r at byte 256 r, its
// 16-byte chunk c at position c ^ (r & 15) (the reads below, 32 rows at one
// chunk, then spread over the banks).
__device__ __forceinline__ void wgrad_dma_w(const GemmArgs &a, int e, int k0, int n0, int lane,
                                            char *slab) {
  const char *wbase = reinterpret_cast<const char *>(a.w + ((size_t)e * a.N + n0) * a.K + k0);
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const uint32_t r = 4u * ii + (uint32_t)(lane >> 4);
    const uint32_t c = (uint32_t)(lane & 15) ^ (r & 15u);
    dma16(wbase, (r * (uint32_t)a.K + c * 8u) * 2u, slab + ii * 1024);
  }
}
// this lane's raw weights of the slab: k = k0 + 32s + 8q + 4h + v, n = n0 + lane%32
__device__ __forceinline__ void wgrad_read_w(const char *slab, int lane, uint2 (&wv)[4][4]) {
  const uint32_t jr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c = (uint32_t)(4 * s + q) ^ (jr & 15u);
      wv[s][q] = *reinterpret_cast<const uint2 *>(slab + jr * 256 + (c << 4) + h * 8);
    }
}
// The scale parameters of one epilogue half (rows n0 .. n0+31, this lane's
// row and eight 16-blocks k0 + 16 j). They are loaded before the epilogue's
// barrier and completed before its first DMA: the compiler does not see the
// DMAs, so a wait it inserts for a load issued among them would drain them.
struct WgradEpiIn {
  float4 th;    // NVFP4: theta of the eight blocks (this lane half's four)
  float g;      // NVFP4: the expert's tensor scale
  float sc[8];  // FP8 / INT8: scale of each block's group
};
template <int WFMT>
__device__ __forceinline__ WgradEpiIn wgrad_epi_load(const GemmArgs &a, int e, int k0, int n0,
                                                     int lane) {
  WgradEpiIn in;
  const size_t srow = ((size_t)e * a.N + n0 + (lane & 31)) * (a.K / a.group);
  if (WFMT == FQ_FMT_NVFP4) {
    in.th = *reinterpret_cast<const float4 *>(a.scale + srow + k0 / 16 + 4 * (lane >> 5));
    in.g = a.gscale[e];
  } else if (WFMT != FQ_FMT_INT4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t gi = a.gdiv16.div((uint32_t)(k0 / 16 + j));
      in.sc[j] = a.scale[srow + gi];
    }
  }
  return in;
}
// the loads of `in` complete here (an empty asm that reads and writes them)
template <int WFMT>
__device__ __forceinline__ void wgrad_epi_ready(WgradEpiIn &in) {
  if (WFMT == FQ_FMT_NVFP4) {
    asm volatile("" : "+v"(in.th.x), "+v"(in.th.y), "+v"(in.th.z), "+v"(in.th.w), "+v"(in.g));
  } else if (WFMT != FQ_FMT_INT4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(in.sc[j]));
  }
}

// `chunk` < 0: this tile's dScale sums are final and go to dscale / dzp;
// otherwise they are partials of row chunk `chunk` (blocks of min(group, 128)).
template <int WFMT, int U>
__device__ __forceinline__ void wgrad_epilogue(const GemmArgs &a, const f32x16 (&acc)[4][2], int e,
                                               int k0, int n0, int lane, const uint2 (&wv)[4][4],
                                               int chunk, const WgradEpiIn &in) {
  const int n = n0 + (lane & 31);
  const int G = a.K / a.group;
  const float g_e = (WFMT == FQ_FMT_NVFP4) ? in.g : 1.0f;
  const size_t srow = ((size_t)e * a.N + n) * G;
  const int blk = a.group < 128 ? a.group : 128;
  const size_t orow = chunk < 0 ? srow : ((size_t)chunk * a.N + n) * (a.K / blk);
  float *ds_out = chunk < 0 ? a.dscale : a.part_s;
  float *dz_out = chunk < 0 ? a.dzp : a.part_z;
  // scale, reciprocal, theta factor and zero point of this lane's eight
  // 16-blocks k0 + 16 j (every group is a multiple of 16 long)
  float sc8[8], r8[8], fac8[8], zp8[8];
  if (WFMT == FQ_FMT_NVFP4) {
    // lane halves share n and all eight blocks: each half derives four of
    // them (theta rounded to E4M3, its reciprocal, the theta factor) and
    // takes the other four from lane ^ 32
    const int h = lane >> 5;
    const float th[4] = {in.th.x, in.th.y, in.th.z, in.th.w};
    float rm[4], fm[4];
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      float v0, v1;
      e4m3_pair(fminf(fmaxf(th[j], 0.0f), kE4M3Max), fminf(fmaxf(th[j + 1], 0.0f), kE4M3Max), v0, v1);
      rm[j] = safe_recip(v0 * g_e);
      rm[j + 1] = safe_recip(v1 * g_e);
      fm[j] = nvfp4_theta_factor(th[j], g_e);
      fm[j + 1] = nvfp4_theta_factor(th[j + 1], g_e);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ro = __shfl_xor(rm[j], 32, 64), fo = __shfl_xor(fm[j], 32, 64);
      r8[j] = h ? ro : rm[j];
      r8[4 + j] = h ? rm[j] : ro;
      fac8[j] = h ? fo : fm[j];
      fac8[4 + j] = h ? fm[j] : fo;
      sc8[j] = sc8[4 + j] = 0.0f;  // the E2M1 factor needs only the reciprocal
      zp8[j] = zp8[4 + j] = 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (WFMT == FQ_FMT_INT4) {  // loaded here (see the caller)
        const uint32_t gi = a.gdiv16.div((uint32_t)(k0 / 16 + j));
        sc8[j] = a.scale[srow + gi];
        zp8[j] = fminf(fmaxf(rintf(a.zero_point[srow + gi]), 0.0f), 15.0f);
      } else {
        sc8[j] = in.sc[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r8[j] = safe_recip(sc8[j]);
      if (WFMT != FQ_FMT_INT4) zp8[j] = 0.0f;
      fac8[j] = 1.0f;
    }
  }
  float part_s[4], part_z[4];
  float o16[8], z16[8];  // group 16: the eight block sums of this lane's row
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float ps16[2], pz16[2];  // the sub-tile's two 16-blocks
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float sc = sc8[2 * s + b], r = r8[2 * s + b], zpi = zp8[2 * s + b];
      const float fac = fac8[2 * s + b];
      float accs = 0.0f, accz = 0.0f;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = 2 * b + qq;
        const float x4[4] = {lo_bf16(wv[s][q].x), hi_bf16(wv[s][q].x), lo_bf16(wv[s][q].y),
                             hi_bf16(wv[s][q].y)};
        float phi[4], dzp[4];
        ste_factor2<WFMT>(x4[0], x4[1], sc, r, zpi, phi[0], phi[1], dzp[0], dzp[1]);
        ste_factor2<WFMT>(x4[2], x4[3], sc, r, zpi, phi[2], phi[3], dzp[2], dzp[3]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float d = acc[s][U][4 * q + v];
          accs = fmaf(d, phi[v], accs);
          if (WFMT == FQ_FMT_INT4) accz = fmaf(d, dzp[v], accz);
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
    o16[2 * s] = ps16[0];
    o16[2 * s + 1] = ps16[1];
    z16[2 * s] = pz16[0];
    z16[2 * s + 1] = pz16[1];
    part_s[s] = ps16[0] + ps16[1];
    part_z[s] = pz16[0] + pz16[1];
  }
  if (a.group == 16) {
    // both lane halves hold the row's eight sums: half h stores blocks
    // 4h .. 4h+3 as one 16-byte store (the 32 rows x 32 bytes in one
    // instruction instead of eight 4-byte ones)
    const int h = lane >> 5;
    const size_t o = orow + k0 / 16 + 4 * h;
    float4 v;
    v.x = h ? o16[4] : o16[0];
    v.y = h ? o16[5] : o16[1];
    v.z = h ? o16[6] : o16[2];
    v.w = h ? o16[7] : o16[3];
    *reinterpret_cast<float4 *>(ds_out + o) = v;
    if (WFMT == FQ_FMT_INT4 && dz_out) {
      float4 z;
      z.x = h ? z16[4] : z16[0];
      z.y = h ? z16[5] : z16[1];
      z.z = h ? z16[6] : z16[2];
      z.w = h ? z16[7] : z16[3];
      *reinterpret_cast<float4 *>(dz_out + o) = z;
    }
  }
  if (lane < 32 && a.group != 16) {
    if (a.group == 32) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kb = (k0 + s * 32) / 32;
        ds_out[orow + kb] = part_s[s];
        if (WFMT == FQ_FMT_INT4 && dz_out) dz_out[orow + kb] = part_z[s];
      }
    } else if (a.group == 64) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int kb = (k0 + h2 * 64) / 64;
        ds_out[orow + kb] = part_s[2 * h2] + part_s[2 * h2 + 1];
        if (WFMT == FQ_FMT_INT4 && dz_out) dz_out[orow + kb] = part_z[2 * h2] + part_z[2 * h2 + 1];
      }
    } else {  // group 128 (final or partial) or a 128-block of a longer group (partial)
      const float s128 = (part_s[0] + part_s[1]) + (part_s[2] + part_s[3]);
      const float z128 = (part_z[0] + part_z[1]) + (part_z[2] + part_z[3]);
      const int kb = k0 / 128;
      ds_out[orow + kb] = s128;
      if (WFMT == FQ_FMT_INT4 && dz_out) dz_out[orow + kb] = z128;
    }
  }
}

// Per-lane global byte offsets of the operand rows this lane streams, fixed
// for a tile. A wave issues 4 DMA instructions per operand per stage, each
// filling 1 KiB of LDS (lane l -> byte 16 l of it).
struct NormalDMA {  // contraction-contiguous: instr covers 8 rows x 128 B; slot = 32 rows
  uint32_t off[4];
  __device__ __forceinline__ void init(size_t ld, int row0, int row_last, int slot, int lane) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const uint32_t idx = 8 * (4 * slot + ii) + (lane >> 3);
      const uint32_t kc = (lane & 7) ^ nrm_sw(idx);
      const int r = min(row0 + (int)idx, row_last);
      off[ii] = (uint32_t)(((size_t)r * ld + kc * 8) * 2);
    }
  }
  // the same rows taken through the routing: row r of the tile reads row
  // perm[r] / topk of the operand
  __device__ __forceinline__ void init_routed(size_t ld, int row0, int row_last, int slot,
                                              int lane, const int32_t *perm, FastDiv topk) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const uint32_t idx = 8 * (4 * slot + ii) + (lane >> 3);
      const uint32_t kc = (lane & 7) ^ nrm_sw(idx);
      const uint32_t r = topk.div((uint32_t)perm[min(row0 + (int)idx, row_last)]);
      off[ii] = (uint32_t)(((size_t)r * ld + kc * 8) * 2);
    }
  }
  template <int S>
  __device__ __forceinline__ void issue(const char *base, char *stage, int c0, int slot) const {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) dma16(base + c0 * 2, off[ii], stage + (4 * slot + ii) * 1024);
  }
};
struct TransDMA {  // transposed: instr covers 2 contraction rows x 512 B; slot = 8 rows
  uint32_t col_off[4];
  int crow0;  // contraction row of instruction ii within the stage: crow0 + 2 ii
  __device__ __forceinline__ int crow(int ii) const { return crow0 + 2 * ii; }
  __device__ __forceinline__ void init(int idx0, int slot, int lane) {
    crow0 = 8 * slot + (lane >> 5);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const uint32_t q = (lane & 31) ^ tr_sw(crow(ii));
      col_off[ii] = (uint32_t)((idx0 + 8 * q) * 2);
    }
  }
  // rows c >= c_end are read from row c0 (valid memory) and zeroed later
  __device__ __forceinline__ void issue(const char *base, uint32_t ld, char *stage, int c0,
                                        int c_end, int slot) const {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int c = c0 + crow(ii);
      const int cc = c < c_end ? c : c0;
      dma16(base, (uint32_t)cc * (ld * 2) + col_off[ii], stage + (4 * slot + ii) * 1024);
    }
  }
  // routed rows: lane m (m < 8) of `pair` holds the (token, slot) pair index
  // of the slot's row crow0 - crow0 % 8 + m, looked up a stage ahead;
  // instruction ii reads operand row pair / topk of its row. Each lane turns
  // its pair into a row offset once and instruction ii takes the offset from
  // lane crow0 % 8 + 2 ii. Dividing here, not at the lookup, keeps the
  // lookup's load from being waited on before this stage.
  __device__ __forceinline__ void issue_rows(const char *base, uint32_t ld, char *stage,
                                             uint32_t pair, FastDiv topk, int slot,
                                             int lane) const {
    const int row_off = (int)(topk.div(pair) * (ld * 2));
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const uint32_t off = (uint32_t)__shfl(row_off, 2 * ii + (lane >> 5), 64);
      dma16(base, off + col_off[ii], stage + (4 * slot + ii) * 1024);
    }
  }
};

// MFMA fragment (8 contraction elements of one row / column) from a stage
__device__ __forceinline__ bf16x8v frag_normal(const char *stage, int base, int ks, int lane) {
  return *reinterpret_cast<const bf16x8v *>(stage + nrm_off(base + (lane & 31), 2 * ks + (lane >> 5)));
}
__device__ __forceinline__ bf16x8v frag_trans(const char *stage, int base, int ks, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint32_t chunk = (uint32_t)(base >> 3) + 2 * (g & 1) + ((j & 3) >> 1);
  const uint32_t half = (j & 1) * 8;
  const uint32_t c = 16 * ks + 8 * (g >> 1) + (j >> 2);
  const v4i16 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(stage + trn_off(c, chunk) + half));
  const v4i16 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(stage + trn_off(c + 4, chunk) + half));
  const v4i16 a[2] = {lo, hi};
  bf16x8v r;
  __builtin_memcpy(&r, a, 16);
  return r;
}
// zero the contraction elements c0 + 16 ks + 8 (lane/32) + t >= c_end
__device__ __forceinline__ bf16x8v zero_tail(bf16x8v f, int cfirst, int c_end) {
  uint32_t w[4];
  __builtin_memcpy(w, &f, 16);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = cfirst + 2 * t;
    const uint32_t keep = (c < c_end ? 0x0000FFFFu : 0u) | (c + 1 < c_end ? 0xFFFF0000u : 0u);
    w[t] &= keep;
  }
  bf16x8v r;
  __builtin_memcpy(&r, w, 16);
  return r;
}

// One output tile: expert e, i range [i0, i0+256), j range [j0, j0+256)
// (FWD / DGRAD: routed rows, valid below j_end).
struct Tile {
  int e, i0, j0, j_end;
  int r0, r1;  // WGRAD: the routed rows [r0, r1) of this row chunk
  int chunk;   // WGRAD: -1 = dScale written directly, else the partial row
  int ks;      // FWD / DGRAD split along the contraction: the part
};

// Tile w of the list. FWD / DGRAD tiles: (row tile, i tile), the row tiles
// of each expert from tile_start, in groups of gm row tiles: a group's tiles
// run i tile by i tile, its row tiles fastest (gm = 1: i fastest), so that
// the tiles in flight on an XCD form a block that shares both operands'
// panels (GROUPED; the routed-X kernels, short of registers, keep gm = 1).
// WGRAD: (expert, j tile, i tile).
template <int MODE, bool SPLIT = false, bool GROUPED = false>
__device__ __forceinline__ Tile decode_tile(const GemmArgs &a, const int *tile_start, int w) {
  Tile t;
  t.j_end = 0;
  t.chunk = -1;
  t.ks = 0;
  if constexpr (SPLIT) {  // unit (tile, part), parts fastest
    t.ks = w % a.ksplit;
    w /= a.ksplit;
  }
  if (MODE == WGRAD) {
    // unit (row chunk c, j tile, i tile); tile_start holds the chunk prefix
    const int per_c = a.n_it * a.n_jt;
    const int c = w / per_c;
    const int rem = w - c * per_c;
    const int jt = rem / a.n_it;
    t.i0 = (rem - jt * a.n_it) * BI;
    t.j0 = jt * BJ;
    t.e = expert_of_tile(tile_start, a.E, c);
    const int lc = c - tile_start[t.e];
    t.r0 = a.seg[t.e] + lc * a.chunk_rows;
    t.r1 = min(t.r0 + a.chunk_rows, a.seg[t.e + 1]);
    const bool single = tile_start[t.e + 1] - tile_start[t.e] == 1;
    t.chunk = (single && a.group <= 128) ? -1 : c;
  } else {
    int tile;
    if constexpr (GROUPED) {
      const int gsz = a.gm * a.n_it;  // units per group
      const int g = w / gsz;
      const int rt0 = g * a.gm;
      const int gs = min(a.gm, tile_start[a.E] - rt0);
      const int win = w - g * gsz;
      const int it = win / gs;
      tile = rt0 + (win - it * gs);
      t.i0 = it * BI;
    } else {
      tile = w / a.n_it;
      t.i0 = (w - tile * a.n_it) * BI;
    }
    t.e = expert_of_tile(tile_start, a.E, tile);
    t.j0 = a.seg[t.e] + (tile - tile_start[t.e]) * BJ;
    t.j_end = a.seg[t.e + 1];
  }
  return t;
}

// The operand streams of one tile: bases, per-lane offsets and the
// contraction length. issue<S>(kt) loads this wave's share of stage kt into
// LDS buffer S.
//
// Shares. A stage of each operand is 8 slots of 4 DMA instructions (4 KiB).
// WGRAD (all waves in step): wave w loads slot w of P and of Q. FWD / DGRAD
// (the ping-pong below): each group loads the LDS locations that it does not
// read in the phase where it issues the loads. Wave w loads Q slot w ^ 4, so
// group B fills the Q rows that group A multiplies (rows 0-127) and A those
// of B. DGRAD's transposed P slot s holds contraction rows 8s..8s+7 of every
// column: wave w loads P slot w ^ 4, so B fills the first half of the stage
// depth, which it has read already, and A the second. FWD's P slot holds 32
// full-depth rows that waves of both groups read, so group A loads all of P
// (slots 2w and 2w + 1) and B none.
template <int MODE>
constexpr int kVmPerStageA = MODE == FWD ? 12 : 8;  // DMA instructions per wave and stage
template <int MODE>
constexpr int kVmPerStageB = MODE == FWD ? 4 : 8;

// ROUTED: X (FWD's Q, WGRAD's P) is read by token row through a.xperm
// (compile time, so the kernels without it keep their registers).
template <int MODE, bool ROUTED, bool SPLIT = false>
struct TileLoads {
  const char *pbase, *qbase;
  int c_total, nk;
  int c_lo;  // SPLIT: the first contraction element of this part
  NormalDMA pn, qn;
  TransDMA pt, qt;
  // WGRAD with routed X: the (token, slot) pair indices of this wave's eight
  // P rows of the next stage to issue (row 8 wave + lane % 8), loaded one
  // stage ahead so that no DMA issue waits on them
  int seg_lo;
  uint32_t ppair;
  // first_kt: the first stage this object will issue (WGRAD: 1 when the
  // previous tile already issued stage 0)
  __device__ __forceinline__ TileLoads(const GemmArgs &a, const Tile &t, int wave, int lane,
                                       int first_kt = 0) {
    seg_lo = (MODE == WGRAD) ? t.r0 : 0;
    c_total = (MODE == WGRAD) ? t.r1 - t.r0 : (MODE == FWD) ? a.K : a.N;
    c_lo = 0;
    if constexpr (SPLIT) {
      c_lo = t.ks * a.kper * BK;
      c_total = min(a.kper * BK, c_total - c_lo);
    }
    nk = (c_total + BK - 1) / BK;
    const size_t NK = (size_t)a.N * a.K;
    const int xs = wave ^ 4;
    if (MODE == FWD) {
      pbase = reinterpret_cast<const char *>(a.p + t.e * NK);  // W_fq[e] [N][K], rows i = n
      qbase = reinterpret_cast<const char *>(a.q);             // Xq rows (absolute)
      // slot 2w here; slot 2w + 1 is the same offsets 32 rows on (N is a
      // multiple of 256, so no P row of a tile is clamped)
      pn.init(a.K, t.i0, a.N - 1, 2 * (wave & 3), lane);
      if constexpr (ROUTED) qn.init_routed(a.K, t.j0, t.j_end - 1, xs, lane, a.xperm, a.xtopk);
      else qn.init(a.K, t.j0, t.j_end - 1, xs, lane);
    } else if (MODE == DGRAD) {
      pbase = reinterpret_cast<const char *>(a.p + t.e * NK);  // W_fq[e] as (c = n, idx = k)
      qbase = reinterpret_cast<const char *>(a.q);             // dY rows (absolute)
      pt.init(t.i0, xs, lane);
      qn.init(a.N, t.j0, t.j_end - 1, xs, lane);
    } else {
      // Xq: (c = r, idx = k), by routed row or (routed X) by token row
      pbase = reinterpret_cast<const char *>(ROUTED ? a.p : a.p + (size_t)seg_lo * a.K);
      qbase = reinterpret_cast<const char *>(a.q + (size_t)seg_lo * a.N);  // dY: (c = r, idx = n)
      pt.init(t.i0, wave, lane);
      qt.init(t.j0, wave, lane);
      if constexpr (ROUTED) {
        if (first_kt < nk) look_ahead(a, first_kt);
      }
    }
  }
  // WGRAD, routed X: the pair indices of stage kt's P rows, one row per
  // lane (rows past the chunk's end read row c0, as in TransDMA::issue)
  __device__ __forceinline__ void look_ahead(const GemmArgs &a, int kt) {
    const int c0 = kt * BK;
    const int c = c0 + (pt.crow0 & ~7) + (int)(threadIdx.x & 7);
    const int cc = c < c_total ? c : c0;
    ppair = (uint32_t)a.xperm[seg_lo + cc];
  }
  // stages are issued in order kt = first_kt, first_kt + 1, ...
  template <int S>
  __device__ __forceinline__ void issue(const GemmArgs &a, int kt, int wave) {
    const int c0 = (SPLIT ? c_lo : 0) + kt * BK;
    const int xs = wave ^ 4;
    if (MODE == FWD) {
      if (wave < 4) {
        pn.template issue<S>(pbase, stage_p<S>(), c0, 2 * wave);
        pn.template issue<S>(pbase + (size_t)64 * a.K, stage_p<S>(), c0, 2 * wave + 1);
      }
      qn.template issue<S>(qbase, stage_q<S>(), c0, xs);
    } else if (MODE == DGRAD) {
      pt.issue(pbase, a.K, stage_p<S>(), c0, (SPLIT ? c_lo : 0) + c_total, xs);
      qn.template issue<S>(qbase, stage_q<S>(), c0, xs);
    } else {
      if constexpr (ROUTED) {
        pt.issue_rows(pbase, a.K, stage_p<S>(), ppair, a.xtopk, wave, (int)(threadIdx.x & 63));
        if (kt + 1 < nk) look_ahead(a, kt + 1);
      } else {
        pt.issue(pbase, a.K, stage_p<S>(), c0, c_total, wave);
      }
      qt.issue(qbase, a.N, stage_q<S>(), c0, c_total, wave);
    }
  }
};

// WGRAD tile, all eight waves in step (the wgrad loop measured faster this
// way than in the ping-pong below: its wider epilogue leaves the ping-pong's
// registers short). If `pre` is set, stage 0 of this tile is already in
// flight; if next_w >= 0, stage 0 of tile next_w is issued once every wave
// is done with this tile's LDS buffers, so that its loads run under this
// tile's epilogue.
template <int MODE, int WFMT, bool ROUTED>
__device__ __forceinline__ void run_tile_wgrad(const GemmArgs &a, const int *tile_start,
                                               const Tile &tl, bool pre, int next_w) {
  static_assert(MODE == WGRAD, "the lockstep loop serves the wgrad tiles");
  const int t = threadIdx.x;
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wi = wave & 1, wj = wave >> 1;  // 2 x 4 waves: 128 (i) x 64 (j) each
  const int e = tl.e, i0 = tl.i0, j0 = tl.j0;
  TileLoads<MODE, ROUTED> ld(a, tl, wave, lane, pre ? 1 : 0);
  const int c_total = ld.c_total, nk = ld.nk;

  auto issue = [&](auto stage_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    ld.template issue<S>(a, kt, wave);
  };
  // stage 0 of the next tile into buffer 0 (every wave must have left this
  // tile's buffers); true if its eight DMA instructions were issued
  auto prefetch_issue = [&]() {
    if (next_w < 0) return false;
    const Tile nt = decode_tile<MODE>(a, tile_start, next_w);
    TileLoads<MODE, ROUTED> nl(a, nt, wave, lane);
    if (nl.nk <= 0) return false;
    nl.template issue<0>(a, 0, wave);
    return true;
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[s][u][v] = 0.0f;

  // MFMA fragments of one 16-deep step: 4 P sub-tiles, 2 Q sub-tiles
  struct Frags {
    bf16x8v p[4], q[2];
  };
  // contraction rows past the chunk's last routed row (its last stage) are
  // zeroed in the fragments
  auto read_frags = [&](auto stage_tag, int kt, int ks, Frags &f) {
    constexpr int S = decltype(stage_tag)::value;
    const char *sp = stage_p<S>();
    const char *sq = stage_q<S>();
#pragma unroll
    for (int s = 0; s < 4; ++s) f.p[s] = frag_trans(sp, wi * 128 + s * 32, ks, lane);
#pragma unroll
    for (int u = 0; u < 2; ++u) f.q[u] = frag_trans(sq, wj * WJ_TILE + u * 32, ks, lane);
    if ((kt + 1) * BK > c_total) {
      const int cfirst = kt * BK + 16 * ks + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < 4; ++s) f.p[s] = zero_tail(f.p[s], cfirst, c_total);
#pragma unroll
      for (int u = 0; u < 2; ++u) f.q[u] = zero_tail(f.q[u], cfirst, c_total);
    }
  };
  auto mfmas = [&](const Frags &f) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[s][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.p[s], f.q[u], acc[s][u], 0, 0, 0);
  };
  // Two-stage ring: stage kt lives in buffer kt % 2. After this wave's loads
  // of stage kt have landed, one barrier both publishes stage kt to every wave
  // and retires the reads of stage kt-1, whose buffer then takes stage kt+1
  // while stage kt is multiplied. One fragment set (two measured slower).
  auto step = [&](auto stage_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    wait_vm<0>();
    block_barrier();
    if (kt + 1 < nk) issue(std::integral_constant<int, S ^ 1>{}, kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      Frags f;
      read_frags(stage_tag, kt, ks, f);
      mfmas(f);
    }
  };
  if (nk > 0 && !pre) issue(std::integral_constant<int, 0>{}, 0);
  for (int kt = 0; kt < nk; kt += NSTAGE) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
  }

  // accumulator (s, u, v) of this lane: i = i0 + wi*128 + s*32 + 8*(v/4) + 4*(lane/32) + v%4,
  //                                     j = j0 + wj*64 + u*32 + lane%32
  // ---- WGRAD epilogue: i = k, j = n of expert e. dS over groups along k.
  {
    // The raw weights come in through ring buffer 1 (free once every wave has
    // left the contraction loop, until the next tile's second stage), each
    // wave's two 32-row slabs one after the other in its own 8 KiB: whole-row
    // DMA instead of 8-byte loads from 32 rows per instruction. Only the wave
    // itself reads its slab, so its own waits order the accesses.
    const int k0 = i0 + wi * 128, n0 = j0 + wj * WJ_TILE;
    char *slab = (wave < 4 ? stage_p<1>() : stage_q<1>()) + (wave & 3) * 8192;
    uint2 wv[4][4];
    // The scale parameters: NVFP4 loads both halves' (5 values each) before
    // the barrier, so that their latency overlaps the wait for the slowest
    // wave, and completes them before the first DMA, so that the first
    // half's arithmetic runs while the second slab and the next tile's stage
    // 0 are in flight. FP8 / INT8 do so for the first half (8 values). INT4
    // (scales and zero points) loads inside each half's arithmetic: held
    // across the DMA set-up, they would spill.
    constexpr bool kEarly0 = WFMT != FQ_FMT_INT4, kEarly1 = WFMT == FQ_FMT_NVFP4;
    WgradEpiIn in0, in1;
    if constexpr (kEarly0) in0 = wgrad_epi_load<WFMT>(a, e, k0, n0, lane);
    if constexpr (kEarly1) in1 = wgrad_epi_load<WFMT>(a, e, k0, n0 + 32, lane);
    block_barrier();
    if constexpr (kEarly0) wgrad_epi_ready<WFMT>(in0);
    if constexpr (kEarly1) wgrad_epi_ready<WFMT>(in1);
    wgrad_dma_w(a, e, k0, n0, lane, slab);
    if (prefetch_issue()) wait_vm<8>();  // the slab, not the next tile's stage 0
    else wait_vm<0>();
    wgrad_read_w(slab, lane, wv);
    wait_lgkm0();                          // read back before the slab is reused
    wgrad_dma_w(a, e, k0, n0 + 32, lane, slab);
    wgrad_epilogue<WFMT, 0>(a, acc, e, k0, n0, lane, wv, tl.chunk, in0);
    wait_vm<0>();
    if constexpr (!kEarly1 && WFMT != FQ_FMT_INT4) in1 = wgrad_epi_load<WFMT>(a, e, k0, n0 + 32, lane);
    wgrad_read_w(slab, lane, wv);
    wgrad_epilogue<WFMT, 1>(a, acc, e, k0, n0 + 32, lane, wv, tl.chunk, in1);
  }
}

// One 256 x 256 output tile: the contraction loop and the epilogue. The
// first `pre` stages of this tile (0, 1 or 2) are already in flight. If
// next_w >= 0, the first two stages of tile next_w are issued as this tile's
// buffers free up (stage 0 before the epilogue, stage 1 after it), so that
// their loads run under the epilogue; the return value is the number of them
// issued.
//
// Ping-pong: waves w and w + 4 share a SIMD (the hardware's placement of an
// 8-wave workgroup), so group A = waves 0-3 and group B = waves 4-7 hold one
// wave of each SIMD. The groups run a quarter stage apart. Between two block
// barriers one group multiplies half a stage (two 16-deep steps) from
// registers while the other reads its fragments of the next half from LDS
// (and, twice a stage, issues its share of the loads two stages ahead), so
// every SIMD always has a wave with MFMAs to issue, and the LDS read latency
// and the barrier wait sit under them. With h = 0, 1 the halves of stage t:
//   phase 4t     : A multiplies t.0  | B reads t.0
//   phase 4t + 1 : B multiplies t.0  | A reads t.1
//   phase 4t + 2 : A multiplies t.1  | B reads t.1,   loads its share of t+2
//   phase 4t + 3 : B multiplies t.1  | A reads t+1.0, loads its share of t+2
// Stage t lives in buffer t % 2. A load may land in LDS as soon as it is
// issued, so a wave issues a load only into locations that no wave reads in
// that phase or later; its own returned reads are not enough, since the
// other waves of its group read the same phase. The shares (TileLoads) make
// this hold: in phase 4t + 2 group B loads only locations of buffer t % 2
// that nobody reads from then on (the Q rows of group A, and for DGRAD the
// first half of the stage depth), and in phase 4t + 3 group A loads the rest,
// after the last read of stage t. Each wave waits for its own loads of a
// stage before the barrier that opens the first phase reading it. A's
// epilogue runs while B multiplies the last half.
template <int MODE, int WFMT, bool ROUTED, bool SPLIT>
__device__ __forceinline__ int run_tile(const GemmArgs &a, const int *tile_start, const Tile &tl,
                                        int pre, int next_w) {
  static_assert(MODE != WGRAD, "the ping-pong serves the forward and dgrad tiles");
  const int t = threadIdx.x;
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wi = wave & 1, wj = wave >> 1;  // 2 x 4 waves: 128 (i) x 64 (j) each
  const bool grp_b = wave >= 4;             // j columns 128..255 of the tile
  const int i0 = tl.i0, j0 = tl.j0, j_end = tl.j_end;
  TileLoads<MODE, ROUTED, SPLIT> ld(a, tl, wave, lane);
  const int nk = ld.nk;
  // a wave whose 64 rows all lie past the expert's last row (the ragged last
  // row tile) skips its fragment reads and MFMAs; it still takes part in the
  // loads and barriers
  const bool live = j0 + wj * WJ_TILE < j_end;

  f32x16 acc[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[s][u][v] = 0.0f;

  // MFMA fragments of one 16-deep step: 4 P sub-tiles, 2 Q sub-tiles; a
  // wave holds half a stage (2 steps) between its read and multiply phases
  struct Frags {
    bf16x8v p[4], q[2];
  };
  Frags f[2];
  // half h of stage kt from buffer S
  auto read_half = [&](auto stage_tag, int h) {
    constexpr int S = decltype(stage_tag)::value;
    const char *sp = stage_p<S>();
    const char *sq = stage_q<S>();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int ks = 2 * h + k2;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        f[k2].p[s] = (MODE == FWD) ? frag_normal(sp, wi * 128 + s * 32, ks, lane)
                                   : frag_trans(sp, wi * 128 + s * 32, ks, lane);
#pragma unroll
      for (int u = 0; u < 2; ++u) f[k2].q[u] = frag_normal(sq, wj * WJ_TILE + u * 32, ks, lane);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[s][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[k2].p[s], f[k2].q[u], acc[s][u], 0,
                                                              0, 0);
  };
  // a block barrier that the scheduler moves nothing across (MFMAs would
  // otherwise drift into the other group's phase)
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // group A, stage kt in buffer S (its first half already read)
  auto a_step = [&](auto stage_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    phase_barrier();  // 4kt
    if (live) multiply();
    phase_barrier();  // 4kt+1
    if (live) read_half(stage_tag, 1);
    wait_lgkm0();
    phase_barrier();  // 4kt+2
    if (live) multiply();
    if (kt + 1 < nk) {
      wait_vm<0>();  // this wave's share of stage kt+1
      phase_barrier();  // 4kt+3
      if (live) read_half(std::integral_constant<int, S ^ 1>{}, 0);
      wait_lgkm0();
      if (kt + 2 < nk) ld.template issue<S>(a, kt + 2, wave);
    }
  };
  // group B, stage kt in buffer S
  auto b_step = [&](auto stage_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    phase_barrier();  // 4kt
    if (live) read_half(stage_tag, 0);
    wait_lgkm0();
    phase_barrier();  // 4kt+1
    if (live) multiply();
    phase_barrier();  // 4kt+2
    if (live) read_half(stage_tag, 1);
    wait_lgkm0();
    if (kt + 2 < nk) {
      ld.template issue<S>(a, kt + 2, wave);
      wait_vm<kVmPerStageB<MODE>>();  // this wave's share of stage kt+1 (read by A next phase)
    } else {
      wait_vm<0>();
    }
    phase_barrier();  // 4kt+3
    if (live) multiply();
  };

  if (nk > 0) {
    if (pre < 1) ld.template issue<0>(a, 0, wave);
    if (pre < 2 && nk > 1) ld.template issue<1>(a, 1, wave);
    if (nk <= 1) wait_vm<0>();  // this wave's share of stage 0
    else if (grp_b) wait_vm<kVmPerStageB<MODE>>();
    else wait_vm<kVmPerStageA<MODE>>();
    phase_barrier();
    if (!grp_b) {
      if (live) read_half(std::integral_constant<int, 0>{}, 0);
      wait_lgkm0();
      for (int kt = 0; kt < nk; kt += 2) {
        a_step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk) a_step(std::integral_constant<int, 1>{}, kt + 1);
      }
      phase_barrier();  // opens phase 4nk-1, B's last multiply
    } else {
      for (int kt = 0; kt < nk; kt += 2) {
        b_step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk) b_step(std::integral_constant<int, 1>{}, kt + 1);
      }
    }
  }

  // Both buffers are free from here on for this wave's group: the other
  // group no longer reads them. Stage 0 of the next tile goes to buffer 0
  // now; buffer 1 serves as this group's staging (A the P half, B the Q
  // half) and takes stage 1 of the next tile after the closing barrier.
  // The next tile's loads are set up once, here, for both stages (with
  // routed rows that means one lookup, made while no store is in flight).
  TileLoads<MODE, ROUTED, SPLIT> nl(
      a, next_w >= 0 ? decode_tile<MODE, SPLIT, SPLIT && !ROUTED>(a, tile_start, next_w) : tl, wave, lane);
  auto issue_next = [&](auto stage_tag) -> bool {
    constexpr int S = decltype(stage_tag)::value;
    if (next_w < 0) return false;
    if (nl.nk <= S) return false;
    nl.template issue<S>(a, S, wave);
    return true;
  };
  char *slab = (wave < 4 ? stage_p<1>() : stage_q<1>()) + (wave & 3) * 8192;

  // accumulator (s, u, v) of this lane: i = i0 + wi*128 + s*32 + 8*(v/4) + 4*(lane/32) + v%4,
  //                                     j = j0 + wj*64 + u*32 + lane%32
  if constexpr (SPLIT) {
    // fp32 sums of this part straight from the accumulators: four
    // consecutive i per lane (one 16-byte store), row j per lane % 32
    (void)issue_next(std::integral_constant<int, 0>{});
    const int ldo = (MODE == FWD) ? a.N : a.K;
    if (live) {
      float *pb = a.part + (size_t)tl.ks * a.part_rows * ldo + i0 + wi * 128 + 4 * (lane >> 5);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + wj * WJ_TILE + u * 32 + (lane & 31);
        if (j < j_end) {
          float *prow = pb + (size_t)j * ldo;
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = make_float4(acc[s][u][4 * q], acc[s][u][4 * q + 1],
                                           acc[s][u][4 * q + 2], acc[s][u][4 * q + 3]);
              *reinterpret_cast<float4 *>(prow + s * 32 + 8 * q) = v;
            }
        }
      }
    }
  } else {
    (void)issue_next(std::integral_constant<int, 0>{});
    // The bf16 tile goes out through LDS: each wave writes its 128 (i) x 32 (j)
    // half-slab row by row into its 8 KiB of buffer 1, then stores whole
    // 256-byte row segments, 16 bytes per lane. Direct stores from the
    // accumulator layout would write each 128-byte line in 16-byte pieces
    // from eight instructions. Row r of the slab is 16 chunks of 16 bytes;
    // chunk c sits at c ^ (r & 15), so the lanes of a write (32 rows, one
    // chunk) and of a read (one row per 16 lanes) spread over the banks.
    const int ldo = (MODE == FWD) ? a.N : a.K;
    // lane terms formed here (an empty asm keeps the compiler from hoisting
    // the addresses derived from them into the contraction loop's registers)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int h = ln >> 5, jr = ln & 31;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!live) break;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 pk;
          pk.x = pack_bf16(acc[s][u][4 * q + 0], acc[s][u][4 * q + 1]);
          pk.y = pack_bf16(acc[s][u][4 * q + 2], acc[s][u][4 * q + 3]);
          const uint32_t c = (uint32_t)(4 * s + q) ^ (uint32_t)(jr & 15);
          *reinterpret_cast<uint2 *>(slab + jr * 256 + c * 16 + h * 8) = pk;
        }
      const int jb = j0 + wj * WJ_TILE + u * 32;
      uint16_t *obase = a.out + (size_t)i0 + wi * 128 + (ln & 15) * 8;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = 4 * it + (ln >> 4);
        const uint4 v = *reinterpret_cast<const uint4 *>(
            slab + r * 256 + (((uint32_t)(ln & 15) ^ (uint32_t)(r & 15)) << 4));
        // whole 128-byte lines, stored non-temporally so that the output
        // stream does not displace operand lines from the L2
        if (jb + r < j_end) {
          uint4 *dst = reinterpret_cast<uint4 *>(obase + (size_t)(jb + r) * ldo);
          __builtin_nontemporal_store(v.x, &dst->x);
          __builtin_nontemporal_store(v.y, &dst->y);
          __builtin_nontemporal_store(v.z, &dst->z);
          __builtin_nontemporal_store(v.w, &dst->w);
        }
      }
    }
    wait_lgkm0();  // the slab is read back before buffer 1 takes the next tile's stage 1
  }
  // every wave's staging in buffer 1 is done: stage 1 of the next tile
  block_barrier();
  if (next_w < 0) return 0;
  return issue_next(std::integral_constant<int, 1>{}) ? 2 : 1;
}

// Persistent grid: one block per CU (the 128 KiB LDS ring allows one). The
// hardware deals block b to XCD b % 8, so XCD x runs blocks x, x+8, ...; it
// owns one contiguous eighth of the tile list and its blocks take tiles
// round-robin, so the tiles in flight on an XCD are neighbours that share
// operand panels in that XCD's L2. FWD / DGRAD tiles: (row tile, i tile)
// with i fastest; the row tiles of each expert follow from seg_offsets.
// WGRAD tiles: (expert, j tile, i tile).
template <int MODE, int WFMT, bool ROUTED, bool SPLIT = false>
__global__ __launch_bounds__(NT) void k_grouped_gemm(GemmArgs a) {
  __shared__ int tile_start[kMaxExperts + 1];
  int total;
  if (MODE == WGRAD) {
    build_tile_prefix(a.seg, a.E, a.chunk_rows, 1, tile_start);
    total = tile_start[a.E] * a.n_it * a.n_jt;
    if (blockIdx.x == 0 && a.chunk_start_out)
      for (int e = threadIdx.x; e <= a.E; e += NT) a.chunk_start_out[e] = tile_start[e];
  } else {
    build_tile_prefix(a.seg, a.E, BJ, 0, tile_start);
    total = tile_start[a.E] * a.n_it * (SPLIT ? a.ksplit : 1);
  }
  const int nslot = gridDim.x >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int w_end = min((xcd + 1) * chunk, total);
  int pre = 0;  // stages of the coming tile already in flight
  for (int w = xcd * chunk + slot; w < w_end; w += nslot) {
    const int next = w + nslot < w_end ? w + nslot : -1;
    const Tile tl = decode_tile<MODE, SPLIT, SPLIT && !ROUTED>(a, tile_start, w);
    if constexpr (MODE == WGRAD) {
      run_tile_wgrad<MODE, WFMT, ROUTED>(a, tile_start, tl, pre != 0, next);
      pre = next >= 0;
    } else {
      pre = run_tile<MODE, WFMT, ROUTED, SPLIT>(a, tile_start, tl, pre, next);
    }
  }
}

// dscale[e, n, g] = sum over the row chunks c of expert e (in order) of the
// sums over the blocks b of group g (in order) of part[c, n, b]; experts
// whose dScale the GEMM wrote directly are skipped. Grid: (N*G / (256*4), E),
// 4 outputs a block stride apart per thread.
__global__ __launch_bounds__(256) void k_reduce_dscale(const float *__restrict__ part_s,
                                                       const float *__restrict__ part_z,
                                                       const int *__restrict__ chunk_start, int N,
                                                       int K, int group, float *__restrict__ dscale,
                                                       float *__restrict__ dzp) {
  const int e = blockIdx.y;
  const int c0 = chunk_start[e], c1 = chunk_start[e + 1];
  if (c1 - c0 == 1 && group <= 128) return;
  const int blk = group < 128 ? group : 128;
  const int G = K / group, Gb = K / blk, per = group / blk;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = (blockIdx.x * 4 + u) * blockDim.x + threadIdx.x;  // n * G + g
    if (i >= N * G) return;
    const int n = i / G, g = i - n * G;
    float acc_s = 0.0f, acc_z = 0.0f;
    for (int c = c0; c < c1; ++c) {
      const size_t base = ((size_t)c * N + n) * Gb + (size_t)g * per;
      for (int b = 0; b < per; ++b) {
        acc_s += part_s[base + b];
        if (dzp) acc_z += part_z[base + b];
      }
    }
    const size_t o = (size_t)e * N * G + i;
    dscale[o] = acc_s;
    if (dzp) dzp[o] = acc_z;
  }
}

// A contraction split into S parts: out[j, i] = bf16(sum over s = 0..S-1, in
// that order, of part[s, j, i]) for the rows [seg[0], seg[E]) the tiles
// cover. Eight columns per thread (two 16-byte loads per part, one 16-byte
// store), grid-stride.
__global__ __launch_bounds__(256) void k_ksplit_reduce(const float *__restrict__ part, int S,
                                                       int part_rows, int ldo,
                                                       const int32_t *__restrict__ seg, int E,
                                                       uint16_t *__restrict__ out) {
  const int r0 = seg[0], r1 = seg[E];
  const int cpr = ldo >> 3;
  const int n = (r1 - r0) * cpr;
  const size_t plane = (size_t)part_rows * ldo;
  for (int idx = blockIdx.x * 256 + threadIdx.x; idx < n; idx += gridDim.x * 256) {
    const int j = r0 + idx / cpr, c = idx - (idx / cpr) * cpr;
    const size_t o = (size_t)j * ldo + (size_t)c * 8;
    float4 lo = *reinterpret_cast<const float4 *>(part + o);
    float4 hi = *reinterpret_cast<const float4 *>(part + o + 4);
    for (int k = 1; k < S; ++k) {
      const float4 a = *reinterpret_cast<const float4 *>(part + k * plane + o);
      const float4 b = *reinterpret_cast<const float4 *>(part + k * plane + o + 4);
      lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
      hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
    }
    uint4 v;
    v.x = pack_bf16(lo.x, lo.y);
    v.y = pack_bf16(lo.z, lo.w);
    v.z = pack_bf16(hi.x, hi.y);
    v.w = pack_bf16(hi.z, hi.w);
    *reinterpret_cast<uint4 *>(out + o) = v;
  }
}

}  // namespace

// ============================================================ launchers ====
// The current device's CU count rounded down to a multiple of 8 (the XCD
// count), read once per device (256 when there is no device).
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  int cus = dev >= 0 ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    cus = 256;
    if (dev >= 0) {
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
      cached[dev].store(cus, std::memory_order_relaxed);
    }
  }
  cus = cus / 8 * 8;
  return cus > 0 ? cus : 8;
}

// One block per CU, a multiple of 8, but no more blocks than an upper bound
// on the work units of the call (a small call then launches a small grid).
static int gemm_grid(size_t max_units) {
  const int cus = device_cus();
  const size_t units8 = (max_units + 7) / 8 * 8;
  return (int)(units8 < (size_t)cus ? (units8 > 0 ? units8 : 8) : (size_t)cus);
}

// FWD / DGRAD row tiles of R rows over E experts, at most: with m non-empty
// experts (m <= min(E, R)) each holds 256 (q_e - 1) + 1 rows or more for its
// q_e tiles, so the tiles number at most (R - m) / 256 + m, largest at
// m = min(E, R)
static size_t rowtile_bound(int R, int E) {
  if (R <= 0) return 0;
  const int m = E < R ? E : R;
  return (size_t)((R - m) / BJ) + (size_t)m;
}
static size_t rowtile_units(int R_max, int E, int n_it) {
  return rowtile_bound(R_max, E) * (size_t)n_it;
}

// S parts asked for, at most 8 and at least 8 stages each (the sums' second
// pass costs about as much as two stages), as the parts of ceil(nk / S)
// stages that cover nk stages
static int ksplit_parts(int S, int nk) {
  S = S < 8 ? S : 8;
  S = S < nk / 8 ? S : nk / 8;
  if (S < 2) return 1;
  const int per = (nk + S - 1) / S;
  return (nk + per - 1) / per;
}
// FWD / DGRAD split along the contraction. A call whose tiles would leave at
// least half of the CUs idle runs each tile as S = CUs / units parts (see
// ksplit_parts), all tiles' parts in one grid; the parts' fp32 sums are added
// in part order afterwards. 1 = no split.
static int ksplit_for_units(size_t units, int nk) {
  const int cus = device_cus();
  if (units == 0 || units * 2 > (size_t)cus) return 1;
  return ksplit_parts((int)((size_t)cus / units), nk);
}
size_t gemm_ksplit_bytes(bool fwd, fq_shape s, int R_max) {
  const int n_it = (fwd ? s.N : s.K) / BI, ldo = fwd ? s.N : s.K;
  const int nk = ((fwd ? s.K : s.N) + BK - 1) / BK;
  if (R_max <= 0 || n_it <= 0) return 0;
  const int S = ksplit_for_units(rowtile_units(R_max, s.E, n_it), nk);
  return S > 1 ? (size_t)S * (size_t)R_max * (size_t)ldo * 4 : 0;
}

// Row tiles per group of the tile order: with T tiles in flight per XCD,
// about sqrt(T) (a square block), but 1 (i fastest) unless a row tile has at
// least twice that many i tiles; otherwise the tiles in flight already span
// sqrt(T) row tiles or more.
static int rowtile_group(int grid, int S, int n_it) {
  const int tiles = grid / 8 / S;
  int g = 1;
  while ((g + 1) * (g + 1) <= tiles) ++g;
  return n_it >= 2 * g ? g : 1;
}

// launches the row-tile kernel, split along the contraction when the call is
// small enough (then `part` holds the parts' sums and a reduce writes `out`)
template <int MODE, bool ROUTED>
static void launch_rowtile_gemm(GemmArgs &a, int R_max, float *part, hipStream_t st) {
  const size_t units = rowtile_units(R_max, a.E, a.n_it);
  const int nk = ((MODE == FWD ? a.K : a.N) + BK - 1) / BK;
  const int S = part ? ksplit_for_units(units, nk) : 1;
  if (S < 2) {
    const int grid = gemm_grid(units);
    a.gm = ROUTED ? 1 : rowtile_group(grid, 1, a.n_it);
    hipLaunchKernelGGL((k_grouped_gemm<MODE, 0, ROUTED>), dim3(grid), dim3(NT), 0, st, a);
    return;
  }
  a.ksplit = S;
  a.kper = (nk + S - 1) / S;
  a.part = part;
  a.part_rows = R_max;
  const int grid = gemm_grid(units * S);
  a.gm = ROUTED ? 1 : rowtile_group(grid, S, a.n_it);
  hipLaunchKernelGGL((k_grouped_gemm<MODE, 0, ROUTED, true>), dim3(grid), dim3(NT), 0, st, a);
  const int ldo = MODE == FWD ? a.N : a.K;
  const long vecs = (long)R_max * (ldo / 8);
  const int blocks = (int)std::min<long>((vecs + 255) / 256, (long)device_cus() * 8);
  hipLaunchKernelGGL(k_ksplit_reduce, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, part, S,
                     R_max, ldo, a.seg, a.E, a.out);
}

void launch_gemm_fwd(const uint16_t *xq, int R_max, const int32_t *seg, fq_shape s,
                     const uint16_t *wfq, uint16_t *y, float *part, hipStream_t st,
                     const int32_t *xperm, int topk) {
  GemmArgs a{};
  a.p = wfq;
  a.q = xq;
  a.xperm = xperm;
  a.xtopk = FastDiv((uint32_t)(topk > 0 ? topk : 1));
  a.seg = seg;
  a.E = s.E;
  a.N = s.N;
  a.K = s.K;
  a.n_it = s.N / BI;
  a.out = y;
  if (R_max <= 0) return;
  if (xperm) launch_rowtile_gemm<FWD, true>(a, R_max, part, st);
  else launch_rowtile_gemm<FWD, false>(a, R_max, part, st);
}

void launch_gemm_dgrad(const uint16_t *dy, int R_max, const int32_t *seg, fq_shape s,
                       const uint16_t *wfq, uint16_t *dx, float *part, hipStream_t st) {
  GemmArgs a{};
  a.p = wfq;
  a.q = dy;
  a.seg = seg;
  a.E = s.E;
  a.N = s.N;
  a.K = s.K;
  a.n_it = s.K / BI;
  a.out = dx;
  if (R_max <= 0) return;
  launch_rowtile_gemm<DGRAD, false>(a, R_max, part, st);
}

size_t wgrad_max_chunks(int E, int R_max) {
  return (size_t)(R_max + kWgradChunkRows - 1) / kWgradChunkRows + E;
}

template <bool ROUTED>
static void launch_wgrad_kernel(int fmt, dim3 grid, dim3 block, hipStream_t st, const GemmArgs &a) {
  switch (fmt) {
    case FQ_FMT_INT8:
      hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_INT8, ROUTED>), grid, block, 0, st, a);
      break;
    case FQ_FMT_INT4:
      hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_INT4, ROUTED>), grid, block, 0, st, a);
      break;
    case FQ_FMT_FP8_E4M3:
      hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_FP8_E4M3, ROUTED>), grid, block, 0, st, a);
      break;
    default:
      hipLaunchKernelGGL((k_grouped_gemm<WGRAD, FQ_FMT_NVFP4, ROUTED>), grid, block, 0, st, a);
      break;
  }
}

void launch_gemm_wgrad_dscale(const uint16_t *dy, const uint16_t *xq, int R_max, const int32_t *seg,
                              fq_shape s,
                              const uint16_t *w, const fq_weight_q &q, float *dscale, float *dzp,
                              float *part_s, float *part_z, int *chunk_start, hipStream_t st,
                              const int32_t *xperm, int topk) {
  GemmArgs a{};
  a.p = xq;
  a.q = dy;
  a.xperm = xperm;
  a.xtopk = FastDiv((uint32_t)(topk > 0 ? topk : 1));
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
  a.chunk_rows = kWgradChunkRows;
  a.gdiv16 = FastDiv((uint32_t)(q.group / 16));
  a.part_s = part_s;
  a.part_z = part_z;
  a.chunk_start_out = chunk_start;
  dim3 grid(gemm_grid(wgrad_max_chunks(s.E, R_max) * (size_t)a.n_it * (size_t)a.n_jt)), block(NT);
  if (xperm) launch_wgrad_kernel<true>(q.fmt, grid, block, st, a);
  else launch_wgrad_kernel<false>(q.fmt, grid, block, st, a);
  const int G = s.K / q.group;
  hipLaunchKernelGGL(k_reduce_dscale, dim3(ceil_div((long)s.N * G, 256 * 4), s.E), dim3(256), 0, st,
                     part_s, part_z, chunk_start, s.N, s.K, q.group, dscale, dzp);
}

}  // namespace fq
