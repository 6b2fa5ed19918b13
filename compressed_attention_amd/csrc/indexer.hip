// Lightning-indexer scores and top-k selection, flat and two-stage (HISA).
//
// [HISA] my.qihongyi.cn/?p=787, "DeepSeek速度狂飙4倍还不丢精度": section 01
// (flat token indexer over the whole prefix), sections 第一阶段 / 第二阶段
// (block-level filter on pooled representatives, then the token indexer
// inside the chosen blocks) and section 05, Step 3 (same output form).
//
// Score of query q (h_i heads) against key row x:
//     S = sum_h w[q][h] * max(0, q_i[q][h] . x)
// The per-head dot products are a dense contraction and run on MFMA:
//   - flat, bf16, 16 heads: 16 queries x 16 heads = 256 rows per workgroup,
//     entries stream through LDS in tiles of 64 (16x16x32 bf16 MFMA); the
//     ReLU, head weights and head sum happen in the accumulator epilogue;
//   - HISA stage 1 on fp32 block means: 16x16x4 fp32 MFMA (keeps the
//     representatives exact; they are not bf16 values);
//   - HISA stage 2: one wave per (query, chosen block), keys gathered straight
//     from HBM into MFMA operands.
// Other shapes take a plain vector kernel.  Scores are written to a
// workspace and reduced by the LDS radix select of select.h.
#include <algorithm>

#include "append.h"
#include "common.h"
#include "internal.h"
#include "select.h"

namespace hattn {

constexpr int kSelCap = 16384;  // keys per LDS-resident selection
constexpr int kSelNT = 1024;    // threads per selection workgroup

HATTN_DEV float to_f(float x) { return x; }
HATTN_DEV float to_f(uint16_t x) { return bf16_to_f32(x); }

// Decodes a linear block id so that the 8 XCDs each sweep whole key chunks:
// the workgroups resident on one XCD share a chunk and re-read it from L2.
// Four consecutive elements as fp32 (8-byte aligned bf16 / 16-byte aligned
// fp32 source).
HATTN_DEV void load4_f32(const float* p, f32x4_t& v) { v = *reinterpret_cast<const f32x4_t*>(p); }
HATTN_DEV void load4_f32(const uint16_t* p, f32x4_t& v) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  v = f32x4_t{bf16lo(r.x), bf16hi(r.x), bf16lo(r.y), bf16hi(r.y)};
}

// The 8 head weights a lane of the 32x32 score layout needs from one
// query's 16 (16-byte aligned row): heads 4*half..+3 and 8+4*half..+3, in
// that order, as two 16-byte loads; zeros when the query does not exist.
HATTN_DEV void load_head_weights(const float* __restrict__ wrow, bool ok, int half, float (&wv)[8]) {
  f32x4_t lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    lo = *reinterpret_cast<const f32x4_t*>(wrow + 4 * half);
    hi = *reinterpret_cast<const f32x4_t*>(wrow + 8 + 4 * half);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    wv[v] = lo[v];
    wv[4 + v] = hi[v];
  }
}

// Sets this workgroup's share of fill[0, fill_n) to -1: the grid's
// workgroups split the array evenly (16-byte stores; the array is 16-byte
// aligned).
HATTN_DEV void fill_share(int32_t* __restrict__ fill, int64_t fill_n) {
  const int64_t nwg = int64_t(gridDim.x) * gridDim.y * gridDim.z;
  const int64_t wg = (int64_t(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t per = ((fill_n + nwg - 1) / nwg + 3) & ~int64_t(3);
  const int64_t lo = wg * per, hi = imin64(fill_n, lo + per);
  const u32x4_t m1 = {~0u, ~0u, ~0u, ~0u};
  for (int64_t i = lo + 4 * int64_t(threadIdx.x); i < hi; i += 4 * int64_t(blockDim.x)) {
    if (i + 3 < hi) {
      *reinterpret_cast<u32x4_t*>(fill + i) = m1;
    } else {
      for (int64_t j = i; j < hi; ++j) fill[j] = -1;
    }
  }
}

HATTN_DEV bool xcd_decode(int id, int ngroups, int nchunks, int* group, int* chunk) {
  const int xcd = id & 7;
  const int slot = id >> 3;
  *group = slot % ngroups;
  *chunk = (slot / ngroups) * 8 + xcd;
  return *chunk < nchunks;
}
static unsigned xcd_grid(int ngroups, int nchunks) { return unsigned(ngroups * ((nchunks + 7) / 8) * 8); }

// ---------------------------------------------------------------------------
// Flat score, bf16, 16 heads, d_i = 32*KS.
// ---------------------------------------------------------------------------
template <int KS, int NWQ>
__global__ __launch_bounds__(64 * NWQ, KS >= 8 ? 1 : 8 / NWQ) void score_flat_mfma_kernel(const uint16_t* __restrict__ q_i,
                                                                 const uint16_t* __restrict__ k_i,
                                                                 const float* __restrict__ w_i,
                                                                 const int32_t* __restrict__ n_vis, int64_t nq,
                                                                 int64_t n, int64_t ld, float* __restrict__ S,
                                                                 int nqb, int nch, int chunk) {
  constexpr int D = 32 * KS;
  constexpr int TN = 64;
  constexpr int PITCH = D + 8;
  constexpr int NT = 64 * NWQ;
  constexpr int QB = 4 * NWQ;                // queries per workgroup (4 per wave)
  constexpr int PIECES = TN * D / 8 / NT;    // 16-byte pieces per thread per tile
  static_assert(TN * D / 8 % NT == 0, "tile split");
  __shared__ __align__(16) uint16_t kt[2][TN * PITCH];
  __shared__ int s_nv[QB];

  int qb, ch;
  if (!xcd_decode(blockIdx.x, nqb, nch, &qb, &ch)) return;
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t q0 = int64_t(qb) * QB;
  if (threadIdx.x < QB) {
    const int64_t q = q0 + threadIdx.x;
    int v = 0;
    if (q < nq) v = int(imin64(n, imax64(0, n_vis[b * nq + q])));
    s_nv[threadIdx.x] = v;
  }
  __syncthreads();
  int maxv = 0;
#pragma unroll
  for (int i = 0; i < QB; ++i) maxv = max(maxv, s_nv[i]);
  const int64_t e_begin = int64_t(ch) * chunk;
  const int64_t e_end = imin64(e_begin + chunk, maxv);
  if (e_begin >= e_end) return;

  u32x4_t a[4][KS];
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t q = q0 + 4 * wave + mt;
    const bool ok = q < nq;
    const uint16_t* qp = q_i + ((b * nq + (ok ? q : 0)) * 16 + r16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[mt][ks] = ok ? ld16(qp + 32 * ks) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = 0.f;
    if (ok) {
      const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(w_i + (b * nq + q) * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[mt][i] = w4[i];
    }
  }
  // Lane group g stores the scores of query 4*wave + g: its visible count
  // (0 for a query beyond nq) and row pointer, fixed for the whole chunk.
  const int64_t my_q = q0 + 4 * wave + g;
  const int my_nv = my_q < nq ? s_nv[4 * wave + g] : 0;
  float* srow = S + (b * nq + (my_q < nq ? my_q : 0)) * ld;

  // Keys: 32-bit row indices (n < 2^31 is checked on the host).  Rows past
  // the end of the cache are read clamped to the last row; their scores are
  // never stored (every stored key is below n_vis <= n).
  const uint16_t* kb = k_i + b * n * D;
  const int n32 = int(n);
  u32x4_t pre[PIECES];
  auto load = [&](int e0) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int p = threadIdx.x + NT * j;
      const int row = p / (D / 8), col = p % (D / 8);
      const int e = min(e0 + row, n32 - 1);
      pre[j] = ld16(kb + size_t(e) * D + col * 8);
    }
  };
  const int eb = int(e_begin), ee = int(e_end);
  load(eb);
  int buf = 0;
  for (int e0 = eb; e0 < ee; e0 += TN, buf ^= 1) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int p = threadIdx.x + NT * j;
      const int row = p / (D / 8), col = p % (D / 8);
      *reinterpret_cast<u32x4_t*>(&kt[buf][row * PITCH + col * 8]) = pre[j];
    }
    __syncthreads();
    if (e0 + TN < ee) load(e0 + TN);
    f32x4_t acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t bf[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bf[nt] = *reinterpret_cast<const u32x4_t*>(&kt[buf][(16 * nt + r16) * PITCH + 32 * ks + 8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma16x16x32(a[mt][ks], bf[nt], acc[mt][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float v[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], relu_bits(acc[mt][nt][i]), s);
        v[mt] = s;  // this lane group's 4 heads
      }
      // lane group g receives (and stores) the row of query 4*wave + g
      const float mine = sum4_transpose(v[0], v[1], v[2], v[3]);
      const int e = e0 + 16 * nt + r16;
      if (e < my_nv) srow[e] = mine;
    }
  }
}

// ---------------------------------------------------------------------------
// Flat score, bf16, 16 heads, d_i = 16*KS in {32, 64, 128}, on the 32x32x16
// MFMA.  Same workgroup tiling as above (16 queries, 64-key LDS tiles,
// double-buffered), but each wave covers two query pairs: an MFMA row is
// (query of the pair, head), a column a key of a 32-key half tile, so a wave
// issues 32 MFMAs per tile.  Lane l holds, for key l%32, heads
// {4h..4h+3, 8+4h..8+4h+3} (h = l/32) of both queries of the pair: it sums
// its 8 heads per query and one lane swap between the wave halves finishes
// both queries' head sums (lanes < 32: first query, lanes >= 32: second).
//
// The key axis may be virtual: key tile t of the launch is tile t * tstride
// of the cache (tstride = 1: every key).  MODE 0 stores every score at its
// launch position (with tstride > 1 that is a compact, evenly spread sample
// of the row).  MODE 1 keeps only the scores >= the row's threshold thr[row]
// (an order key): a wave owns its four queries for the whole chunk, so it
// packs their candidates (score, key index) into the chunk's span of the
// query's row of S, in increasing key order, with ballot ranks, and stores
// the counts in ccnt[row][chunk] (a count above the span's capacity of
// chunk/2 pairs means some were dropped).  A row whose threshold is key 0
// (take every key) gets plain scores, as in MODE 0.  A nonzero gate skips
// the workgroups none of whose queries has gate[row] != 0.
// ---------------------------------------------------------------------------
template <int KS, int MODE>
__global__ __launch_bounds__(256, 2) void score_flat_mfma32_kernel(const uint16_t* __restrict__ q_i,
                                                                   const uint16_t* __restrict__ k_i,
                                                                   const float* __restrict__ w_i,
                                                                   const int32_t* __restrict__ n_vis, int64_t nq,
                                                                   int64_t n, int64_t ld, float* __restrict__ S,
                                                                   int nqb, int nch, int chunk, int tstride,
                                                                   const uint32_t* __restrict__ thr,
                                                                   int32_t* __restrict__ ccnt,
                                                                   const int32_t* __restrict__ gate) {
  constexpr int D = 16 * KS;
  constexpr int TN = 64;
  constexpr int PITCH = D + 8;
  constexpr int PIECES = TN * D / 8 / 256;  // 16-byte pieces per thread per tile
  static_assert(TN * D / 8 % 256 == 0, "tile split");
  __shared__ __align__(16) uint16_t kt[2][TN * PITCH];
  __shared__ int s_nv[16];

  int qb, ch;
  if (!xcd_decode(blockIdx.x, nqb, nch, &qb, &ch)) return;
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, c32 = lane & 31;
  const int64_t q0 = int64_t(qb) * 16;
  if (threadIdx.x < 16) {
    const int64_t q = q0 + threadIdx.x;
    int v = 0;
    if (q < nq && (!gate || gate[b * nq + q] != 0)) v = int(imin64(n, imax64(0, n_vis[b * nq + q])));
    s_nv[threadIdx.x] = v;
  }
  __syncthreads();
  int maxv = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) maxv = max(maxv, s_nv[i]);
  // launch keys [e_begin, e_end): launch tile t holds cache keys
  // [64 t tstride, 64 t tstride + 64)
  const int64_t e_begin = int64_t(ch) * chunk;
  const int64_t tiles_vis = (int64_t(maxv) + 64LL * tstride - 1) / (64LL * tstride);
  const int64_t e_end = imin64(e_begin + chunk, tiles_vis * 64);
  if (e_begin >= e_end) return;

  // A operand: row c32 of pair p = (query 4*wave + 2p + c32/16, head c32%16)
  u32x4_t a[2][KS];
  // weights of this lane's 8 heads, for both queries of each pair
  float wv[2][2][8];
  int my_nv[2];
  float* srow[2];
  float my_thr[2];     // MODE 1: the query's threshold as a score
  bool my_all[2];      // MODE 1: the query takes every key (plain scores)
  float* creg[2];      // MODE 1: the chunk's span of the query's row
  int my_cap[2];       // MODE 1: candidate pairs the chunk's span holds
  // MODE 1: candidates so far of each pair's first / second query (uniform;
  // two arrays indexed by the unrolled pair only, so they stay in registers)
  int cnt_a[2] = {0, 0}, cnt_b[2] = {0, 0};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    {
      const int64_t q = q0 + 4 * wave + 2 * p + (c32 >> 4);
      const bool ok = q < nq;
      const uint16_t* qp = q_i + ((b * nq + (ok ? q : 0)) * 16 + (c32 & 15)) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[p][ks] = ok ? ld16(qp + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t q = q0 + 4 * wave + 2 * p + j;
      load_head_weights(w_i + (b * nq + (q < nq ? q : 0)) * 16, q < nq, half, wv[p][j]);
    }
    // this lane stores query 4*wave + 2p + half
    const int64_t mq = q0 + 4 * wave + 2 * p + half;
    my_nv[p] = mq < nq ? s_nv[4 * wave + 2 * p + half] : 0;
    srow[p] = S + (b * nq + (mq < nq ? mq : 0)) * ld;
    if (MODE == 1) {
      // key 0 (take all) maps to -inf; any other key to the score it encodes
      const uint32_t t = mq < nq ? thr[b * nq + mq] : 0u;
      my_all[p] = t == 0u;
      my_thr[p] = t == 0u ? INFINITY : key_to_float(t);  // +inf: nothing packed
      creg[p] = srow[p] + e_begin;
      my_cap[p] = int(imin64(chunk, ld - e_begin)) / 2;
    }
  }

  // MODE 1: does any of the wave's queries take every key (uniform)?
  const bool any_all = MODE == 1 && ballot(my_all[0] || my_all[1]) != 0ull;
  // MODE 1: all-ones in the lanes of each pair's second query
  const uint32_t hsel = half ? 0xffffffffu : 0u;

  // Keys: 32-bit row indices (n < 2^31 is checked on the host).  Rows past
  // the end of the cache are read clamped to the last row; their scores are
  // never stored (every stored key is below n_vis <= n).  A launch tile
  // starting at e0 starts at cache key e0 * tstride.
  const uint16_t* kb = k_i + b * n * D;
  const int n32 = int(n);
  const int ts = MODE == 1 ? 1 : tstride;  // the collecting pass reads every key
  u32x4_t pre[PIECES];
  auto load = [&](int e0) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int pc = threadIdx.x + 256 * j;
      const int row = pc / (D / 8), col = pc % (D / 8);
      const int e = min(e0 * ts + row, n32 - 1);
      pre[j] = ld16(kb + size_t(e) * D + col * 8);
    }
  };
  const int eb = int(e_begin), ee = int(e_end);
  load(eb);
  int buf = 0;
  for (int e0 = eb; e0 < ee; e0 += TN, buf ^= 1) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int pc = threadIdx.x + 256 * j;
      const int row = pc / (D / 8), col = pc % (D / 8);
      *reinterpret_cast<u32x4_t*>(&kt[buf][row * PITCH + col * 8]) = pre[j];
    }
    __syncthreads();
    if (e0 + TN < ee) load(e0 + TN);
    f32x16_t acc[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[p][kh][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t bf[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        bf[kh] = *reinterpret_cast<const u32x4_t*>(&kt[buf][(32 * kh + c32) * PITCH + 16 * ks + 8 * half]);
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) acc[p][kh] = mfma32x32x16(a[p][ks], bf[kh], acc[p][kh]);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float s0 = 0.f, s1 = 0.f;  // this lane's 8 heads of the pair's first / second query
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          s0 = fmaf(wv[p][0][v], relu_bits(acc[p][kh][v]), s0);
          s1 = fmaf(wv[p][1][v], relu_bits(acc[p][kh][8 + v]), s1);
        }
        // lanes < 32 receive the first query's total, lanes >= 32 the second's
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int el = e0 + 32 * kh + c32;   // launch position
        if (MODE == 0) {
          const int e = e0 * ts + 32 * kh + c32;  // cache key
          if (e < my_nv[p]) srow[p][el] = tot;
        } else {
          if (any_all && my_all[p] && el < my_nv[p]) srow[p][el] = tot;
          // rows that take every key store plain scores above and pack
          // nothing (their threshold +inf would still admit a score of +inf)
          const bool ok = !my_all[p] && el < my_nv[p] && tot >= my_thr[p];
          const uint64_t m = ballot(ok);
          if (m != 0ull) {
            const uint32_t mlo = uint32_t(m), mhi = uint32_t(m >> 32);
            const int clo = __popc(mlo), chi = __popc(mhi);
            // rank among the set lanes below this one over the whole wave,
            // minus the first query's count in the second query's lanes, plus
            // the lane's query's running count
            const int delta = (cnt_b[p] - clo) - cnt_a[p];  // uniform
            const int slot = int(__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u))) + cnt_a[p] +
                             int(uint32_t(delta) & hsel);
            if (ok && slot < my_cap[p])
              *reinterpret_cast<float2*>(creg[p] + 2 * slot) = make_float2(tot, __int_as_float(el));
            cnt_a[p] += clo;
            cnt_b[p] += chi;
          }
        }
      }
  }
  if (MODE == 1 && c32 == 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t mq = q0 + 4 * wave + 2 * p + half;
      if (mq < nq) ccnt[(b * nq + mq) * nch + ch] = half ? cnt_b[p] : cnt_a[p];
    }
  }
}

// ---------------------------------------------------------------------------
// Flat score for one query per sequence (decode), bf16, 16 heads,
// d_i = 32*KS in {32, 64, 128}: the 16-query tiles above would leave 15 of
// every 16 MFMA rows empty here.  Each wave owns one chunk of launch keys
// of its row and streams it 64 keys at a time, with the arithmetic of the
// decode HISA stage 2 (score_stage2_mfma_kernel), so both give every key the
// same score: 16x16x32 MFMA with A = the query's 16 heads and B = 16 keys,
// lane (g, r) = (l/16, l%16) loading elements 32ks + 8g .. +7 of key r of
// each 16-key subtile (64 contiguous bytes of 16 rows per load
// instruction), the weighted ReLU sum of the lane's 4 heads, and one
// transpose-sum over the 4 lane groups that leaves key 16g + r of the
// 64 in lane l.  No LDS and no barrier; two register buffers keep the next
// 64 keys in flight.  Modes, launch-key mapping (tstride),
// thresholds, chunk spans and counts are those of score_flat_mfma32_kernel;
// a chunk is a wave's, 4 per workgroup.
// ---------------------------------------------------------------------------
template <int KS, int MODE>
__global__ __launch_bounds__(256) void score_flat_dec_kernel(const uint16_t* __restrict__ q_i,
                                                             const uint16_t* __restrict__ k_i,
                                                             const float* __restrict__ w_i,
                                                             const int32_t* __restrict__ n_vis, int64_t n,
                                                             int64_t ld, float* __restrict__ S, int nch, int chunk,
                                                             int tstride, const uint32_t* __restrict__ thr,
                                                             int32_t* __restrict__ ccnt,
                                                             const int32_t* __restrict__ gate) {
  constexpr int D = 32 * KS;
  const int64_t row = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ch = blockIdx.x * 4 + wave;
  if (ch >= nch) return;
  const int g = lane >> 4, r16 = lane & 15;
  int nv = int(imin64(n, imax64(0, n_vis[row])));
  if (gate && gate[row] == 0) nv = 0;
  const int64_t e_begin = int64_t(ch) * chunk;
  const int64_t tiles_vis = (int64_t(nv) + 64LL * tstride - 1) / (64LL * tstride);
  const int64_t e_end = imin64(e_begin + chunk, tiles_vis * 64);
  if (e_begin >= e_end) return;

  u32x4_t a[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) a[ks] = ld16(q_i + (row * 16 + r16) * D + 8 * g + 32 * ks);
  const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(w_i + row * 16 + 4 * g);
  float* srow = S + row * ld;
  float thr_f = INFINITY;
  bool all = true;
  float* creg = nullptr;
  int cap = 0, cnt = 0;
  if (MODE == 1) {
    const uint32_t t = thr[row];
    all = t == 0u;  // take every key: plain scores
    thr_f = all ? INFINITY : key_to_float(t);
    creg = srow + e_begin;
    cap = int(imin64(chunk, ld - e_begin)) / 2;
  }
  const uint16_t* kb = k_i + row * n * D + 8 * g;
  const int n32 = int(n);
  const int ts = MODE == 1 ? 1 : tstride;

  // 64 keys per step; the next step's keys load while this one is scored.
  // Plain loads: an instruction reads 64 bytes of each of 16 rows, half of
  // a 128-byte line, and L2 serves the other half to the next instruction
  // (non-temporal loads here measured 1.45x slower).
  auto ldk = [&](int64_t e0, u32x4_t (&dst)[4][KS]) {
    const int64_t c0 = (e0 / 64) * 64 * ts;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int key = int(imin64(c0 + 16 * nt + r16, n32 - 1));  // rows past the cache are read clamped, never stored
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[nt][ks] = ld16(kb + size_t(key) * D + 32 * ks);
    }
  };
  auto step = [&](int64_t e0, const u32x4_t (&bf)[4][KS]) {
    const int64_t c0 = (e0 / 64) * 64 * ts;  // launch keys e0 .. e0 + 63 are cache keys c0 .. c0 + 63
    float v[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(a[ks], bf[nt][ks], acc);
      float sv = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) sv = fmaf(wv[i], relu_bits(acc[i]), sv);
      v[nt] = sv;  // this lane group's 4 heads
    }
    const float x = sum4_transpose(v[0], v[1], v[2], v[3]);  // key 16g + r16 = lane of the 64
    const int el = int(e0) + lane;                             // its launch position
    const bool vis = c0 + lane < nv;                           // its cache key is visible
    if (MODE == 0 || all) {
      if (vis) srow[el] = x;
    } else {
      const bool ok = vis && x >= thr_f;
      const uint64_t m = ballot(ok);
      if (m != 0ull) {
        const int slot = cnt + mbcnt(m);  // lanes in key order
        if (ok && slot < cap) *reinterpret_cast<float2*>(creg + 2 * slot) = make_float2(x, __int_as_float(el));
        cnt += __popcll(m);
      }
    }
  };
  u32x4_t b0[4][KS], b1[4][KS];
  ldk(e_begin, b0);
  for (int64_t e0 = e_begin; e0 < e_end; e0 += 128) {
    const bool more = e0 + 64 < e_end;
    if (more) ldk(e0 + 64, b1);
    step(e0, b0);
    if (!more) break;
    if (e0 + 128 < e_end) ldk(e0 + 128, b0);
    step(e0 + 64, b1);
  }
  if (MODE == 1 && lane == 0) ccnt[row * nch + ch] = cnt;
}

// ---------------------------------------------------------------------------
// HISA stage 1 score on fp32 block representatives, 16 heads, d_i = 16*KQ.
// A workgroup owns QPW queries (1 or 4) and one LDS tile of 64 block means;
// its 4 waves cover the (query, 16-block subtile) pairs: with 4 queries each
// wave takes one query and all four subtiles, with one query (decode) each
// wave takes one subtile.
// ---------------------------------------------------------------------------
template <typename TQ, int KQ, int QPW>
__global__ __launch_bounds__(256, 2) void score_stage1_kernel(const TQ* __restrict__ q_i,
                                                              const float* __restrict__ reps,
                                                              const float* __restrict__ w_i,
                                                              const int32_t* __restrict__ n_vis, int64_t nq,
                                                              int64_t n, int B, int64_t nb, int64_t ld,
                                                              float* __restrict__ S1, int nqg, int nch, int chunk,
                                                              int32_t* __restrict__ fill, int64_t fill_n) {
  // Clears the block-major chooser lists (the block select of the same call
  // fills them), every workgroup its share.
  if (fill) fill_share(fill, fill_n);
  constexpr int D = 16 * KQ;
  constexpr int TB = 64;
  constexpr int PITCH = D + 4;
  constexpr int PIECES = TB * D / 4 / 256;
  constexpr int NTW = 4 / (4 / QPW);  // subtiles per wave: 4 (QPW=4) or 1 (QPW=1)
  __shared__ __align__(16) float rt[TB * PITCH];
  __shared__ int s_nb[QPW];

  int qg, ch;
  if (!xcd_decode(blockIdx.x, nqg, nch, &qg, &ch)) return;
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int qw = QPW == 4 ? wave : 0;           // this wave's query within the group
  const int nt0 = QPW == 4 ? 0 : wave;          // first subtile of this wave
  const int64_t q = int64_t(qg) * QPW + qw;
  const int64_t j_begin = int64_t(ch) * chunk;
  const float* rb = reps + b * nb * D;
  // The first tile of block means goes out before the visible counts are
  // known (it is needed whenever this workgroup has any work).
  auto load_tile = [&](int64_t j0, u32x4_t(&v)[PIECES]) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int p = threadIdx.x + 256 * u;
      const int64_t j = j0 + p / (D / 4);
      v[u] = j < nb ? ld16_nt(rb + j * D + (p % (D / 4)) * 4) : u32x4_t{0, 0, 0, 0};
    }
  };
  u32x4_t v[PIECES];
  load_tile(j_begin, v);
  const bool ok = q < nq;
  f32x4_t a[KQ];
  float wv[4];
  {
    // 4 consecutive elements per (lane, kq): one 8-byte (bf16) or 16-byte
    // (fp32) load each, not four scalar ones
    const TQ* qp = q_i + ((b * nq + (ok ? q : 0)) * 16 + r16) * D + 4 * g;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) load4_f32(qp + 16 * kq, a[kq]);
    if (!ok)
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) a[kq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = 0.f;
    if (ok) {
      const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(w_i + (b * nq + q) * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = w4[i];
    }
  }
  if (threadIdx.x < QPW) {
    const int64_t qq = int64_t(qg) * QPW + threadIdx.x;
    int nbq = 0;
    if (qq < nq) {
      const int64_t nvq = imin64(n, imax64(0, n_vis[b * nq + qq]));
      nbq = int(idiv(nvq + B - 1, B));
    }
    s_nb[threadIdx.x] = nbq;
  }
  __syncthreads();
  int maxb = 0;
#pragma unroll
  for (int i = 0; i < QPW; ++i) maxb = max(maxb, s_nb[i]);
  const int64_t j_end = imin64(j_begin + chunk, maxb);
  if (j_begin >= j_end) return;
  const int my_nb = s_nb[qw];
  for (int64_t j0 = j_begin; j0 < j_end; j0 += TB) {
    __syncthreads();
    if (j0 != j_begin) load_tile(j0, v);
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int p = threadIdx.x + 256 * u;
      *reinterpret_cast<u32x4_t*>(&rt[(p / (D / 4)) * PITCH + (p % (D / 4)) * 4]) = v[u];
    }
    __syncthreads();
    if (!ok || j0 >= my_nb) continue;
    f32x4_t acc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int nt = nt0 + t;
        const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&rt[(16 * nt + r16) * PITCH + 16 * kq + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kq][j], bv[j], acc[t], 0, 0, 0);
      }
    }
    float hs[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wv[i], relu_bits(acc[t][i]), s);
      hs[t] = s;  // this lane group's 4 heads
    }
    if constexpr (NTW == 4) {
      // lane group g receives (and stores) subtile nt0 + g
      const float s = sum4_transpose(hs[0], hs[1], hs[2], hs[3]);
      const int64_t j = j0 + 16 * (nt0 + g) + r16;
      if (j < my_nb) S1[(b * nq + q) * ld + j] = s;
    } else {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float s = sum_groups(hs[t]);
        const int64_t j = j0 + 16 * (nt0 + t) + r16;
        if (g == 0 && j < my_nb) S1[(b * nq + q) * ld + j] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// HISA stage 1 on the bf16 MFMA for many queries (bf16 queries, 16 heads,
// d_i = 16*KS in {32, 64, 128}).  Every fp32 block mean is split exactly into
// three bf16 parts, hi + mid + lo (each captures the next 8 significant bits
// of the remaining value), while its tile is staged in LDS; each MFMA step
// then accumulates q.hi + q.mid + q.lo.  Each product of two bf16 values is
// exact in fp32, so the scores carry the fp32 block means in full; the
// tiling, head reduction and layout are those of the 32x32x16 flat score
// kernel (16 queries per workgroup, 64 blocks per tile).  Candidate blocks of
// a query are those whose first entry is visible.
// ---------------------------------------------------------------------------
HATTN_DEV void split3_bf16(float x, uint16_t* hi, uint16_t* mid, uint16_t* lo) {
  const uint16_t h = f32_to_bf16(x);
  const float r1 = x - bf16_to_f32(h);
  const uint16_t m = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(m);
  *hi = h;
  *mid = m;
  *lo = f32_to_bf16(r2);
}

template <int KS>
__global__ __launch_bounds__(256, 2) void score_stage1_x3_kernel(const uint16_t* __restrict__ q_i,
                                                                 const float* __restrict__ reps,
                                                                 const float* __restrict__ w_i,
                                                                 const int32_t* __restrict__ n_vis, int64_t nq,
                                                                 int64_t n, int B, int64_t nb, int64_t ld,
                                                                 float* __restrict__ S1, int nqb, int nch, int chunk,
                                                                 int32_t* __restrict__ fill, int64_t fill_n) {
  if (fill) fill_share(fill, fill_n);
  constexpr int D = 16 * KS;
  constexpr int TN = 64;
  constexpr int PITCH = D + 8;
  constexpr int PIECES = TN * D / 4 / 256;  // 16-byte (4 x fp32) pieces per thread per tile
  static_assert(TN * D / 4 % 256 == 0, "tile split");
  __shared__ __align__(16) uint16_t kt[3][TN * PITCH];
  __shared__ int s_nb[16];

  int qb, ch;
  if (!xcd_decode(blockIdx.x, nqb, nch, &qb, &ch)) return;
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, c32 = lane & 31;
  const int64_t q0 = int64_t(qb) * 16;
  if (threadIdx.x < 16) {
    const int64_t q = q0 + threadIdx.x;
    int v = 0;
    if (q < nq) {
      const int64_t nvq = imin64(n, imax64(0, n_vis[b * nq + q]));
      v = int(idiv(nvq + B - 1, B));
    }
    s_nb[threadIdx.x] = v;
  }
  __syncthreads();
  int maxb = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) maxb = max(maxb, s_nb[i]);
  const int jb = ch * chunk;
  const int je = min(jb + chunk, maxb);
  if (jb >= je) return;

  u32x4_t a[2][KS];
  float wv[2][2][8];
  int my_nb[2];
  float* srow[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    {
      const int64_t q = q0 + 4 * wave + 2 * p + (c32 >> 4);
      const bool ok = q < nq;
      const uint16_t* qp = q_i + ((b * nq + (ok ? q : 0)) * 16 + (c32 & 15)) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[p][ks] = ok ? ld16(qp + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t q = q0 + 4 * wave + 2 * p + j;
      load_head_weights(w_i + (b * nq + (q < nq ? q : 0)) * 16, q < nq, half, wv[p][j]);
    }
    const int64_t mq = q0 + 4 * wave + 2 * p + half;
    my_nb[p] = mq < nq ? s_nb[4 * wave + 2 * p + half] : 0;
    srow[p] = S1 + (b * nq + (mq < nq ? mq : 0)) * ld;
  }

  // Block means: 32-bit row indices; rows past nb are read clamped (their
  // scores are never stored: every stored block is below its query's count).
  const float* rb = reps + b * nb * D;
  const int nb32 = int(nb);
  u32x4_t pre[PIECES];
  auto load = [&](int j0) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pc = threadIdx.x + 256 * u;
      const int row = pc / (D / 4), col = pc % (D / 4);
      const int j = min(j0 + row, nb32 - 1);
      pre[u] = ld16(rb + size_t(j) * D + col * 4);
    }
  };
  load(jb);
  for (int j0 = jb; j0 < je; j0 += TN) {
    __syncthreads();  // the previous tile's readers are done
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pc = threadIdx.x + 256 * u;
      const int row = pc / (D / 4), col = pc % (D / 4);
      uint16_t hv[4], mv[4], lv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split3_bf16(__uint_as_float(pre[u][e]), &hv[e], &mv[e], &lv[e]);
      const int off = row * PITCH + col * 4;
      *reinterpret_cast<u32x2_t*>(&kt[0][off]) = u32x2_t{uint32_t(hv[0]) | (uint32_t(hv[1]) << 16),
                                                         uint32_t(hv[2]) | (uint32_t(hv[3]) << 16)};
      *reinterpret_cast<u32x2_t*>(&kt[1][off]) = u32x2_t{uint32_t(mv[0]) | (uint32_t(mv[1]) << 16),
                                                         uint32_t(mv[2]) | (uint32_t(mv[3]) << 16)};
      *reinterpret_cast<u32x2_t*>(&kt[2][off]) = u32x2_t{uint32_t(lv[0]) | (uint32_t(lv[1]) << 16),
                                                         uint32_t(lv[2]) | (uint32_t(lv[3]) << 16)};
    }
    __syncthreads();
    if (j0 + TN < je) load(j0 + TN);
    f32x16_t acc[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[p][kh][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int part = 0; part < 3; ++part) {
        u32x4_t bf[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          bf[kh] = *reinterpret_cast<const u32x4_t*>(&kt[part][(32 * kh + c32) * PITCH + 16 * ks + 8 * half]);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) acc[p][kh] = mfma32x32x16(a[p][ks], bf[kh], acc[p][kh]);
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          s0 = fmaf(wv[p][0][v], relu_bits(acc[p][kh][v]), s0);
          s1 = fmaf(wv[p][1][v], relu_bits(acc[p][kh][8 + v]), s1);
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int j = j0 + 32 * kh + c32;
        if (j < my_nb[p]) srow[p][j] = tot;
      }
  }
}

// ---------------------------------------------------------------------------
// Decode front: HISA stage 1 for one query per sequence (the CSA layer) in
// the same launch as the step's cache maintenance (the cache-maintenance
// roles of append_kernel).  Grid (nch_grid + nroles, bt), 256 threads:
//   x < nch_grid  stage 1 over 64 block means, as score_stage1_kernel with
//                 one query; the visible count comes from q_pos and the CSA
//                 geometry.  When the new token completes entry e, the
//                 workgroup holding block e / B recomputes that block's mean
//                 from K_I (entries past the last one count as zero), scores
//                 it and writes it back to reps.
//   x >= nch_grid role 0: the CSA entry the token completes + its visible
//                 count; role 1: the same for the HCA layer.
// The same arithmetic as hattn_decode_append + the stage-1 kernel; one
// kernel boundary less on the decode critical path.
// ---------------------------------------------------------------------------
template <int KQ>
__global__ __launch_bounds__(256, 2) void decode_front_kernel(const uint16_t* __restrict__ q_i,
                                                              float* __restrict__ reps,
                                                              const float* __restrict__ w_i,
                                                              const int32_t* __restrict__ q_pos, int B, int64_t nb,
                                                              int64_t ld, float* __restrict__ S1, int nch,
                                                              int nch_grid, AppendK la, AppendK lb, int nroles) {
  constexpr int D = 16 * KQ;
  constexpr int TB = 64;
  constexpr int PITCH = D + 4;
  constexpr int PIECES = TB * D / 4 / 256;
  constexpr int V = 8;  // bf16 per 16-byte slot
  __shared__ __align__(16) float rt[TB * PITCH];
  __shared__ float red[2];
  const int64_t b = blockIdx.y;
  if (int(blockIdx.x) >= nch_grid) {
    const int role = int(blockIdx.x) - nch_grid;
    const int64_t p = q_pos[b];
    if (role == 0) append_entry_body<uint16_t, 256>(la, b, p, rt, red);
    else if (role == 1 && nroles > 1) append_entry_body<uint16_t, 256>(lb, b, p, rt, red);
    return;
  }
  int qg, ch;
  if (!xcd_decode(blockIdx.x, 1, nch, &qg, &ch)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t n = la.N;
  const int64_t j0 = int64_t(ch) * TB;
  const float* rb = reps + b * nb * D;
  u32x4_t v[PIECES];
#pragma unroll
  for (int u = 0; u < PIECES; ++u) {
    const int pp = threadIdx.x + 256 * u;
    const int64_t j = j0 + pp / (D / 4);
    v[u] = j < nb ? ld16_nt(rb + j * D + (pp % (D / 4)) * 4) : u32x4_t{0, 0, 0, 0};
  }
  f32x4_t a[KQ];
  {
    const uint16_t* qp = q_i + (b * 16 + r16) * D + 4 * g;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) load4_f32(qp + 16 * kq, a[kq]);
  }
  const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(w_i + b * 16 + 4 * g);
  const int64_t p = q_pos[b];
  int64_t nv;
  const int64_t e = append_entry_of(la, p, &nv);
  const int my_nb = int(idiv(nv + B - 1, B));
  if (j0 >= my_nb) return;
  // The block holding a newly completed entry: its mean, from K_I.
  const int64_t jl = e >= 0 ? idiv(e, B) : -1;
  const bool fresh = jl >= j0 && jl < j0 + TB;  // uniform
  float mean_c = 0.f;
  if (fresh) {
    const int slots = D / V;
    const int RG = 256 / slots;
    const int cs = threadIdx.x % slots, rg = threadIdx.x / slots;
    const int64_t i0 = jl * B;
    const int cnt = int(imin64(n, i0 + B) - i0);
    float* part = rt;  // [RG][D], before the tile lands
    if (rg < RG) {
      const uint16_t* kb = static_cast<const uint16_t*>(la.k_i) + (b * n + i0) * D + cs * V;
      u32x4_t first[kAppUNR];
      append_first(kb, D, cnt, rg, first, RG);
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      append_rows(kb, D, cnt, rg, RG, first, [](int) { return 1.f; }, acc);
#pragma unroll
      for (int i = 0; i < V; ++i) part[rg * D + cs * V + i] = acc[i];
    }
    __syncthreads();
    if (threadIdx.x < D) {
      float r = 0.f;
      for (int gg = 0; gg < RG; ++gg) r += part[gg * D + threadIdx.x];
      mean_c = r * (1.f / float(B));
      reps[(b * nb + jl) * D + threadIdx.x] = mean_c;
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < PIECES; ++u) {
    const int pp = threadIdx.x + 256 * u;
    *reinterpret_cast<u32x4_t*>(&rt[(pp / (D / 4)) * PITCH + (pp % (D / 4)) * 4]) = v[u];
  }
  if (fresh) {
    __syncthreads();  // the stale row has landed; replace it
    if (threadIdx.x < D) rt[(jl - j0) * PITCH + threadIdx.x] = mean_c;
  }
  __syncthreads();
  // one 16-block subtile per wave (the one-query layout of stage 1)
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq) {
    const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&rt[(16 * wave + r16) * PITCH + 16 * kq + 4 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kq][j], bv[j], acc, 0, 0, 0);
  }
  float hsum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) hsum = fmaf(wv[i], relu_bits(acc[i]), hsum);
  const float sc = sum_groups(hsum);
  const int64_t j = j0 + 16 * wave + r16;
  if (g == 0 && j < my_nb) S1[b * ld + j] = sc;
}

// ---------------------------------------------------------------------------
// HISA stage 2 score, bf16, 16 heads: one wave per (query, chosen block,
// 64-key tile group): workgroup x = slot * halves + h takes the block's
// tiles h, h + halves, ...  (two workgroups per 128-key block: twice the
// waves in flight of one wave per block, with half the registers each).
// Candidate position j = slot*B + offset; visible candidates form a prefix.
// ---------------------------------------------------------------------------
template <int KS>
__global__ __launch_bounds__(64) void score_stage2_mfma_kernel(
    const uint16_t* __restrict__ q_i, const uint16_t* __restrict__ k_i, const float* __restrict__ w_i,
    const int32_t* __restrict__ n_vis, const int32_t* __restrict__ blk, int64_t nq, int64_t n, int B, int m,
    int64_t ld, float* __restrict__ S2, int halves) {
  constexpr int D = 32 * KS;
  const int64_t row = blockIdx.y;
  const int slot = int(blockIdx.x) / halves, h = int(blockIdx.x) - slot * halves;
  const int64_t b = idiv(row, nq);
  const int lane = threadIdx.x;
  const int g = lane >> 4, r16 = lane & 15;
  // Every load is issued before any branch: query, weights, block id and
  // visible count together, then the first tile's keys as soon as the block
  // id arrives (rows past the cache end, or of an empty slot, read a valid
  // row and are never stored).
  u32x4_t a[KS];
  const uint16_t* qp = q_i + (row * 16 + r16) * D + 8 * g;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) a[ks] = ld16(qp + 32 * ks);
  const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(w_i + row * 16 + 4 * g);
  const int bid = blk[row * m + slot];
  const int64_t nv = imin64(n, imax64(0, n_vis[row]));
  const int64_t e_begin = int64_t(max(bid, 0)) * B;
  const int64_t e_end = bid < 0 ? e_begin : imin64(e_begin + B, nv);
  const uint16_t* kb = k_i + b * n * D + 8 * g;
  float* out = S2 + row * ld + int64_t(slot) * B;
  u32x4_t bf[4][KS];
  auto load_keys = [&](int64_t e0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t e = imax64(0, imin64(e0 + 16 * nt + r16, n - 1));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bf[nt][ks] = ld16_nt(kb + e * D + 32 * ks);
    }
  };
  auto tile = [&](int64_t e0) {
    float v[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(a[ks], bf[nt][ks], acc);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(wv[i], relu_bits(acc[i]), s);
      v[nt] = s;  // this lane group's 4 heads
    }
    // lane group g receives (and stores) key tile g
    const float s = sum4_transpose(v[0], v[1], v[2], v[3]);
    const int64_t e = e0 + 16 * g + r16;
    if (e < e_end) out[e - e_begin] = s;
  };
  const int64_t first = e_begin + 64 * h;
  load_keys(first);
  __builtin_amdgcn_sched_barrier(0);
  for (int64_t e0 = first; e0 < e_end; e0 += 64 * halves) {
    if (e0 != first) {
      load_keys(e0);
      __builtin_amdgcn_sched_barrier(0);
    }
    tile(e0);
  }
}

// ---------------------------------------------------------------------------
// HISA stage 2, block-major (bf16, 16 heads, d_i = 16*KS, B <= 128): used
// when many queries choose each block.  The block-select kernel wrote, for
// every query q of sequence b that chose block blk, the slot it chose into
// list[b][blk][q] (-1 elsewhere).  A workgroup reads its block's column,
// packs the choosers into an LDS list in query order, loads block blk's keys into LDS once and scores them for groups
// of 16 choosers (32x32x16 MFMA, the flat kernel's per-wave layout: query
// pairs, 32-key column tiles).  Workgroups of one block take every
// nslice-th group, so a block chosen by many queries is spread over nslice
// of them.  Scores land where the per-slot kernel puts them:
// S2[row][slot*B + j] for the visible entries j of the block.
// ---------------------------------------------------------------------------
template <int KS>
__global__ __launch_bounds__(256, 4) void score_stage2_bm_kernel(const uint16_t* __restrict__ q_i,
                                                                 const uint16_t* __restrict__ k_i,
                                                                 const float* __restrict__ w_i,
                                                                 const int32_t* __restrict__ n_vis,
                                                                 const int32_t* __restrict__ list, int64_t nq,
                                                                 int64_t n, int B, int m, int64_t nb, int64_t ld2,
                                                                 float* __restrict__ S2, int nslice) {
  constexpr int D = 16 * KS;
  constexpr int BMAX = 128;
  constexpr int PITCH = D + 8;
  constexpr int QMAX = 4096;  // queries per sequence (checked on the host)
  __shared__ __align__(16) uint16_t kt[BMAX * PITCH];
  extern __shared__ int32_t lst[];  // [nq]: row * m + slot of the block's choosers
  constexpr int CPT = QMAX / 256;   // column steps of 256 queries
  static_assert(CPT * 4 == kWave, "one ballot mask per lane");
  __shared__ uint64_t cmask[CPT * 4];  // chooser ballot of step j, wave w at [4 * j + w]
  const int slice = blockIdx.x;
  const int64_t blkid = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, c32 = lane & 31;

  // The block's column of chooser slots and its keys: every load in flight
  // at once (both loops have compile-time trip counts and unroll).
  const int32_t* colp = list + (b * nb + blkid) * nq;
  int cv[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = threadIdx.x + 256 * j;
    cv[j] = q < nq ? colp[q] : -1;
  }
  // (rows past the cache end read clamped; never stored)
  const uint16_t* kb = k_i + b * n * D;
  const int64_t e_blk = blkid * B;
  constexpr int KPT = BMAX * (D / 8) / 256;  // 16-byte pieces per thread
  u32x4_t kp[KPT];
#pragma unroll
  for (int it = 0; it < KPT; ++it) {
    const int pc = threadIdx.x + 256 * it;
    const int row = pc / (D / 8), col = pc % (D / 8);
    const int64_t e = imin64(e_blk + imin64(row, B - 1), n - 1);
    kp[it] = ld16(kb + e * D + col * 8);
  }
  // Pack the choosers in query order: every workgroup of the block builds
  // the same list (its slices partition it by group), so the order must not
  // depend on timing.  Ballot masks go to LDS; each wave scans the 64 counts
  // (one per lane) for its bases.
  uint64_t mks[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    mks[j] = ballot(cv[j] >= 0);
    if (lane == 0) cmask[4 * j + wave] = mks[j];
  }
#pragma unroll
  for (int it = 0; it < KPT; ++it) {
    const int pc = threadIdx.x + 256 * it;
    const int row = pc / (D / 8), col = pc % (D / 8);
    if (row < B) *reinterpret_cast<u32x4_t*>(&kt[row * PITCH + col * 8]) = kp[it];
  }
  __syncthreads();
  const uint32_t pcnt = uint32_t(__popcll(cmask[lane]));
  const uint32_t pincl = wave_prefix_incl(pcnt);
  const int c = __builtin_amdgcn_readlane(int(pincl), 63);
  const int pexcl = int(pincl - pcnt);
  const int wv4 = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (mks[j]) {
      const int base = __builtin_amdgcn_readlane(pexcl, 4 * j + wv4);
      if (cv[j] >= 0) lst[base + mbcnt(mks[j])] = int32_t((b * nq + threadIdx.x + 256 * j) * m + cv[j]);
    }
  }
  __syncthreads();
  const int ngroups = (c + 15) / 16;
  if (slice >= ngroups) return;
  // this wave's four entries of group gi (entries 16*gi + 4*wave + 0..3;
  // pair p holds entries 2p, 2p+1), read one group ahead
  auto load_entries = [&](int gi, int (&pk)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ent = 16 * gi + 4 * wave + i;
      pk[i] = gi < ngroups && ent < c ? lst[ent] : -1;
    }
  };
  int pk_next[4];
  load_entries(slice, pk_next);

  for (int gi = slice; gi < ngroups; gi += nslice) {
    int pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pk_next[i];
    load_entries(gi + nslice, pk_next);
    // One query pair at a time: half the registers of both pairs at once
    // (four resident workgroups instead of two), each pair reading the key
    // tile from LDS on its own.
#pragma unroll 1
    for (int p = 0; p < 2; ++p) {
      const int pk0 = p ? pk[2] : pk[0], pk1 = p ? pk[3] : pk[1];
      const int r0 = pk0 < 0 ? -1 : pk0 / m, r1 = pk1 < 0 ? -1 : pk1 / m;
      u32x4_t a[KS];
      {
        const int r = (c32 >> 4) ? r1 : r0;
        const uint16_t* qp = q_i + (int64_t(r < 0 ? 0 : r) * 16 + (c32 & 15)) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = r >= 0 ? ld16(qp + 16 * ks) : u32x4_t{0, 0, 0, 0};
      }
      float wv[2][8];
      load_head_weights(w_i + int64_t(r0 < 0 ? 0 : r0) * 16, r0 >= 0, half, wv[0]);
      load_head_weights(w_i + int64_t(r1 < 0 ? 0 : r1) * 16, r1 >= 0, half, wv[1]);
      // this lane stores entry 2p + half of the pair
      const int r = half ? r1 : r0;
      const int pkh = half ? pk1 : pk0;
      const int slot = pkh < 0 ? 0 : pkh % m;
      const int64_t nvr = r >= 0 ? imin64(n, imax64(0, n_vis[r])) : 0;
      const int my_nv = int(imax64(0, imin64(int64_t(B), nvr - e_blk)));  // visible entries of this block
      float* srow = S2 + int64_t(r < 0 ? 0 : r) * ld2 + int64_t(slot) * B;
      for (int t0 = 0; t0 < B; t0 += 64) {
        f32x16_t acc[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[kh][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4_t bf[2];
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
            bf[kh] = *reinterpret_cast<const u32x4_t*>(&kt[(t0 + 32 * kh + c32) * PITCH + 16 * ks + 8 * half]);
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) acc[kh] = mfma32x32x16(a[ks], bf[kh], acc[kh]);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            s0 = fmaf(wv[0][v], relu_bits(acc[kh][v]), s0);
            s1 = fmaf(wv[1][v], relu_bits(acc[kh][8 + v]), s1);
          }
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
          const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          const int jloc = t0 + 32 * kh + c32;
          if (jloc < my_nv) srow[jloc] = tot;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Vector fallback for any dtype / head count / dim.  MODE 0: flat entries;
// MODE 1: stage-1 block representatives (fp32 keys); MODE 2: stage-2
// entries inside the chosen blocks.  One query per workgroup row of the grid.
// ---------------------------------------------------------------------------
template <typename TQ, typename TK, int MODE>
__global__ __launch_bounds__(256) void score_valu_kernel(const TQ* __restrict__ q_i, const TK* __restrict__ keys,
                                                         const float* __restrict__ w_i,
                                                         const int32_t* __restrict__ n_vis,
                                                         const int32_t* __restrict__ blk, int64_t nq, int h_i,
                                                         int d_i, int64_t n, int64_t keys_per_seq, int B, int m,
                                                         int64_t ld, float* __restrict__ S) {
  extern __shared__ float qs[];  // [h_i][d_i] then [h_i] weights
  const int64_t row = blockIdx.y;
  const int64_t b = idiv(row, nq);
  for (int i = threadIdx.x; i < h_i * d_i; i += blockDim.x) qs[i] = to_f(q_i[row * h_i * d_i + i]);
  for (int i = threadIdx.x; i < h_i; i += blockDim.x) qs[h_i * d_i + i] = w_i[row * h_i + i];
  __syncthreads();
  const int64_t nv = imin64(n, imax64(0, n_vis[row]));
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t krow;
  if (MODE == 0) {
    if (j >= nv) return;
    krow = j;
  } else if (MODE == 1) {
    if (j >= idiv(nv + B - 1, B)) return;
    krow = j;
  } else {
    const int64_t slot = j / B;
    if (slot >= m) return;
    const int bid = blk[row * m + slot];
    const int64_t e = int64_t(bid) * B + (j % B);
    if (bid < 0 || e >= nv) return;
    krow = e;
  }
  const TK* kp = keys + (b * keys_per_seq + krow) * d_i;
  float s = 0.f;
  for (int h = 0; h < h_i; ++h) {
    float dot = 0.f;
    for (int c = 0; c < d_i; ++c) dot = fmaf(qs[h * d_i + c], to_f(kp[c]), dot);
    s = fmaf(qs[h_i * d_i + h], fmaxf(dot, 0.f), s);
  }
  S[row * ld + j] = s;
}

// ---------------------------------------------------------------------------
// Selection kernels.
// ---------------------------------------------------------------------------
// Number of valid candidates of a row.  MODE 0: visible entries; MODE 1:
// blocks whose first entry is visible; MODE 2 / 3: visible entries inside
// the chosen blocks (a prefix of slot space, see the stage-2 kernel), summed
// by every wave on its own from the row's block ids (no barrier).  MODE 2
// keeps the block ids in LDS (m <= kSelNT), MODE 3 reads them from global
// memory.
template <int MODE>
HATTN_DEV int row_valid_count(const int32_t* n_vis, const int32_t* bids, int64_t row, int64_t n, int B, int m) {
  const int64_t nv = imin64(n, imax64(0, n_vis[row]));
  if (MODE == 0) return int(nv);
  if (MODE == 1) return int(idiv(nv + B - 1, B));
  uint32_t c = 0;
  for (int s = threadIdx.x & (kWave - 1); s < m; s += kWave) {
    const int bid = bids[s];
    if (bid >= 0) c += uint32_t(imax64(0, imin64(B, nv - int64_t(bid) * B)));
  }
  return int(wave_total(c));
}

// Flat rows on 512 threads ask for 8 waves per SIMD (four workgroups per
// CU, so 1,024 rows run in one round): the compiler then keeps 78 SGPRs
// and moves the rest into VGPR lanes.  Measured on the prefill chunk's
// selection (1,024 rows): 23.3 -> 21.1 us.  Token rows would spill VGPRs to
// memory at that bound (no gain at 128K), and the few-row decode selections
// gain nothing from occupancy.
template <int MODE, int NT>
__global__ __launch_bounds__(NT, MODE == 0 && NT == 512 ? 8 : 1) void select_rows_kernel(const float* __restrict__ S, int64_t ld,
                                                             const int32_t* __restrict__ n_vis,
                                                             const int32_t* __restrict__ blk, int64_t n, int B, int m,
                                                             int k, int32_t* __restrict__ idx,
                                                             float* __restrict__ score_out,
                                                             int32_t* __restrict__ inv_list, int64_t nq,
                                                             int64_t nb) {
  __shared__ SelectShared<NT> sh;
  constexpr bool TOK = MODE >= 2;                 // token rows (stage 2)
  constexpr int CAP = kSelIT * NT;                // keys a row may hold
  __shared__ int32_t bsh[MODE == 2 ? NT : 1];  // chosen block ids
  const int64_t row = blockIdx.x;
  const int32_t* brow = blk + row * m;
  // Block and token rows: the scores of every slot a row can have are loaded
  // at once, before the valid count is known (slots past it are masked
  // below), so the two loads overlap.  Flat rows load only what is visible.
  float v[kSelIT];
  SelSeg sg;
  if (MODE != 0) {
    const int cap = TOK ? min(CAP, m * B) : int(imin64(CAP, idiv(n + B - 1, B)));
    sg = wave_segment<NT>(cap);
    seg_load_scores(S + row * ld, sg, v);
  }
  if (MODE == 2)
    for (int s = threadIdx.x; s < m; s += NT) bsh[s] = brow[s];
  select_clear(sh);
  __syncthreads();
  const int nvalid = min(CAP, row_valid_count<TOK ? 2 : MODE>(n_vis, MODE == 2 ? bsh : brow, row, n, B, m));
  if (MODE == 0) {
    sg = wave_segment<NT>(nvalid);
    seg_load_scores(S + row * ld, sg, v);
  }
  uint32_t kc[kSelIT];
  seg_keys_masked(v, sg, nvalid, kc);
  const bool pow2 = (B & (B - 1)) == 0;
  const int lgB = __builtin_ctz(unsigned(B));
  // Token rows: candidate i of slot s = i / B is entry blk[s] * B + i - s * B,
  // i.e. i + dl[it].  The block ids are read here, so their LDS round trips
  // overlap the threshold search instead of preceding each emitted store.
  int dl[TOK ? kSelIT : 1];
  if (TOK) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int it = 0; it < kSelIT; ++it) {
      const int i = sg.p0 + it * kWave + lane;
      const int sl = pow2 ? i >> lgB : i / B;
      dl[it] = it < sg.iters && i < sg.p1 ? ((MODE == 2 ? bsh[sl] : brow[sl]) - sl) * B : 0;
    }
  }
  const SelThr st = radix_threshold<NT, kSelIT, true>(kc, sg.iters, k, sh);
  int32_t* orow = idx + row * k;
  float* scrow = score_out ? score_out + row * k : nullptr;
  // MODE 1, block-major stage 2: list[b][block][q] = slot of every block
  // query q of sequence b chose (the lists were cleared to -1 by stage 1)
  const int64_t bseq = MODE == 1 && inv_list ? idiv(row, nq) : 0;
  int32_t* lrow = MODE == 1 && inv_list ? inv_list + bseq * nb * nq + (row - bseq * nq) : nullptr;
  const int chosen = emit_selected<NT, kSelIT>(kc, sg, sh, st, [&](int slot, int i, uint32_t key, int it) {
    orow[slot] = TOK ? i + dl[TOK ? it : 0] : i;
    if (scrow) scrow[slot] = key_to_float(key);
    if (MODE == 1 && lrow) lrow[int64_t(i) * nq] = slot;
  });
  for (int s = chosen + threadIdx.x; s < k; s += NT) {
    orow[s] = -1;
    if (scrow) scrow[s] = -INFINITY;
  }
}

// Row selection with one wave per row, for rows of at most 64 * IT
// candidates: the same arguments and result as select_rows_kernel<MODE>
// (MODE 2 for at most 512 chosen blocks), with no cross-wave barriers.
// Lane l holds candidates 64 * it + l.  Launched for HISA block selection
// (16 keys per lane).  For rows of 8,192 candidates (128 per lane) one
// wave's serial work dominated: the 128K chunk's token selection took 65.8
// against 27.5 us, the prefill chunk's flat selection 59 against 23.6 us.
template <int MODE, int IT>
__global__ __launch_bounds__(64) void select_rows_wave_kernel(const float* __restrict__ S, int64_t ld,
                                                              const int32_t* __restrict__ n_vis,
                                                              const int32_t* __restrict__ blk, int64_t n, int B,
                                                              int m, int k, int32_t* __restrict__ idx,
                                                              float* __restrict__ score_out,
                                                              int32_t* __restrict__ inv_list, int64_t nq,
                                                              int64_t nb) {
  __shared__ __align__(16) uint32_t hist[256];
  __shared__ int32_t bsh[MODE == 2 ? 512 : 1];  // chosen block ids
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t* brow = MODE == 2 ? blk + row * m : nullptr;
  // every slot the row can have is loaded before the valid count is known
  const int cap = MODE == 0 ? int(imin64(kWave * IT, n))
                            : (MODE == 1 ? int(imin64(kWave * IT, idiv(n + B - 1, B))) : min(kWave * IT, m * B));
  const float* srow = S + row * ld;
  float v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = kWave * it + lane;
    v[it] = i < cap ? srow[i] : 0.f;
  }
  if (MODE == 2)
    for (int s = lane; s < m; s += kWave) bsh[s] = brow[s];
  const int nvalid = min(cap, row_valid_count<MODE == 2 ? 3 : MODE>(n_vis, brow, row, n, B, m));
  uint32_t kc[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) kc[it] = kWave * it + lane < nvalid ? order_key(v[it]) : 0u;
  const SelThr st = wave_radix_threshold<IT>(kc, k, hist);  // its barriers also publish bsh
  int32_t* orow = idx + row * k;
  float* scrow = score_out ? score_out + row * k : nullptr;
  const bool pow2 = (B & (B - 1)) == 0;
  const int lgB = __builtin_ctz(unsigned(B));
  const int64_t bseq = MODE == 1 && inv_list ? idiv(row, nq) : 0;
  int32_t* lrow = MODE == 1 && inv_list ? inv_list + bseq * nb * nq + (row - bseq * nq) : nullptr;
  const int chosen = wave_emit_selected<IT>(kc, st, [&](int slot, int i, uint32_t key) {
    int32_t val = i;
    if (MODE == 2) {
      const int s = pow2 ? i >> lgB : i / B;
      const int off = pow2 ? i & (B - 1) : i - s * B;
      val = bsh[s] * B + off;
    }
    orow[slot] = val;
    if (scrow) scrow[slot] = key_to_float(key);
    if (MODE == 1 && lrow) lrow[int64_t(i) * nq] = slot;
  });
  for (int s = chosen + lane; s < k; s += kWave) {
    orow[s] = -1;
    if (scrow) scrow[s] = -INFINITY;
  }
}

// Long flat rows (more than kSelCap candidates), one workgroup per row:
//  1. threshold: tau = the key of rank r in an evenly spaced sample of 8192
//     scores, with r about 1.5 * k * 8192 / n (expected ~1.5 k keys >= tau);
//  2. collect: each wave streams its contiguous part of the row once with
//     16-byte loads and appends the keys >= tau, with their positions, to its
//     own LDS region in position order (ballot prefix sums);
//  3. exact top-k over the collected candidates (empty region slots hold the
//     key 0, which is never chosen), emitted in position order.
// The result is exact whatever the sample says: if fewer than k keys were
// collected the threshold was too high, if a region overflowed it was too
// low; both retry with a rank 2x lower / higher, and a row that still fails
// is flagged and finished by the exact segment + merge kernels below.
constexpr int kSampNT = 512;                 // threads per workgroup (two resident per CU: 4 waves/SIMD)
constexpr int kSampleN = 8192;               // sample size, and candidate slots per row
constexpr int kSampW = kSampNT / kWave;      // waves per workgroup
constexpr int kRegion = kSampleN / kSampW;   // candidate slots per wave
constexpr size_t kSampLds = kSampleN * 6;    // u32 keys + u16 positions

// With gate_by_flags, only rows whose flag is already nonzero run.
__global__ __launch_bounds__(kSampNT, 4) void select_sampled_kernel(const float* __restrict__ S, int64_t ld,
                                                                const int32_t* __restrict__ n_vis, int64_t n, int k,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ score_out,
                                                                int32_t* __restrict__ flags, int gate_by_flags,
                                                                int64_t rows) {
  constexpr int NW = kSampW;
  static_assert(NW * kRegion == kSampleN && kRegion % kWave == 0, "region layout");
  extern __shared__ uint32_t dyn[];
  uint32_t* rkey = dyn;  // [NW][kRegion] candidate keys; first holds the sample
  uint16_t* rpos = reinterpret_cast<uint16_t*>(dyn + kSampleN);  // [NW][kRegion] offsets in the wave's segment
  uint32_t* samp = rkey;
  __shared__ SelectShared<kSampNT> sh;
  __shared__ int wcnt[NW];
  __shared__ int bracket;
  // One row per trip (a gated launch uses a small grid and loops over the
  // rows; each row's work ends with a return from the lambda).
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    if (gate_by_flags && flags[row] == 0) continue;
    auto run_row = [&]() {
      const int nv = int(imin64(n, imax64(0, n_vis[row])));
      const float* srow = S + row * ld;
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      int32_t* orow = idx + row * k;
      float* scrow = score_out ? score_out + row * k : nullptr;

      if (nv <= kSampleN) {  // short row: plain selection over all of it
        const SelSeg sg = wave_segment<kSampNT>(nv);
        uint32_t kc[kSelIT];
        seg_keys_from_scores(srow, sg, kc);
        const SelThr st = radix_threshold<kSampNT, kSelIT>(kc, sg.iters, k, sh);
        const int chosen = emit_selected<kSampNT, kSelIT>(kc, sg, sh, st, [&](int slot, int i, uint32_t key, int) {
          orow[slot] = i;
          if (scrow) scrow[slot] = key_to_float(key);
        });
        for (int t = chosen + threadIdx.x; t < k; t += kSampNT) {
          orow[t] = -1;
          if (scrow) scrow[t] = -INFINITY;
        }
        if (threadIdx.x == 0) flags[row] = 0;
        return;
      }
      // Candidate positions are kept as 16-bit offsets inside each wave's
      // segment; a row too long for that goes to the exact fallback.
      const int segw = ((nv + NW - 1) / NW + 255) & ~255;
      if (segw > 65536) {
        if (threadIdx.x == 0) flags[row] = 1;
        return;
      }
      // 1. sample: 16 evenly spaced runs of 512 scores (16-byte aligned)
      {
        const int stride = (nv / 16) & ~3;
        for (int c = 0; c < 16; ++c) load_score_keys<kSampNT>(srow + c * stride, 512, samp + c * 512);
      }
      __syncthreads();
      const SelSeg ssg = wave_segment<kSampNT>(kSampleN);
      uint32_t skc[kSelIT];
      seg_keys_from_u32(samp, ssg, skc);
      __syncthreads();  // the sample's LDS becomes the candidate area
      int r = min(kSampleN, int((3LL * k * kSampleN) / (2LL * nv)) + 32);
      const int p0 = wave * segw, p1 = min(nv, p0 + segw);
      bool done = false;
      for (int attempt = 0; attempt < 4 && !done; ++attempt) {
        const SelThr st = radix_threshold<kSampNT, kSelIT>(skc, ssg.iters, r, sh);
        const uint32_t tau = st.thr;  // key of the r-th largest sample (0: all)
        // 2. collect keys >= tau of this wave's segment, in position order
        uint32_t* rk = rkey + wave * kRegion;
        uint16_t* rp = rpos + wave * kRegion;
        int cnt = 0;
        // kCollectU 16-byte loads per lane in flight per sweep step
        constexpr int kCollectU = 4;
        for (int base = p0; base < p1; base += 256 * kCollectU) {
          f32x4_t v[kCollectU];
    #pragma unroll
          for (int u = 0; u < kCollectU; ++u) {
            const int i = base + u * 256 + lane * 4;
            if (i + 3 < p1) {
              v[u] = *reinterpret_cast<const f32x4_t*>(srow + i);
            } else {
    #pragma unroll
              for (int e = 0; e < 4; ++e) v[u][e] = i + e < p1 ? srow[i + e] : 0.f;
            }
          }
    #pragma unroll
          for (int u = 0; u < kCollectU; ++u) {
            const int i = base + u * 256 + lane * 4;
            uint32_t key[4];
            bool sel[4];
            uint64_t bal[4];
            int below = 0, total = 0;
            const uint64_t lt = (1ull << lane) - 1ull;
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
              key[e] = i + e < p1 ? order_key(v[u][e]) : 0u;
              sel[e] = key[e] != 0u && key[e] >= tau;
              bal[e] = ballot(sel[e]);
              below += __popcll(bal[e] & lt);
              total += __popcll(bal[e]);
            }
            int slot = cnt + below;
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (sel[e]) {
                if (slot < kRegion) {
                  rk[slot] = key[e];
                  rp[slot] = uint16_t(i + e - p0);
                }
                ++slot;
              }
            }
            cnt += total;
          }
        }
        if (lane == 0) wcnt[wave] = cnt;
        __syncthreads();
        if (threadIdx.x == 0) {
          int tot = 0, ovf = 0;
          for (int w = 0; w < NW; ++w) {
            tot += wcnt[w];
            ovf |= wcnt[w] > kRegion;
          }
          bracket = ovf ? 1 : (tot < k ? 2 : 0);  // 1: tau too low, 2: tau too high
        }
        __syncthreads();
        const int vd = bracket;
        if (vd == 0) {
          for (int t = min(cnt, kRegion) + lane; t < kRegion; t += 64) rk[t] = 0u;
          done = true;
        } else {
          const int r2 = vd == 1 ? max(1, r / 2) : min(kSampleN, r * 2);
          if (r2 == r) break;
          r = r2;
        }
        __syncthreads();
      }
      if (!done) {
        if (threadIdx.x == 0) flags[row] = 1;  // finished by the segment + merge kernels
        return;
      }
      // 3. exact selection over the candidates (key 0 = empty slot); the wave
      // segments of kSampleN keys are exactly the waves' regions
      const SelSeg csg = wave_segment<kSampNT>(kSampleN);
      uint32_t ckc[kSelIT];
      seg_keys_from_u32(rkey, csg, ckc);
      const SelThr st = radix_threshold<kSampNT, kSelIT>(ckc, csg.iters, k, sh);
      // candidate i lies in the region (and segment) of the wave that emits it
      const int chosen = emit_selected<kSampNT, kSelIT>(ckc, csg, sh, st, [&](int slot, int i, uint32_t key, int) {
        orow[slot] = p0 + int(rpos[i]);
        if (scrow) scrow[slot] = key_to_float(key);
      });
      for (int t = chosen + threadIdx.x; t < k; t += kSampNT) {
        orow[t] = -1;
        if (scrow) scrow[t] = -INFINITY;
      }
      if (threadIdx.x == 0) flags[row] = 0;
    };
    run_row();
    __syncthreads();
  }
}

// Level 1 for long flat rows: exact top-k of each segment (an element outside
// its segment's top-k has k larger elements and cannot be chosen overall).
// Candidate lists are stored with a stride of kp = k rounded up to 4 entries.
__global__ __launch_bounds__(kSelNT) void select_segment_kernel(const float* __restrict__ S, int64_t ld,
                                                                const int32_t* __restrict__ n_vis, int64_t n, int seg,
                                                                int nseg, int k, int kp, uint32_t* __restrict__ ckey,
                                                                int32_t* __restrict__ cpos,
                                                                const int32_t* __restrict__ flags, int64_t rows) {
  __shared__ SelectShared<kSelNT> sh;
  // One row per trip: a gated launch uses a small grid and loops over rows.
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
    if (flags[row] == 0) continue;  // already selected by select_sampled_kernel
    const int s = blockIdx.x;
    const int64_t nv = imin64(n, imax64(0, n_vis[row]));
    const int64_t p0 = int64_t(s) * seg;
    const int cnt = int(imax64(0, imin64(seg, nv - p0)));
    const SelSeg sg = wave_segment<kSelNT>(cnt);
    uint32_t kc[kSelIT];
    seg_keys_from_scores(S + row * ld + p0, sg, kc);
    const SelThr st = radix_threshold<kSelNT, kSelIT>(kc, sg.iters, k, sh);
    uint32_t* ok = ckey + (row * nseg + s) * int64_t(kp);
    int32_t* op = cpos + (row * nseg + s) * int64_t(kp);
    const int chosen = emit_selected<kSelNT, kSelIT>(kc, sg, sh, st, [&](int slot, int i, uint32_t key, int) {
      ok[slot] = key;
      op[slot] = int32_t(p0 + i);
    });
    for (int t = chosen + threadIdx.x; t < kp; t += kSelNT) {
      ok[t] = 0u;
      op[t] = -1;
    }
    __syncthreads();
  }
}

// Level >= 2: merges groups of G candidate lists (ascending positions, key 0
// = empty slot).  With one group left it writes the final indices.
__global__ __launch_bounds__(kSelNT) void select_merge_kernel(const uint32_t* __restrict__ ikey,
                                                              const int32_t* __restrict__ ipos, int nin, int G, int k,
                                                              int kp, uint32_t* __restrict__ okey,
                                                              int32_t* __restrict__ opos,
                                                              int32_t* __restrict__ idx, float* __restrict__ score_out,
                                                              const int32_t* __restrict__ flags, int64_t rows) {
  __shared__ SelectShared<kSelNT> sh;
  // One row per trip: a gated launch uses a small grid and loops over rows.
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
    if (flags[row] == 0) continue;  // already selected by select_sampled_kernel
    const int grp = blockIdx.x;
    const int nout = (nin + G - 1) / G;
    const int l0 = grp * G, l1 = min(nin, l0 + G);
    const int cnt = (l1 - l0) * kp;
    const uint32_t* ik = ikey + (row * nin + l0) * int64_t(kp);
    const int32_t* ip = ipos + (row * nin + l0) * int64_t(kp);
    const SelSeg sg = wave_segment<kSelNT>(cnt);
    uint32_t kc[kSelIT];
    int32_t pc[kSelIT];
    {
      const int lane = threadIdx.x & (kWave - 1);
  #pragma unroll
      for (int it = 0; it < kSelIT; ++it) {
        const int i = sg.p0 + it * kWave + lane;
        const bool in = it < sg.iters && i < sg.p1;
        kc[it] = in ? ik[i] : 0u;
        pc[it] = in ? ip[i] : -1;
      }
    }
    const SelThr st = radix_threshold<kSelNT, kSelIT>(kc, sg.iters, k, sh);
    if (nout == 1) {
      int32_t* orow = idx + row * k;
      float* scrow = score_out ? score_out + row * k : nullptr;
      const int chosen = emit_selected<kSelNT, kSelIT>(kc, sg, sh, st, [&](int slot, int, uint32_t key, int it) {
        orow[slot] = pc[it];
        if (scrow) scrow[slot] = key_to_float(key);
      });
      for (int t = chosen + threadIdx.x; t < k; t += kSelNT) {
        orow[t] = -1;
        if (scrow) scrow[t] = -INFINITY;
      }
    } else {
      uint32_t* ok = okey + (row * nout + grp) * int64_t(kp);
      int32_t* op = opos + (row * nout + grp) * int64_t(kp);
      const int chosen = emit_selected<kSelNT, kSelIT>(kc, sg, sh, st, [&](int slot, int, uint32_t key, int it) {
        ok[slot] = key;
        op[slot] = pc[it];
      });
      for (int t = chosen + threadIdx.x; t < kp; t += kSelNT) {
        ok[t] = 0u;
        op[t] = -1;
      }
    }
    __syncthreads();
  }
}

// Fused long flat rows, step 1 of 2 (after the sample scores): the row's
// candidate threshold.  The sample holds the scores of every tstride-th
// 64-key tile, packed (sample position i is cache key
// (i / 64) * 64 * tstride + i % 64).  With v visible keys of which the
// sample holds s, the threshold is the sample key of rank
// r = max(2 k s / v, floor) (at most s): about max(2k, floor v / s) keys of
// the whole row are expected at or above it.  The floor, 64 or less when
// 64 v / s would pass half the candidate select's capacity (4,096), keeps
// the rank's relative spread small: at least k keys pass with overwhelming
// probability for any row whose scores do not depend on the key's position
// modulo the stride.  Rows with v <= k, or a sample of at most r keys, take
// every key (threshold key 0).  Also clears the row's chunk counts.
constexpr int kThrNT = 256;
__global__ __launch_bounds__(kThrNT) void flat_threshold_kernel(const float* __restrict__ Ssamp, int64_t lds,
                                                                const int32_t* __restrict__ n_vis, int64_t n,
                                                                int tstride, int k, uint32_t* __restrict__ thr,
                                                                int32_t* __restrict__ ccnt, int nch) {
  __shared__ SelectShared<kThrNT> sh;
  const int64_t row = blockIdx.x;
  for (int c = threadIdx.x; c < nch; c += kThrNT) ccnt[row * nch + c] = 0;
  const int nv = int(imin64(n, imax64(0, n_vis[row])));
  const int64_t span = 64LL * tstride;
  // sample keys below nv: whole tiles, then the part of the tile holding nv
  const int64_t full = nv / span;
  const int ns = int(int64_t(full) * 64 + imin64(64, nv - full * span));
  const int nsl = int(imin64(lds, ((nv + span - 1) / span) * 64));
  const SelSeg sg = wave_segment<kThrNT>(nsl);
  uint32_t kc[kSelIT];
  {
    const float* src = Ssamp + row * lds;
    const int lane = threadIdx.x & (kWave - 1);
    float v[kSelIT];
#pragma unroll
    for (int it = 0; it < kSelIT; ++it) {
      const int i = sg.p0 + it * kWave + lane;
      v[it] = it < sg.iters && i < sg.p1 ? src[i] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < kSelIT; ++it) {
      const int i = sg.p0 + it * kWave + lane;
      const int64_t e = int64_t(i / 64) * span + (i & 63);
      kc[it] = it < sg.iters && i < sg.p1 && e < nv ? order_key(v[it]) : 0u;
    }
  }
  const int64_t floor_r = imax64(1, imin64(64, 4096LL * ns / imax64(1, nv)));
  int r = int(imin64(ns, imax64(floor_r, (2LL * k * ns + nv - 1) / imax64(1, nv))));
  if (nv <= k) r = ns;  // every key
  const SelThr st = radix_threshold<kThrNT, kSelIT>(kc, sg.iters, r, sh);
  if (threadIdx.x == 0) thr[row] = nv <= k ? 0u : st.thr;
}

// Fused long flat rows, step 2 of 2: exact top-k over the row's candidates
// (every key at or above the threshold, packed per key chunk by the score
// kernel in increasing key order, so the concatenated list is in key order
// and the usual position-order emission gives ascending indices and the
// lower-index tie rule).  The result equals the top-k of the whole row when
// at least k candidates exist (or every visible key is one) and no chunk's
// span overflowed; otherwise the row is flagged for the full path.
constexpr int kCandNT = 512;
constexpr int kCandMaxChunks = 2 * kCandNT;
// 8 waves per SIMD, as for flat rows in select_rows_kernel: the 128K
// chunk's 1,024 rows then run in one round (36.9 -> 31.4 us).
__global__ __launch_bounds__(kCandNT, 8) void flat_cand_select_kernel(const float* __restrict__ S, int64_t ld,
                                                                   const uint32_t* __restrict__ thr,
                                                                   const int32_t* __restrict__ ccnt, int nch,
                                                                   int chunk, const int32_t* __restrict__ n_vis,
                                                                   int64_t n, int k, int32_t* __restrict__ idx,
                                                                   float* __restrict__ score_out,
                                                                   int32_t* __restrict__ flags) {
  __shared__ SelectShared<kCandNT> sh;
  __shared__ int pre[kCandMaxChunks + 1];
  __shared__ int bad;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int nv = int(imin64(n, imax64(0, n_vis[row])));
  int32_t* orow = idx + row * k;
  float* scrow = score_out ? score_out + row * k : nullptr;
  if (thr[row] == 0u) {  // every visible key: plain scores at their positions
    if (nv > kSelIT * kCandNT) {
      if (threadIdx.x == 0) flags[row] = 1;
      return;
    }
    const SelSeg sg = wave_segment<kCandNT>(nv);
    uint32_t kc[kSelIT];
    seg_keys_from_scores(S + row * ld, sg, kc);
    const SelThr st = radix_threshold<kCandNT, kSelIT>(kc, sg.iters, k, sh);
    const int chosen = emit_selected<kCandNT, kSelIT>(kc, sg, sh, st, [&](int slot, int i, uint32_t key, int) {
      orow[slot] = i;
      if (scrow) scrow[slot] = key_to_float(key);
    });
    for (int t = chosen + threadIdx.x; t < k; t += kCandNT) {
      orow[t] = -1;
      if (scrow) scrow[t] = -INFINITY;
    }
    if (threadIdx.x == 0) flags[row] = 0;
    return;
  }
  // chunk c's span holds min(chunk, ld - c*chunk) / 2 pairs
  if (threadIdx.x == 0) bad = 0;
  // thread t owns chunks 2t and 2t+1 (nch <= 2 * kCandNT)
  int my[2] = {0, 0};
  bool over = false;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 2 * int(threadIdx.x) + j;
    if (c < nch) {
      const int cap = int(imin64(chunk, ld - int64_t(c) * chunk)) / 2;
      my[j] = ccnt[row * nch + c];
      over |= my[j] > cap;
    }
  }
  __syncthreads();
  if (over) bad = 1;
  // exclusive prefix of the counts
  {
    const int wave = wave_index();
    const uint32_t v = uint32_t(my[0] + my[1]);
    const uint32_t incl = wave_prefix_incl(v);
    if (lane == kWave - 1) sh.wtot[wave] = incl;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += sh.wtot[w];
    const int c = 2 * int(threadIdx.x);
    const int ex = int(base + incl - v);
    if (c < nch) pre[c] = ex;
    if (c + 1 < nch) pre[c + 1] = ex + my[0];
    if (c + 1 == nch) pre[nch] = ex + my[0];
    if (c + 2 == nch) pre[nch] = ex + my[0] + my[1];
  }
  __syncthreads();
  const int total = pre[nch];
  if (bad || total > kSelIT * kCandNT || (total < k && total < nv)) {
    if (threadIdx.x == 0) flags[row] = 1;  // finished by the full path
    return;
  }
  const SelSeg sg = wave_segment<kCandNT>(total);
  uint32_t kc[kSelIT];
  int32_t pc[kSelIT];
  {
    const float* srow = S + row * ld;
    float2 v[kSelIT];
#pragma unroll
    for (int it = 0; it < kSelIT; ++it) {
      const int i = sg.p0 + it * kWave + lane;
      v[it] = make_float2(0.f, 0.f);
      if (it < sg.iters && i < sg.p1) {
        // chunk holding candidate i: the last c with pre[c] <= i
        int lo = 0, hi = nch - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        v[it] = *reinterpret_cast<const float2*>(srow + int64_t(lo) * chunk + 2 * (i - pre[lo]));
      }
    }
#pragma unroll
    for (int it = 0; it < kSelIT; ++it) {
      const int i = sg.p0 + it * kWave + lane;
      const bool in = it < sg.iters && i < sg.p1;
      kc[it] = in ? order_key(v[it].x) : 0u;
      pc[it] = in ? __float_as_int(v[it].y) : -1;
    }
  }
  const SelThr st = radix_threshold<kCandNT, kSelIT>(kc, sg.iters, k, sh);
  const int chosen = emit_selected<kCandNT, kSelIT>(kc, sg, sh, st, [&](int slot, int, uint32_t key, int it) {
    orow[slot] = pc[it];
    if (scrow) scrow[slot] = key_to_float(key);
  });
  for (int t = chosen + threadIdx.x; t < k; t += kCandNT) {
    orow[t] = -1;
    if (scrow) scrow[t] = -INFINITY;
  }
  if (threadIdx.x == 0) flags[row] = 0;
}

// ---------------------------------------------------------------------------
// Block-sparse selection: every visible entry of each chosen block.  Slot
// s * B + j of a row is entry blk[s] * B + j when the block exists and the
// entry is visible, else -1.  Chosen blocks are ascending and only the last
// of them can be partly visible (it holds the row's last visible entry), so
// the list is ascending with the -1s at its end.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void expand_blocks_kernel(const int32_t* __restrict__ blk,
                                                            const int32_t* __restrict__ n_vis, int64_t n, int B,
                                                            int m, int32_t* __restrict__ idx) {
  const int64_t row = blockIdx.y;
  const int t = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (t >= m * B) return;
  const int s = t / B, j = t - s * B;
  const int bid = blk[row * m + s];
  const int64_t nv = imin64(n, imax64(0, n_vis[row]));
  const int64_t e = int64_t(bid) * B + j;
  idx[row * int64_t(m) * B + t] = bid >= 0 && e < nv ? int32_t(e) : -1;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static int64_t round4(int64_t x) { return (x + 3) & ~int64_t(3); }

static bool flat_mfma_ok(const IndexArgs& a) {
  return a.dtype == 1 && a.h_i == 16 && (a.d_i == 32 || a.d_i == 64 || a.d_i == 128 || a.d_i == 256) &&
         a.n < (int64_t(1) << 31);
}

// Key chunk of the MFMA flat score over nkeys launch keys: 8192 keys, halved
// (down to 256) until the grid has about four workgroups per CU (two
// resident, 256 CUs).  Long chunks spread each workgroup's query-fragment
// loads over more tiles (measured at 128K: 8192-key chunks beat 2048).
static int flat_chunk(const IndexArgs& a, int64_t nkeys, int64_t target_wg = 1024) {
  const int64_t nqb = (a.nq + 15) / 16;
  int chunk = 8192;
  while (chunk > 256 && nqb * a.bt * ((nkeys + chunk - 1) / chunk) < target_wg) chunk /= 2;
  return chunk;
}


// Flat score for one query per sequence (score_flat_dec_kernel): chunks of
// a multiple of 64 launch keys, one per wave, about 4,096 waves per launch
// and at most kCandMaxChunks chunks per row.
static bool flat_dec_ok(const IndexArgs& a) { return flat_mfma_ok(a) && a.nq == 1 && a.d_i <= 128; }
static int flat_dec_chunk(const IndexArgs& a, int64_t nkeys) {
  int64_t c = std::max<int64_t>((a.bt * nkeys + 4095) / 4096, (nkeys + kCandMaxChunks - 1) / kCandMaxChunks);
  return int(std::max<int64_t>(64, (c + 63) / 64 * 64));
}

struct FlatPlan {
  int64_t rows, ld;
  bool multi;
  int seg, nseg, G, kp;
  // fused path (long rows on the 32x32 MFMA score kernel): sample stride and
  // row length, key chunk of the collecting pass and its chunk count
  bool fused;
  int tstride, chunk, nch;
  int64_t lds;
  size_t s_bytes, cand_bytes, flag_bytes, samp_bytes, thr_bytes, ccnt_bytes, total;
};

static FlatPlan plan_flat(const IndexArgs& a, int k) {
  FlatPlan p{};
  p.rows = a.bt * a.nq;
  p.ld = round4(std::max<int64_t>(a.n, 1));
  p.multi = a.n > kSelCap;
  p.s_bytes = align256(size_t(p.rows) * p.ld * 4);
  if (p.multi) {
    p.seg = kSelCap;
    p.nseg = int((a.n + p.seg - 1) / p.seg);
    p.kp = (k + 3) & ~3;
    p.G = kSelCap / p.kp;
    // ping-pong candidate buffers: level-1 lists, then merged lists
    const size_t l1 = size_t(p.rows) * p.nseg * p.kp * 8;
    const size_t l2 = size_t(p.rows) * ((p.nseg + p.G - 1) / p.G) * p.kp * 8;
    p.cand_bytes = align256(l1) + align256(l2);
    p.flag_bytes = align256(size_t(p.rows) * 4);
    const int64_t ntiles = (a.n + 63) / 64;
    p.chunk = flat_dec_ok(a) ? flat_dec_chunk(a, a.n) : flat_chunk(a, a.n);
    p.nch = int((a.n + p.chunk - 1) / p.chunk);
    // The threshold keeps about 2k candidates (+-12% at the smallest sample);
    // the candidate select holds kSelIT * kCandNT = 8,192 of them, so larger
    // k would flag most rows and rerun them on the full path.
    p.fused = flat_mfma_ok(a) && a.d_i <= 128 && p.nch <= kCandMaxChunks && ntiles >= 64 && k <= 3072;
    if (p.fused) {
      // 32 to 64 sample tiles spread evenly (the threshold kernel holds
      // 4,096 sample keys), the most for small k, where the threshold rank
      // 2ks/v is lowest.
      p.tstride = int(std::max<int64_t>((ntiles + 63) / 64, std::min<int64_t>(ntiles / 32, std::max(k / 32, 1))));
      p.lds = (ntiles + p.tstride - 1) / p.tstride * 64;
      p.samp_bytes = align256(size_t(p.rows) * p.lds * 4);
      p.thr_bytes = align256(size_t(p.rows) * 4);
      p.ccnt_bytes = align256(size_t(p.rows) * p.nch * 4);
    }
  }
  p.total = p.s_bytes + p.cand_bytes + p.flag_bytes + p.samp_bytes + p.thr_bytes + p.ccnt_bytes;
  return p;
}

size_t flat_topk_ws_bytes(const IndexArgs& a, int k) { return plan_flat(a, k).total; }

static void set_lds_limits() {
  static bool done = false;
  if (done) return;
  done = true;
  (void)hipFuncSetAttribute((const void*)select_sampled_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kSampLds);
}

template <int MODE, typename TQ, typename TK>
static void launch_valu_score(const IndexArgs& a, const TK* keys, int64_t keys_per_seq, int64_t ncand,
                              const int32_t* blk, int B, int m, int64_t ld, float* S, hipStream_t st) {
  const size_t smem = size_t(a.h_i) * a.d_i * 4 + size_t(a.h_i) * 4;
  dim3 grid(unsigned((ncand + 255) / 256), unsigned(a.bt * a.nq));
  LaunchScope ls(MODE == 0 ? "score_valu_flat" : MODE == 1 ? "score_valu_stage1" : "score_valu_stage2", st);
  HATTN_LAUNCH((score_valu_kernel<TQ, TK, MODE>), grid, dim3(256), smem, st, (const TQ*)a.q_i, keys, a.w_i,
                     a.n_vis, blk, a.nq, a.h_i, a.d_i, a.n, keys_per_seq, B, m, ld, S);
}

// Flat scores of every visible key into S (row stride ld).  On the 32x32
// MFMA kernel the extra arguments select the sample (tstride > 1: launch key
// e is cache key (e / 64) * 64 * tstride + e % 64, nkeys launch keys per
// row), the candidate collection (thr, ccnt, with chunk fixed by the plan),
// or a gated pass (rows with gate[row] != 0 only).
struct FlatScoreMode {
  int64_t nkeys;
  int tstride = 1;
  const uint32_t* thr = nullptr;
  int32_t* ccnt = nullptr;
  const int32_t* gate = nullptr;
  int chunk = 0;  // 0: flat_chunk(nkeys)
  int64_t target_wg = 1024;
};

static hipError_t launch_flat_score(const IndexArgs& a, int64_t ld, float* S, const FlatScoreMode& fm,
                                    hipStream_t st) {
  if (flat_dec_ok(a)) {
    const int chunk = fm.chunk ? fm.chunk : flat_dec_chunk(a, fm.nkeys);
    const int nch = int((fm.nkeys + chunk - 1) / chunk);
    const dim3 grid(unsigned((nch + 3) / 4), unsigned(a.bt));
    const bool collect = fm.thr != nullptr;
    LaunchScope ls(collect             ? "score_flat_collect"
                   : fm.tstride > 1    ? "score_flat_sample"
                   : fm.gate != nullptr ? "score_flat_fallback"
                                        : "score_flat_mfma",
                   st);
#define HATTN_FLATDEC(KS, MODE)                                                                                \
  HATTN_LAUNCH((score_flat_dec_kernel<KS, MODE>), grid, dim3(256), 0, st, (const uint16_t*)a.q_i,            \
               (const uint16_t*)a.k_i, a.w_i, a.n_vis, a.n, ld, S, nch, chunk, fm.tstride, fm.thr, fm.ccnt, \
               fm.gate)
    switch (a.d_i) {
      case 32:
        if (collect) HATTN_FLATDEC(1, 1);
        else HATTN_FLATDEC(1, 0);
        break;
      case 64:
        if (collect) HATTN_FLATDEC(2, 1);
        else HATTN_FLATDEC(2, 0);
        break;
      default:
        if (collect) HATTN_FLATDEC(4, 1);
        else HATTN_FLATDEC(4, 0);
        break;
    }
#undef HATTN_FLATDEC
    return hipGetLastError();
  }
  if (flat_mfma_ok(a)) {
    // 16 queries per workgroup.  (32, with 8 waves sharing each key tile,
    // measured slower: one resident workgroup per CU and longer barriers.)
    const int nqb = int((a.nq + 15) / 16);
    const int chunk = fm.chunk ? fm.chunk : flat_chunk(a, fm.nkeys, fm.target_wg);
    const int nch = int((fm.nkeys + chunk - 1) / chunk);
    dim3 grid(xcd_grid(nqb, nch), unsigned(a.bt));
    const bool collect = fm.thr != nullptr;
    LaunchScope ls(collect             ? "score_flat_collect"
                   : fm.tstride > 1    ? "score_flat_sample"
                   : fm.gate != nullptr ? "score_flat_fallback"
                                        : "score_flat_mfma",
                   st);
#define HATTN_FLAT32(KS, MODE)                                                                               \
  HATTN_LAUNCH((score_flat_mfma32_kernel<KS, MODE>), grid, dim3(256), 0, st, (const uint16_t*)a.q_i,        \
               (const uint16_t*)a.k_i, a.w_i, a.n_vis, a.nq, a.n, ld, S, nqb, nch, chunk, fm.tstride, fm.thr, \
               fm.ccnt, fm.gate)
#define HATTN_FLAT(KS)                                                                                       \
  HATTN_LAUNCH((score_flat_mfma_kernel<KS, 4>), grid, dim3(256), 0, st, (const uint16_t*)a.q_i,             \
               (const uint16_t*)a.k_i, a.w_i, a.n_vis, a.nq, a.n, ld, S, nqb, nch, chunk)
    if (a.d_i == 256 && (collect || fm.tstride != 1 || fm.gate)) return hipErrorInvalidValue;
    switch (a.d_i) {
      case 32:
        if (collect) HATTN_FLAT32(2, 1);
        else HATTN_FLAT32(2, 0);
        break;
      case 64:
        if (collect) HATTN_FLAT32(4, 1);
        else HATTN_FLAT32(4, 0);
        break;
      case 128:
        if (collect) HATTN_FLAT32(8, 1);
        else HATTN_FLAT32(8, 0);
        break;
      default: HATTN_FLAT(8); break;
    }
#undef HATTN_FLAT32
#undef HATTN_FLAT
  } else {
    if (fm.thr || fm.tstride != 1 || fm.gate) return hipErrorInvalidValue;
    if (a.dtype == 0) launch_valu_score<0, float>(a, (const float*)a.k_i, a.n, a.n, nullptr, 1, 1, ld, S, st);
    else launch_valu_score<0, uint16_t>(a, (const uint16_t*)a.k_i, a.n, a.n, nullptr, 1, 1, ld, S, st);
  }
  return hipGetLastError();
}

hipError_t launch_flat_topk(const IndexArgs& a, int k, int32_t* idx, float* score, void* ws, hipStream_t st) {
  set_lds_limits();
  const FlatPlan p = plan_flat(a, k);
  float* S = reinterpret_cast<float*>(ws);
  FlatScoreMode full;
  full.nkeys = a.n;
  hipError_t e;
  if (!p.multi) {
    e = launch_flat_score(a, p.ld, S, full, st);
    if (e != hipSuccess) return e;
    LaunchScope ls("select_rows", st);
    // More rows than CUs: throughput counts, and 512-thread workgroups (rows
    // of up to 8,192 keys) let four rows share a CU instead of two.
    if (p.rows >= 256 && a.n <= kSelIT * 512)
      HATTN_LAUNCH((select_rows_kernel<0, 512>), dim3(unsigned(p.rows)), dim3(512), 0, st, S, p.ld, a.n_vis,
                   nullptr, a.n, 1, 1, k, idx, score, nullptr, int64_t(1), int64_t(1));
    else
      HATTN_LAUNCH((select_rows_kernel<0, kSelNT>), dim3(unsigned(p.rows)), dim3(kSelNT), 0, st, S, p.ld, a.n_vis,
                   nullptr, a.n, 1, 1, k, idx, score, nullptr, int64_t(1), int64_t(1));
    return hipGetLastError();
  }
  char* cb = reinterpret_cast<char*>(ws) + p.s_bytes;
  const size_t l1 = align256(size_t(p.rows) * p.nseg * p.kp * 8);
  uint32_t* bufk[2];
  int32_t* bufp[2];
  bufk[0] = reinterpret_cast<uint32_t*>(cb);
  bufp[0] = reinterpret_cast<int32_t*>(cb + size_t(p.rows) * p.nseg * p.kp * 4);
  bufk[1] = reinterpret_cast<uint32_t*>(cb + l1);
  const int n2 = (p.nseg + p.G - 1) / p.G;
  bufp[1] = reinterpret_cast<int32_t*>(cb + l1 + size_t(p.rows) * n2 * p.kp * 4);
  int32_t* flags = reinterpret_cast<int32_t*>(cb + p.cand_bytes);
  if (p.fused) {
    // sample scores -> per-row threshold -> scores >= threshold, packed per
    // chunk -> exact top-k of the candidates; rows the candidates cannot
    // decide are flagged and run the full path below, gated by their flag
    char* fb = cb + p.cand_bytes + p.flag_bytes;
    float* Ssamp = reinterpret_cast<float*>(fb);
    uint32_t* thr = reinterpret_cast<uint32_t*>(fb + p.samp_bytes);
    int32_t* ccnt = reinterpret_cast<int32_t*>(fb + p.samp_bytes + p.thr_bytes);
    FlatScoreMode sm;
    sm.nkeys = p.lds;
    sm.tstride = p.tstride;
    sm.target_wg = 512;  // twice as many tiles per workgroup as the full pass: half the query-fragment loads
    e = launch_flat_score(a, p.lds, Ssamp, sm, st);
    if (e != hipSuccess) return e;
    {
      LaunchScope ls("flat_threshold", st);
      HATTN_LAUNCH(flat_threshold_kernel, dim3(unsigned(p.rows)), dim3(kThrNT), 0, st, Ssamp, p.lds, a.n_vis, a.n,
                   p.tstride, k, thr, ccnt, p.nch);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    FlatScoreMode cm;
    cm.nkeys = a.n;
    cm.thr = thr;
    cm.ccnt = ccnt;
    cm.chunk = p.chunk;
    e = launch_flat_score(a, p.ld, S, cm, st);
    if (e != hipSuccess) return e;
    {
      LaunchScope ls("flat_cand_select", st);
      HATTN_LAUNCH(flat_cand_select_kernel, dim3(unsigned(p.rows)), dim3(kCandNT), 0, st, S, p.ld, thr, ccnt, p.nch,
                   p.chunk, a.n_vis, a.n, k, idx, score, flags);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    FlatScoreMode gm;
    gm.nkeys = a.n;
    gm.gate = flags;
    e = launch_flat_score(a, p.ld, S, gm, st);
  } else {
    e = launch_flat_score(a, p.ld, S, full, st);
  }
  if (e != hipSuccess) return e;
  // After the fused path only flagged rows (normally none) remain: small
  // grids whose workgroups loop over the rows keep these launches cheap.
  const int64_t grows = p.fused ? std::min<int64_t>(p.rows, 64) : p.rows;
  {
    LaunchScope ls("select_sampled", st);
    HATTN_LAUNCH(select_sampled_kernel, dim3(unsigned(p.fused ? std::min<int64_t>(p.rows, 256) : p.rows)),
                 dim3(kSampNT), kSampLds, st, S, p.ld, a.n_vis, a.n, k, idx, score, flags, p.fused ? 1 : 0, p.rows);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    LaunchScope ls("select_segment", st);
    HATTN_LAUNCH(select_segment_kernel, dim3(unsigned(p.nseg), unsigned(grows)), dim3(kSelNT), 0, st,
                       S, p.ld, a.n_vis, a.n, p.seg, p.nseg, k, p.kp, bufk[0], bufp[0], flags, p.rows);
  }
  int nin = p.nseg, cur = 0;
  while (true) {
    const int nout = (nin + p.G - 1) / p.G;
    LaunchScope ls("select_merge", st);
    // Lists of a row at level i+1 never outnumber those at level i, so the
    // two buffers (sized for levels 1 and 2) alternate safely.
    HATTN_LAUNCH(select_merge_kernel, dim3(unsigned(nout), unsigned(grows)), dim3(kSelNT), 0, st,
                       bufk[cur], bufp[cur], nin, p.G, k, p.kp, bufk[cur ^ 1], bufp[cur ^ 1], idx, score, flags,
                       p.rows);
    e = hipGetLastError();
    if (e != hipSuccess || nout == 1) return e;
    nin = nout;
    cur ^= 1;
  }
}

// ---- HISA -------------------------------------------------------------------
struct HisaPlan {
  int64_t rows, nb, ld1, ld2;
  bool bm;  // block-major stage 2
  size_t s1_bytes, blk_bytes, s2_bytes, list_bytes, total;
};

static HisaPlan plan_hisa(const IndexArgs& a, int B, int m) {
  HisaPlan p{};
  p.rows = a.bt * a.nq;
  p.nb = (a.n + B - 1) / B;
  p.ld1 = round4(std::max<int64_t>(p.nb, 1));
  p.ld2 = round4(int64_t(m) * B);
  p.s1_bytes = align256(size_t(p.rows) * p.ld1 * 4);
  p.blk_bytes = align256(size_t(p.rows) * m * 4);
  p.s2_bytes = align256(size_t(p.rows) * p.ld2 * 4);
  // Block-major stage 2 pays off once each block has many choosers.  Its
  // per-block chooser lists have one slot per query of the sequence (the
  // chosen slot, or -1), cleared by stage 1 every call: at most 8M entries,
  // and at most 4096 queries (a block's compacted list lives in LDS).
  p.bm = a.dtype == 1 && a.h_i == 16 && (a.d_i == 32 || a.d_i == 64 || a.d_i == 128) && B <= 128 &&
         B % 64 == 0 && a.nq >= 128 && a.nq <= 4096 && int64_t(a.nq) * m >= 8 * p.nb && p.nb <= 65535 &&
         a.bt <= 65535 && a.bt * p.nb * a.nq <= (int64_t(1) << 23) && p.rows * m < (int64_t(1) << 31);
  if (p.bm) p.list_bytes = align256(size_t(a.bt) * p.nb * a.nq * 4);
  p.total = p.s1_bytes + p.blk_bytes + p.s2_bytes + p.list_bytes;
  return p;
}

size_t hisa_topk_ws_bytes(const IndexArgs& a, int B, int m, int k) {
  (void)k;
  return plan_hisa(a, B, m).total;
}

// Head sizes with an MFMA stage-1 (and decode front) instantiation: the
// kernels are compiled for d_i = 16 * KQ with KQ in {1, 2, 4, 8, 16} only, so
// every other width must take the vector kernel.
static bool stage1_mfma_dim(int d_i) {
  return d_i == 16 || d_i == 32 || d_i == 64 || d_i == 128 || d_i == 256;
}

// The front kernel's static LDS tile (64 * (d_i + 4) floats) doubles as the
// scratch of its cache-maintenance roles: an entry role needs w softmax
// weights plus 2,048 floats of row-group sums (256 threads x 8 bf16 each),
// and the fresh block mean needs 2,048 floats of row-group sums too.
size_t block_sparse_ws_bytes(const IndexArgs& a, int B, int m) {
  const HisaPlan p = plan_hisa(a, B, m);
  return p.s1_bytes + p.blk_bytes;
}

bool decode_front_ok(const IndexArgs& a, int B, int m, int max_w) {
  const int64_t tile = 64LL * (a.d_i + 4);
  return a.dtype == 1 && a.h_i == 16 && stage1_mfma_dim(a.d_i) && a.nq == 1 && !plan_hisa(a, B, m).bm &&
         a.n > 0 && tile >= int64_t(max_w) + 2048;
}

hipError_t launch_decode_front(const IndexArgs& a, float* reps, int B, int m, void* ws, const int32_t* q_pos,
                               const void* x1, const float* z1, const float* bias1, int w1, int s1, void* y1,
                               int32_t* n_vis1, const void* x2, const float* z2, const float* bias2, int w2, int s2,
                               void* y2, int64_t N2, int32_t* n_vis2, int64_t L, int C, hipStream_t st,
                               int raw_rows) {
  const HisaPlan p = plan_hisa(a, B, m);
  float* S1 = reinterpret_cast<float*>(ws);
  const AppendK la{x1, L, C, z1, bias1, w1, s1, y1, a.n, n_vis1, a.k_i, a.d_i, B, reps, raw_rows};
  const AppendK lb{x2, L, C, z2, bias2, w2, s2, y2, N2, n_vis2, nullptr, 0, 0, nullptr, raw_rows};
  const int nch = int((p.nb + 63) / 64);
  const int nch_grid = int(xcd_grid(1, nch));
  const int nroles = x2 ? 2 : 1;
  dim3 grid(unsigned(nch_grid + nroles), unsigned(a.bt));
  LaunchScope ls("decode_front", st);
#define HATTN_FRONT(KQ)                                                                                      \
  HATTN_LAUNCH(decode_front_kernel<KQ>, grid, dim3(256), 0, st, (const uint16_t*)a.q_i, reps, a.w_i, q_pos, B, \
               p.nb, p.ld1, S1, nch, nch_grid, la, lb, nroles)
  // (d_i = 16 never gets here: its LDS tile cannot hold the append roles'
  // scratch, so decode_front_ok sends it to the separate kernels)
  switch (a.d_i) {
    case 32: HATTN_FRONT(2); break;
    case 64: HATTN_FRONT(4); break;
    case 128: HATTN_FRONT(8); break;
    case 256: HATTN_FRONT(16); break;
    default: return hipErrorInvalidValue;  // decode_front_ok admits no other width
  }
#undef HATTN_FRONT
  return hipGetLastError();
}

// HISA's first stage for every row of a call: block scores of the blocks
// whose first entry is visible into S1 (row stride ld1), then the top-m
// blocks of each row into blk_out (ascending, -1 padded).  bm_list: the
// block-major stage 2's chooser lists (cleared here, filled by the block
// selection), or nullptr.  stage1_done: S1 already holds the scores (the
// decode front kernel wrote them).
static hipError_t launch_hisa_blocks(const IndexArgs& a, const float* reps, int B, int m, const HisaPlan& p, float* S1,
                                     int32_t* blk_out, int32_t* bm_list, bool stage1_done, hipStream_t st) {
  // Stage 1: block scores.
  const bool mfma1 = a.h_i == 16 && stage1_mfma_dim(a.d_i);
  const int64_t bm_fill = bm_list ? a.bt * p.nb * a.nq : 0;
  const bool x3 = mfma1 && a.dtype == 1 && a.nq >= 16 && (a.d_i == 32 || a.d_i == 64 || a.d_i == 128) &&
                  p.nb < (int64_t(1) << 31);
  if (stage1_done) {
    // S1 was written by the decode front kernel
  } else if (x3) {
    const int nqb = int((a.nq + 15) / 16);
    int chunk = 1024;  // blocks per workgroup, halved until ~4 workgroups per CU
    while (chunk > 64 && int64_t(nqb) * a.bt * ((p.nb + chunk - 1) / chunk) < 1024) chunk /= 2;
    const int nch = int((p.nb + chunk - 1) / chunk);
    dim3 grid(xcd_grid(nqb, nch), unsigned(a.bt));
    LaunchScope ls("score_stage1_mfma", st);
#define HATTN_S1X3(KS)                                                                                       \
  HATTN_LAUNCH(score_stage1_x3_kernel<KS>, grid, dim3(256), 0, st, (const uint16_t*)a.q_i, reps, a.w_i,     \
               a.n_vis, a.nq, a.n, B, p.nb, p.ld1, S1, nqb, nch, chunk, bm_list, bm_fill)
    switch (a.d_i) {
      case 32: HATTN_S1X3(2); break;
      case 64: HATTN_S1X3(4); break;
      default: HATTN_S1X3(8); break;
    }
#undef HATTN_S1X3
  } else if (mfma1) {
    const int qpw = a.nq >= 4 ? 4 : 1;  // queries per workgroup
    const int nqg = int((a.nq + qpw - 1) / qpw);
    const int chunk = 64;  // one LDS tile of block means per workgroup
    const int nch = int((p.nb + chunk - 1) / chunk);
    dim3 grid(xcd_grid(nqg, nch), unsigned(a.bt));
    LaunchScope ls("score_stage1_mfma", st);
#define HATTN_S1(T, KQ)                                                                                      \
  if (qpw == 4)                                                                                              \
    HATTN_LAUNCH((score_stage1_kernel<T, KQ, 4>), grid, dim3(256), 0, st, (const T*)a.q_i, reps, a.w_i, \
                 a.n_vis, a.nq, a.n, B, p.nb, p.ld1, S1, nqg, nch, chunk, bm_list, bm_fill);                 \
  else                                                                                                       \
    HATTN_LAUNCH((score_stage1_kernel<T, KQ, 1>), grid, dim3(256), 0, st, (const T*)a.q_i, reps, a.w_i, \
                 a.n_vis, a.nq, a.n, B, p.nb, p.ld1, S1, nqg, nch, chunk, bm_list, bm_fill)
    if (a.dtype == 0) {
      switch (a.d_i) {
        case 16: HATTN_S1(float, 1); break;
        case 32: HATTN_S1(float, 2); break;
        case 64: HATTN_S1(float, 4); break;
        case 128: HATTN_S1(float, 8); break;
        default: HATTN_S1(float, 16); break;  // 256 (stage1_mfma_dim)
      }
    } else {
      switch (a.d_i) {
        case 16: HATTN_S1(uint16_t, 1); break;
        case 32: HATTN_S1(uint16_t, 2); break;
        case 64: HATTN_S1(uint16_t, 4); break;
        case 128: HATTN_S1(uint16_t, 8); break;
        default: HATTN_S1(uint16_t, 16); break;  // 256 (stage1_mfma_dim)
      }
    }
#undef HATTN_S1
  } else if (a.dtype == 0) {
    launch_valu_score<1, float>(a, reps, p.nb, p.nb, nullptr, B, m, p.ld1, S1, st);
  } else {
    launch_valu_score<1, uint16_t>(a, reps, p.nb, p.nb, nullptr, B, m, p.ld1, S1, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    LaunchScope ls("select_blocks", st);
    // Many rows of up to 1,024 blocks: one wave per row (128K chunk, 1,024
    // rows: 16.1 -> 10.3 us).  A few rows (decode) are latency-bound, and
    // there the 512-thread workgroup is faster (8.0 against 12.2 us for
    // 8 rows of 2,048 blocks).  Up to 8,192 blocks: 512 threads (measured
    // faster than 1,024 on these short rows: fewer waves meet at each
    // barrier).
    if (p.nb <= 1024 && p.rows >= 256)
      HATTN_LAUNCH((select_rows_wave_kernel<1, 16>), dim3(unsigned(p.rows)), dim3(kWave), 0, st, S1, p.ld1,
                   a.n_vis, nullptr, a.n, B, m, m, blk_out, nullptr, bm_list, a.nq, p.nb);
    else if (p.nb <= kSelIT * 512)
      HATTN_LAUNCH((select_rows_kernel<1, 512>), dim3(unsigned(p.rows)), dim3(512), 0, st, S1, p.ld1, a.n_vis,
                   nullptr, a.n, B, m, m, blk_out, nullptr, bm_list, a.nq, p.nb);
    else
      HATTN_LAUNCH((select_rows_kernel<1, kSelNT>), dim3(unsigned(p.rows)), dim3(kSelNT), 0, st, S1, p.ld1,
                   a.n_vis, nullptr, a.n, B, m, m, blk_out, nullptr, bm_list, a.nq, p.nb);
  }
  return hipGetLastError();
}

hipError_t launch_hisa_topk(const IndexArgs& a, const float* reps, int B, int m, int k, int32_t* idx, int32_t* blk,
                            void* ws, hipStream_t st, bool stage1_done) {
  set_lds_limits();
  const HisaPlan p = plan_hisa(a, B, m);
  char* base = reinterpret_cast<char*>(ws);
  float* S1 = reinterpret_cast<float*>(base);
  int32_t* blk_ws = reinterpret_cast<int32_t*>(base + p.s1_bytes);
  float* S2 = reinterpret_cast<float*>(base + p.s1_bytes + p.blk_bytes);
  int32_t* blk_out = blk ? blk : blk_ws;

  // Stage 1: block scores and the top-m blocks.  (The block-major stage 2
  // needs the stage-1 MFMA kernel, which clears its chooser lists.)
  const bool bm = p.bm && a.h_i == 16 && stage1_mfma_dim(a.d_i);
  int32_t* bm_list = bm ? reinterpret_cast<int32_t*>(base + p.s1_bytes + p.blk_bytes + p.s2_bytes) : nullptr;
  hipError_t e = launch_hisa_blocks(a, reps, B, m, p, S1, blk_out, bm_list, stage1_done, st);
  if (e != hipSuccess) return e;

  // Stage 2: token scores inside the chosen blocks.
  const bool mfma2 = a.dtype == 1 && a.h_i == 16 && B % 16 == 0 &&
                     (a.d_i == 32 || a.d_i == 64 || a.d_i == 128 || a.d_i == 256);
  if (bm) {
    // Workgroups per block: about two groups of 16 choosers each on average
    // (each workgroup first loads the block's keys and its first group's
    // queries; fewer, longer workgroups amortise that).
    const int64_t groups = (a.bt * a.nq * m + 16 * a.bt * p.nb - 1) / (16 * a.bt * p.nb);
    const int nslice = int(std::max<int64_t>(1, std::min<int64_t>(16, (groups + 1) / 2)));
    dim3 grid(unsigned(nslice), unsigned(p.nb), unsigned(a.bt));
    LaunchScope ls("score_stage2_bm", st);
#define HATTN_S2BM(KS)                                                                                       \
  HATTN_LAUNCH(score_stage2_bm_kernel<KS>, grid, dim3(256), size_t(a.nq) * 4, st, (const uint16_t*)a.q_i,   \
               (const uint16_t*)a.k_i, a.w_i, a.n_vis, bm_list, a.nq, a.n, B, m, p.nb, p.ld2, S2, nslice)
    switch (a.d_i) {
      case 32: HATTN_S2BM(2); break;
      case 64: HATTN_S2BM(4); break;
      default: HATTN_S2BM(8); break;
    }
#undef HATTN_S2BM
  } else if (mfma2) {
    const int halves = B > 64 ? 2 : 1;  // 64-key tile groups per chosen block
    dim3 grid(unsigned(m * halves), unsigned(p.rows));
    LaunchScope ls("score_stage2_mfma", st);
#define HATTN_S2(KS)                                                                                         \
  HATTN_LAUNCH(score_stage2_mfma_kernel<KS>, grid, dim3(64), 0, st, (const uint16_t*)a.q_i,           \
                     (const uint16_t*)a.k_i, a.w_i, a.n_vis, blk_out, a.nq, a.n, B, m, p.ld2, S2, halves)
    switch (a.d_i) {
      case 32: HATTN_S2(1); break;
      case 64: HATTN_S2(2); break;
      case 128: HATTN_S2(4); break;
      default: HATTN_S2(8); break;
    }
#undef HATTN_S2
  } else if (a.dtype == 0) {
    launch_valu_score<2, float>(a, (const float*)a.k_i, a.n, int64_t(m) * B, blk_out, B, m, p.ld2, S2, st);
  } else {
    launch_valu_score<2, uint16_t>(a, (const uint16_t*)a.k_i, a.n, int64_t(m) * B, blk_out, B, m, p.ld2, S2, st);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    LaunchScope ls("select_tokens", st);
    // as for flat rows: 512 threads when many rows share the chip.  A few
    // rows keep 1,024 (decode, 8 rows of 8,192 candidates: 11.1-11.3 us
    // against 11.4-11.8 us with 512 threads and 16 keys per lane)
    if (p.rows >= 256 && m <= 512 && int64_t(m) * B <= kSelIT * 512)
      HATTN_LAUNCH((select_rows_kernel<2, 512>), dim3(unsigned(p.rows)), dim3(512), 0, st, S2, p.ld2, a.n_vis,
                   blk_out, a.n, B, m, k, idx, nullptr, nullptr, int64_t(1), int64_t(1));
    else if (m <= kSelNT)
      HATTN_LAUNCH((select_rows_kernel<2, kSelNT>), dim3(unsigned(p.rows)), dim3(kSelNT), 0, st, S2, p.ld2,
                   a.n_vis, blk_out, a.n, B, m, k, idx, nullptr, nullptr, int64_t(1), int64_t(1));
    else
      HATTN_LAUNCH((select_rows_kernel<3, kSelNT>), dim3(unsigned(p.rows)), dim3(kSelNT), 0, st, S2, p.ld2,
                   a.n_vis, blk_out, a.n, B, m, k, idx, nullptr, nullptr, int64_t(1), int64_t(1));
  }
  return hipGetLastError();
}

hipError_t launch_block_sparse(const IndexArgs& a, const float* reps, int B, int m, int32_t* idx, int32_t* blk,
                               void* ws, hipStream_t st) {
  const HisaPlan p = plan_hisa(a, B, m);
  char* base = reinterpret_cast<char*>(ws);
  float* S1 = reinterpret_cast<float*>(base);
  int32_t* blk_out = blk ? blk : reinterpret_cast<int32_t*>(base + p.s1_bytes);
  hipError_t e = launch_hisa_blocks(a, reps, B, m, p, S1, blk_out, nullptr, false, st);
  if (e != hipSuccess) return e;
  LaunchScope ls("expand_blocks", st);
  HATTN_LAUNCH(expand_blocks_kernel, dim3(unsigned((int64_t(m) * B + 255) / 256), unsigned(p.rows)), dim3(256), 0,
               st, blk_out, a.n_vis, a.n, B, m, idx);
  return hipGetLastError();
}

}  // namespace hattn
