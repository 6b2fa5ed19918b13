// MQA attention over compressed entries plus a sliding window of raw tokens.
//
// [HYB] process-cxr.github.io "Hybrid Attention", section Compressed Sparse
// Attention (attend to selected positions only) and [HCA] daiw.net
// "前代 · HCA：128 倍压缩后再做稠密注意力", sections 128 倍是什么概念 / 怎么压
// (dense attention over every compressed entry; all query heads share one
// K/V; an extra branch over the latest 128 raw tokens).  One softmax runs
// over the union of a query's compressed keys and its window rows.
//
// Each query's key list is cut into chunks; a workgroup handles one (query,
// chunk) pair and all heads (MQA: every head reads the same K/V, so the
// chunk crosses HBM once).  K|V rows of 64 keys are staged in LDS; each wave
// owns 16 heads:
//   S^T = K . Q^T    16x16x32 bf16 MFMA, A = K rows from LDS, B = Q in VGPRs
//   online softmax   per head in the log2 domain, fp32
//   O^T += V^T . P^T A = V columns gathered from LDS, B = P (bf16) straight
//                    from the S^T accumulators (no re-layout needed)
// With more than one chunk per query the unnormalised (O, max, sum) partials
// are combined by a second kernel with the log-sum-exp identity.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace hattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Source row of virtual key j of a query: compressed keys first, then the
// window rows.  Returns nullptr for skipped keys (index -1 / out of range).
template <typename T, bool SPARSE>
HATTN_DEV const T* key_row(int64_t j, int64_t nc, const int32_t* idx_row, const T* ckv_b, int64_t n, const T* raw_b,
                           int64_t L, int64_t p, int nw, int C) {
  if (j < nc) {
    const int64_t e = SPARSE ? int64_t(idx_row[j]) : j;
    if (e < 0 || e >= n) return nullptr;
    return ckv_b + e * C;
  }
  const int64_t r = p - nw + 1 + (j - nc);
  if (r < 0 || r >= L) return nullptr;
  return raw_b + r * C;
}

template <int D, int NW, bool SPARSE>
__global__ __launch_bounds__(64 * NW) void attn_mfma_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ ckv, int64_t n,
                                                            const int32_t* __restrict__ idx, int k,
                                                            const int32_t* __restrict__ n_vis,
                                                            const uint16_t* __restrict__ raw, int64_t L,
                                                            const int32_t* __restrict__ q_pos, int window,
                                                            float scale_log2, int64_t nq, int chunk, int nsplit,
                                                            float* __restrict__ out, float* __restrict__ lse,
                                                            float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int H = 16 * NW;
  constexpr int C = 2 * D;
  constexpr int TK = 64;
  constexpr int PITCH = C + 8;
  constexpr int NT = 64 * NW;
  constexpr int PPR = C / 8;                // 16-byte pieces per row
  constexpr int PIECES = TK * PPR / NT;     // per thread per tile
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  static_assert(TK * PPR % NT == 0, "tile split");
  __shared__ __align__(16) uint16_t tile[TK * PITCH];
  __shared__ uint64_t vmask;

  const int64_t qrow = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t b = qrow / nq;
  const int64_t p = q_pos[qrow];
  const int nw = int(imax64(0, imin64(window, p + 1)));
  const int64_t nc = SPARSE ? int64_t(k) : imin64(n, imax64(0, n_vis[qrow]));
  const int64_t total = nc + nw;
  const int64_t j_begin = int64_t(split) * chunk;
  const int64_t j_end = imin64(total, j_begin + chunk);
  const int32_t* idx_row = SPARSE ? idx + qrow * k : nullptr;
  const uint16_t* ckv_b = ckv + b * n * C;
  const uint16_t* raw_b = raw + b * L * C;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int head = 16 * wave + r16;

  u32x4_t qf[KS];
  {
    const uint16_t* qp = q + (qrow * H + head) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = ld16(qp + 32 * ks);
  }
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  u32x4_t pre[PIECES];
  auto prefetch = [&](int64_t j0) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pidx = tid + NT * u;
      const int row = pidx / PPR, col = pidx % PPR;
      const int64_t j = j0 + row;
      const uint16_t* src =
          j < j_end ? key_row<uint16_t, SPARSE>(j, nc, idx_row, ckv_b, n, raw_b, L, p, nw, C) : nullptr;
      pre[u] = src ? ld16(src + col * 8) : u32x4_t{0, 0, 0, 0};
    }
  };
  if (j_begin < j_end) prefetch(j_begin);
  for (int64_t j0 = j_begin; j0 < j_end; j0 += TK) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pidx = tid + NT * u;
      const int row = pidx / PPR, col = pidx % PPR;
      *reinterpret_cast<u32x4_t*>(&tile[row * PITCH + col * 8]) = pre[u];
    }
    if (wave == 0) {
      const int64_t j = j0 + lane;
      const bool ok =
          j < j_end && key_row<uint16_t, SPARSE>(j, nc, idx_row, ckv_b, n, raw_b, L, p, nw, C) != nullptr;
      const uint64_t mk = ballot(ok);
      if (lane == 0) vmask = mk;
    }
    __syncthreads();
    if (j0 + TK < j_end) prefetch(j0 + TK);
    const uint64_t mk = vmask;

    // S^T = K . Q^T for 64 keys x 16 heads (this wave's heads).
    f32x4_t s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&tile[(16 * mt + r16) * PITCH + 32 * ks + 8 * g]);
        s[mt] = mfma16x16x32(a, qf[ks], s[mt]);
      }
    }
    // Online softmax (log2 domain) for head r16 of this wave.
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 16 * mt + 4 * g + i;
        const bool ok = (mk >> kk) & 1ull;
        const float x = ok ? s[mt][i] * scale_log2 : -INFINITY;
        s[mt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = m_new == -INFINITY ? 0.f : exp2f(s[mt][i] - m_new);
        s[mt][i] = e;
        psum += e;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

    // O^T += V^T . P^T, two steps of 32 keys.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      u32x4_t pb;
      pb[0] = pack_bf16x2(s[2 * k2][0], s[2 * k2][1]);
      pb[1] = pack_bf16x2(s[2 * k2][2], s[2 * k2][3]);
      pb[2] = pack_bf16x2(s[2 * k2 + 1][0], s[2 * k2 + 1][1]);
      pb[3] = pack_bf16x2(s[2 * k2 + 1][2], s[2 * k2 + 1][3]);
      const int key0 = 32 * k2 + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vcol = &tile[D + 16 * dt + r16];
        u32x4_t va;
        va[0] = uint32_t(vcol[(key0 + 0) * PITCH]) | (uint32_t(vcol[(key0 + 1) * PITCH]) << 16);
        va[1] = uint32_t(vcol[(key0 + 2) * PITCH]) | (uint32_t(vcol[(key0 + 3) * PITCH]) << 16);
        va[2] = uint32_t(vcol[(key0 + 16) * PITCH]) | (uint32_t(vcol[(key0 + 17) * PITCH]) << 16);
        va[3] = uint32_t(vcol[(key0 + 18) * PITCH]) | (uint32_t(vcol[(key0 + 19) * PITCH]) << 16);
        o[dt] = mfma16x16x32(va, pb, o[dt]);
      }
    }
    __syncthreads();
  }

  // Lane partial sums cover this lane's keys only; sum over lane groups.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = out + (qrow * H + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4_t v = o[dt] * inv;
      *reinterpret_cast<f32x4_t*>(op + 16 * dt) = v;
    }
    if (lse && g == 0) lse[qrow * H + head] = (m_run + __log2f(l_tot)) * kLn2;
  } else {
    const int64_t pr = qrow * nsplit + split;
    float* op = part_o + (pr * H + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t*>(op + 16 * dt) = o[dt];
    if (g == 0) {
      part_ml[(pr * H + head) * 2 + 0] = m_run;
      part_ml[(pr * H + head) * 2 + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Vector kernel for any dtype and shape (h*d <= 8192): same chunking and
// partial protocol, fp32 throughout.
// ---------------------------------------------------------------------------
template <typename T, bool SPARSE>
__global__ __launch_bounds__(256) void attn_valu_kernel(const T* __restrict__ q, const T* __restrict__ ckv, int64_t n,
                                                        const int32_t* __restrict__ idx, int k,
                                                        const int32_t* __restrict__ n_vis, const T* __restrict__ raw,
                                                        int64_t L, const int32_t* __restrict__ q_pos, int window,
                                                        float scale_log2, int64_t nq, int H, int D, int chunk,
                                                        int nsplit, float* __restrict__ out, float* __restrict__ lse,
                                                        float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int TK = 32;
  constexpr int MAXO = 32;  // outputs per thread: h*d <= 256*32
  extern __shared__ float sm[];
  const int C = 2 * D;
  float* qs = sm;                 // [H][D]
  float* kt = qs + H * D;         // [TK][D]
  float* vt = kt + TK * D;        // [TK][D]
  float* pl = vt + TK * D;        // [H][TK]
  float* mrun = pl + H * TK;      // [H]
  float* lrun = mrun + H;         // [H]
  float* alph = lrun + H;         // [H]
  __shared__ int valid[TK];

  const int64_t qrow = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t b = qrow / nq;
  const int64_t p = q_pos[qrow];
  const int nw = int(imax64(0, imin64(window, p + 1)));
  const int64_t nc = SPARSE ? int64_t(k) : imin64(n, imax64(0, n_vis[qrow]));
  const int64_t total = nc + nw;
  const int64_t j_begin = int64_t(split) * chunk;
  const int64_t j_end = imin64(total, j_begin + chunk);
  const int32_t* idx_row = SPARSE ? idx + qrow * k : nullptr;
  const T* ckv_b = ckv + b * n * C;
  const T* raw_b = raw + b * L * C;
  const int tid = threadIdx.x;

  for (int i = tid; i < H * D; i += 256) qs[i] = to_float(q[qrow * H * D + i]);
  for (int h = tid; h < H; h += 256) {
    mrun[h] = -INFINITY;
    lrun[h] = 0.f;
  }
  float acc[MAXO];
#pragma unroll
  for (int u = 0; u < MAXO; ++u) acc[u] = 0.f;
  __syncthreads();

  for (int64_t j0 = j_begin; j0 < j_end; j0 += TK) {
    for (int i = tid; i < TK * D; i += 256) {
      const int r = i / D, c = i % D;
      const int64_t j = j0 + r;
      const T* src = j < j_end ? key_row<T, SPARSE>(j, nc, idx_row, ckv_b, n, raw_b, L, p, nw, C) : nullptr;
      kt[i] = src ? to_float(src[c]) : 0.f;
      vt[i] = src ? to_float(src[D + c]) : 0.f;
      if (c == 0) valid[r] = src != nullptr;
    }
    __syncthreads();
    for (int i = tid; i < H * TK; i += 256) {
      const int h = i / TK, r = i % TK;
      float dot = 0.f;
      for (int c = 0; c < D; ++c) dot = fmaf(qs[h * D + c], kt[r * D + c], dot);
      pl[i] = valid[r] ? dot * scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int h = tid; h < H; h += 256) {
      float mx = -INFINITY;
      for (int r = 0; r < TK; ++r) mx = fmaxf(mx, pl[h * TK + r]);
      const float m_new = fmaxf(mrun[h], mx);
      const float a = m_new == -INFINITY ? 1.f : exp2f(mrun[h] - m_new);
      float s = 0.f;
      for (int r = 0; r < TK; ++r) {
        const float e = m_new == -INFINITY ? 0.f : exp2f(pl[h * TK + r] - m_new);
        pl[h * TK + r] = e;
        s += e;
      }
      lrun[h] = lrun[h] * a + s;
      mrun[h] = m_new;
      alph[h] = a;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MAXO; ++u) {
      const int i = tid + 256 * u;
      if (i < H * D) {
        const int h = i / D, c = i % D;
        float v = acc[u] * alph[h];
        for (int r = 0; r < TK; ++r) v = fmaf(pl[h * TK + r], vt[r * D + c], v);
        acc[u] = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < MAXO; ++u) {
    const int i = tid + 256 * u;
    if (i < H * D) {
      const int h = i / D;
      if (nsplit == 1) {
        const float l = lrun[h];
        out[qrow * H * D + i] = l > 0.f ? acc[u] / l : 0.f;
      } else {
        part_o[(qrow * nsplit + split) * H * D + i] = acc[u];
      }
    }
  }
  for (int h = tid; h < H; h += 256) {
    if (nsplit == 1) {
      if (lse) lse[qrow * H + h] = (mrun[h] + __log2f(lrun[h])) * kLn2;
    } else {
      part_ml[((qrow * nsplit + split) * H + h) * 2 + 0] = mrun[h];
      part_ml[((qrow * nsplit + split) * H + h) * 2 + 1] = lrun[h];
    }
  }
}

// Combines per-chunk partials: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
__global__ void attn_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int nsplit,
                                  int H, int D, float* __restrict__ out, float* __restrict__ lse) {
  const int64_t qrow = blockIdx.y;
  const int h = blockIdx.x;
  const int c = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((qrow * nsplit + s) * H + h) * 2]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t pr = (qrow * nsplit + s) * H + h;
    const float ms = part_ml[pr * 2];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
    den = fmaf(w, part_ml[pr * 2 + 1], den);
    if (c < D) num = fmaf(w, part_o[pr * D + c], num);
  }
  if (c < D) out[(qrow * H + h) * D + c] = den > 0.f ? num / den : 0.f;
  if (c == 0 && lse) lse[qrow * H + h] = (M + __log2f(den)) * kLn2;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static bool mfma_shape(const AttnArgs& a) {
  return a.dtype == 1 && (a.d == 64 || a.d == 128) && (a.h == 16 || a.h == 32 || a.h == 64);
}

bool attn_supported(const AttnArgs& a) {
  if (mfma_shape(a)) return true;
  return a.h * a.d <= 256 * 32 && a.d <= 256;
}

struct AttnPlan {
  int chunk, nsplit;
  size_t po_bytes, total;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static AttnPlan plan_attn(const AttnArgs& a) {
  AttnPlan p{};
  const int tk = mfma_shape(a) ? 64 : 32;
  const int64_t rows = a.bt * a.nq;
  const int64_t maxkeys = (a.idx ? int64_t(a.k) : a.n) + a.window;
  // Aim for about four workgroups per compute unit overall, never a chunk
  // under 256 keys (partials cost 32 KiB per chunk and query).
  const int64_t target_wg = 1024;
  int64_t chunk = (rows * maxkeys + target_wg - 1) / target_wg;
  chunk = std::max<int64_t>(chunk, 256);
  chunk = (chunk + tk - 1) / tk * tk;
  if (chunk >= maxkeys) chunk = (maxkeys + tk - 1) / tk * tk;
  p.chunk = int(chunk);
  p.nsplit = int((maxkeys + chunk - 1) / chunk);
  if (p.nsplit > 1) {
    p.po_bytes = align256(size_t(rows) * p.nsplit * a.h * a.d * 4);
    p.total = p.po_bytes + align256(size_t(rows) * p.nsplit * a.h * 2 * 4);
  }
  return p;
}

size_t attn_ws_bytes(const AttnArgs& a) { return plan_attn(a).total; }

template <bool SPARSE>
static void launch_attn_mfma(const AttnArgs& a, const AttnPlan& pl, float* po, float* pml, hipStream_t st) {
  const float sl2 = a.scale * kLog2e;
  dim3 grid(unsigned(pl.nsplit), unsigned(a.bt * a.nq));
#define HATTN_ATTN(D, NW)                                                                                      \
  hipLaunchKernelGGL((attn_mfma_kernel<D, NW, SPARSE>), grid, dim3(64 * NW), 0, st, (const uint16_t*)a.q,      \
                     (const uint16_t*)a.ckv, a.n, a.idx, a.k, a.n_vis, (const uint16_t*)a.raw_kv, a.L, a.q_pos, \
                     a.window, sl2, a.nq, pl.chunk, pl.nsplit, a.out, a.lse, po, pml)
  const int nw = a.h / 16;
  if (a.d == 128) {
    switch (nw) {
      case 1: HATTN_ATTN(128, 1); break;
      case 2: HATTN_ATTN(128, 2); break;
      default: HATTN_ATTN(128, 4); break;
    }
  } else {
    switch (nw) {
      case 1: HATTN_ATTN(64, 1); break;
      case 2: HATTN_ATTN(64, 2); break;
      default: HATTN_ATTN(64, 4); break;
    }
  }
#undef HATTN_ATTN
}

template <typename T, bool SPARSE>
static void launch_attn_valu(const AttnArgs& a, const AttnPlan& pl, float* po, float* pml, hipStream_t st) {
  const float sl2 = a.scale * kLog2e;
  dim3 grid(unsigned(pl.nsplit), unsigned(a.bt * a.nq));
  const size_t smem = size_t(a.h) * a.d * 4 + 2 * 32 * size_t(a.d) * 4 + size_t(a.h) * 32 * 4 + 3 * size_t(a.h) * 4;
  hipLaunchKernelGGL((attn_valu_kernel<T, SPARSE>), grid, dim3(256), smem, st, (const T*)a.q, (const T*)a.ckv, a.n,
                     a.idx, a.k, a.n_vis, (const T*)a.raw_kv, a.L, a.q_pos, a.window, sl2, a.nq, a.h, a.d, pl.chunk,
                     pl.nsplit, a.out, a.lse, po, pml);
}

hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t st) {
  const AttnPlan pl = plan_attn(a);
  float* po = nullptr;
  float* pml = nullptr;
  if (pl.nsplit > 1) {
    po = reinterpret_cast<float*>(ws);
    pml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + pl.po_bytes);
  }
  const bool sparse = a.idx != nullptr;
  {
    LaunchScope ls(mfma_shape(a) ? (sparse ? "attn_sparse_mfma" : "attn_dense_mfma")
                                 : (sparse ? "attn_sparse_valu" : "attn_dense_valu"),
                   st);
    if (mfma_shape(a)) {
      if (sparse) launch_attn_mfma<true>(a, pl, po, pml, st);
      else launch_attn_mfma<false>(a, pl, po, pml, st);
    } else if (a.dtype == 0) {
      if (sparse) launch_attn_valu<float, true>(a, pl, po, pml, st);
      else launch_attn_valu<float, false>(a, pl, po, pml, st);
    } else {
      if (sparse) launch_attn_valu<uint16_t, true>(a, pl, po, pml, st);
      else launch_attn_valu<uint16_t, false>(a, pl, po, pml, st);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  LaunchScope ls("attn_merge", st);
  hipLaunchKernelGGL(attn_merge_kernel, dim3(unsigned(a.h), unsigned(a.bt * a.nq)), dim3(unsigned(a.d)), 0, st, po,
                     pml, pl.nsplit, a.h, a.d, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace hattn
