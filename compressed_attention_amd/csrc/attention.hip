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
#include <mutex>

#include "common.h"
#include "internal.h"

namespace hattn {

// Device scratch for callers that cannot allocate (hattn_sparse_attn_noalloc):
// the split-K partials of one attention call.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSparseChunkMax = 2048;  // keys per sparse MFMA workgroup (their indices are staged in LDS)
constexpr float kLn2 = 0.6931471805599453f;

// Source row of virtual key j of a query: compressed keys first, then the
// window rows.  Returns nullptr for skipped keys (index -1 / out of range).
template <typename T, bool SPARSE>
HATTN_DEV const T* key_row(int64_t j, int64_t nc, const int32_t* idx_row, const T* ckv_b, int64_t n, const T* raw_b,
                           int64_t L, int64_t p, int nw, int C, int R) {
  if (j < nc) {
    const int64_t e = SPARSE ? int64_t(idx_row[j]) : j;
    if (e < 0 || e >= n) return nullptr;
    return ckv_b + e * C;
  }
  const int64_t r = p - nw + 1 + (j - nc);
  if (r < 0 || r >= L) return nullptr;
  return raw_b + (R ? r % R : r) * C;  // R > 0: the raw rows are a ring of R
}

// Source row of virtual key j (0 <= j < 2^31) for the MFMA kernel, computed
// branch-free in 32-bit arithmetic (each sequence's cache holds fewer than
// 2^31 elements, checked on the host).  `ok` says whether the key exists;
// when it does not, the row is row 0 of the raw sequence (always valid,
// L >= 1) and its data is never used.  Sparse indices come from the
// workgroup's LDS copy of its chunk (sidx[t] = index of key j_base + t, for
// the chunk's compressed keys), read at a clamped slot.
template <bool SPARSE>
HATTN_DEV const uint16_t* key_src32(int j, int j_end, int nc, const int32_t* sidx, int j_base,
                                    const uint16_t* ckv_b, int n, const uint16_t* raw_b, int L, int rbase, int C,
                                    bool* ok, int R = 0) {
  const bool in_c = j < nc;
  int e;
  if (SPARSE) e = sidx[in_c && j < j_end ? j - j_base : 0];
  else e = j;
  const int r = rbase + j;  // rbase = p - nw + 1 - nc
  const bool okc = in_c && unsigned(e) < unsigned(n);
  const bool okr = !in_c && unsigned(r) < unsigned(L);
  const bool v = j < j_end && (okc || okr);
  *ok = v;
  const int slot = R && okr ? r % R : r;  // raw rows in a ring: slot r % R
  const unsigned off = v ? unsigned(okc ? e : slot) * unsigned(C) : 0u;
  return (v && okc ? ckv_b : raw_b) + off;
}

// MFMA attention workgroup: one query, one chunk of its key list, 16 heads
// per wave (H = 16*NW), head dim D.  Tiles of 64 keys are shared by the
// waves through LDS (small enough that the prefetch registers leave room for
// the compiler to keep several LDS operand reads in flight per MFMA chain):
//   load    the next tile's K|V rows into registers (16-byte loads) while
//           the current tile is computed
//   S^T     = K . Q^T   (A = K rows via ds_read_b128, B = Q in VGPRs)
//   softmax per head in the log2 domain; the reference maximum moves only
//           when a tile maximum exceeds it by more than 8, so O and l are
//           rescaled rarely and P stays below 2^8
//   O^T    += V^T . P^T (A = V columns via the gfx950 LDS transpose read,
//           B = P straight from the S^T accumulators, no re-layout)
// The workgroup writes the normalised output, or an unnormalised partial
// (O, max, sum) when the key list is split over several workgroups.
// Arguments of one MFMA attention launch (one query set).
struct AttnK {
  const uint16_t* q;
  const uint16_t* ckv;
  int64_t n;
  const int32_t* idx;
  int k;
  const int32_t* n_vis;
  const uint16_t* raw;
  int64_t L;
  const int32_t* q_pos;
  int window;
  float scale_log2;
  int64_t nq;
  int chunk, nsplit;
  float* out;
  float* lse;
  _Float16* part_o;  // split-K partials: O / l of the split (scaled), fp16
  float* part_ml;    // per head: (max, sum, multiplier of part_o, 0), fp32
  // Head groups of a query row: the row has 16 * NW * hg heads and a
  // workgroup takes one group of 16 * NW (layers that share one cache and
  // one selection fold into the head axis: MQA heads share every key).
  int hg = 1;
  // Raw rows held per sequence: 0 = all L (row r at r); R > 0 = a ring
  // holding the newest R rows (row r at slot r % R).
  int R = 0;
};

template <int D>
struct AttnLds {
  static constexpr int TK = 64, KP = D + 8, VP = D + 16;
  __align__(16) uint16_t kt[TK * KP];
  __align__(16) uint16_t vt[TK * VP];
  uint64_t vmask[TK / 64];
};

// STREAM: K|V rows are read once by the launch (one query per sequence), so
// they are loaded non-temporally; otherwise the queries of a sequence share
// its cache and plain loads keep it in L2.  (A template parameter: the
// compiler merges a runtime choice between the two loads into a plain one.)
template <int D, int NW, bool SPARSE, bool STREAM>
HATTN_DEV void attn_mfma_body(const AttnK& a, int split, int64_t qrow, AttnLds<D>& lds, int32_t* sidx,
                              int hgroup = 0) {
  const uint16_t* __restrict__ q = a.q;
  const uint16_t* __restrict__ ckv = a.ckv;
  const int64_t n = a.n;
  const int32_t* __restrict__ idx = a.idx;
  const int k = a.k;
  const int32_t* __restrict__ n_vis = a.n_vis;
  const uint16_t* __restrict__ raw = a.raw;
  const int64_t L = a.L;
  const int32_t* __restrict__ q_pos = a.q_pos;
  const int window = a.window;
  const float scale_log2 = a.scale_log2;
  const int64_t nq = a.nq;
  const int chunk = a.chunk, nsplit = a.nsplit;
  float* __restrict__ out = a.out;
  float* __restrict__ lse = a.lse;
  _Float16* __restrict__ part_o = a.part_o;
  float* __restrict__ part_ml = a.part_ml;
  constexpr int H = 16 * NW;
  constexpr int C = 2 * D;
  constexpr int TK = 64;      // keys per tile (32 KiB of K|V at d = 128)
  constexpr int MT = TK / 16;
  constexpr int KP = D + 8;   // K rows 4 banks apart: conflict-free b128 operand reads
  constexpr int VP = D + 16;  // V rows 8 banks apart: conflict-free transpose reads
  constexpr int NT = 64 * NW;
  constexpr int PPR = C / 8;             // 16-byte pieces per row
  constexpr int PIECES = TK * PPR / NT;  // per thread per tile
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  static_assert(TK * PPR % NT == 0, "tile split");
  uint16_t* kt = lds.kt;
  uint16_t* vt = lds.vt;
  uint64_t* vmask = lds.vmask;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int HT = H * a.hg;                        // heads of the query row
  const int head = hgroup * H + 16 * wave + r16;  // this lane's head in the row
  // Loads that need no other load go first: the query fragments and the
  // speculative first tile below.
  u32x4_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = ld16(q + (qrow * HT + head) * D + 32 * ks + 8 * g);
  const int64_t b = idiv(qrow, nq);
  const int j_begin = split * chunk;
  const uint16_t* ckv_b = ckv + b * n * C;
  // Dense chunks whose first tile lies inside the cache (rows j_begin ..
  // j_begin + TK - 1 < n) issue that tile's loads before the query's
  // position and visible count arrive, so the first tile costs one memory
  // round trip instead of two.  The data is kept when the tile is a plain
  // run of compressed rows (exactly the rows fetch() reads then), and
  // fetched again otherwise.
  const bool spec = !SPARSE && int64_t(j_begin) + TK <= n;
  u32x4_t pre[PIECES];
  if (spec) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pidx = tid + NT * u;
      const uint16_t* src = ckv_b + size_t(j_begin) * C + (pidx / PPR) * C + (pidx % PPR) * 8;
      pre[u] = STREAM ? ld16_nt(src) : ld16(src);
    }
  }
  const int64_t p = q_pos[qrow];
  const int64_t nv_raw = SPARSE ? 0 : n_vis[qrow];
  const int nw = int(imax64(0, imin64(window, p + 1)));
  const int64_t nc = SPARSE ? int64_t(k) : imin64(n, imax64(0, nv_raw));
  const int total = int(nc) + nw;
  const int j_end = min(total, j_begin + chunk);
  const int32_t* idx_row = SPARSE ? idx + qrow * k : nullptr;
  const int R = a.R;
  const uint16_t* raw_b = raw + b * (R ? int64_t(R) : L) * C;
  const int rbase = int(p) - nw + 1 - int(nc);
  const int n32 = int(n), L32 = int(L), nc32 = int(nc);

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // A tile is "plain" when all its TK keys exist and sit in one contiguous
  // run of rows (dense entries, or window rows): then row r is base + r*C
  // and every key is valid.  Other tiles take the general per-row path.
  auto plain_base = [&](int j0) -> const uint16_t* {
    if (SPARSE || j0 + TK > j_end) return nullptr;
    if (j0 + TK <= nc32) return ckv_b + size_t(j0) * C;
    if (j0 >= nc32) {
      // window rows rbase + j0 .. + TK - 1 (>= 0): contiguous unless they
      // wrap around the ring
      const int r0 = rbase + j0;
      if (!R) return raw_b + size_t(r0) * C;
      const int s0 = r0 % R;
      return s0 + TK <= R ? raw_b + size_t(s0) * C : nullptr;
    }
    return nullptr;
  };
  auto fetch = [&](int j0) {
    const uint16_t* base = plain_base(j0);
    if (base) {
#pragma unroll
      for (int u = 0; u < PIECES; ++u) {
        const int pidx = tid + NT * u;
        const uint16_t* src = base + (pidx / PPR) * C + (pidx % PPR) * 8;
        pre[u] = STREAM ? ld16_nt(src) : ld16(src);
      }
    } else {
#pragma unroll
      for (int u = 0; u < PIECES; ++u) {
        const int pidx = tid + NT * u;
        bool ok;
        // Skipped keys read raw row 0 (finite data); their logits are masked.
        const uint16_t* src = key_src32<SPARSE>(j0 + pidx / PPR, j_end, nc32, sidx, j_begin, ckv_b, n32, raw_b,
                                                L32, rbase, C, &ok, R);
        pre[u] = STREAM ? ld16_nt(src + (pidx % PPR) * 8) : ld16(src + (pidx % PPR) * 8);
      }
    }
  };
  if (SPARSE) {
    // Stage the chunk's indices once: every tile then computes its row
    // addresses from LDS instead of a dependent global load.  (The chunk's
    // compressed keys end at min(j_begin + chunk, k) whatever the window
    // length, so these loads need not wait for the query position.)
    const int cend = min(j_begin + chunk, nc32);
    for (int t = tid; j_begin + t < cend; t += NT) sidx[t] = idx_row[j_begin + t];
    __syncthreads();
  }
  // the speculative tile is the one fetch() would load iff plain_base(j_begin)
  // is ckv_b + j_begin * C
  const bool spec_ok = spec && j_begin + TK <= j_end && j_begin + TK <= nc32;
  if (j_begin < j_end && !spec_ok) fetch(j_begin);
  for (int j0 = j_begin; j0 < j_end; j0 += TK) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pidx = tid + NT * u;
      const int row = pidx / PPR, col = pidx % PPR;
      uint16_t* dst = col < PPR / 2 ? kt + row * KP + col * 8 : vt + row * VP + (col - PPR / 2) * 8;
      *reinterpret_cast<u32x4_t*>(dst) = pre[u];
    }
    const bool plain = plain_base(j0) != nullptr;  // uniform: every key valid
    if (!plain && wave == 0) {
#pragma unroll
      for (int h = 0; h < TK / 64; ++h) {
        bool ok;
        key_src32<SPARSE>(j0 + 64 * h + lane, j_end, nc32, sidx, j_begin, ckv_b, n32, raw_b, L32, rbase, C, &ok, R);
        const uint64_t mk = ballot(ok);
        if (lane == 0) vmask[h] = mk;
      }
    }
    __syncthreads();
    if (j0 + TK < j_end) fetch(j0 + TK);

    f32x4_t s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kt + (16 * mt + r16) * KP + 32 * ks + 8 * g);
        s[mt] = mfma16x16x32(a, qf[ks], s[mt]);
      }

    float mx = -INFINITY;
    if (plain) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[mt][i] *= scale_log2;
          mx = fmaxf(mx, s[mt][i]);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint64_t mk = vmask[mt >> 2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = (16 * mt + 4 * g + i) & 63;
          const float x = ((mk >> kk) & 1ull) ? s[mt][i] * scale_log2 : -INFINITY;
          s[mt][i] = x;
          mx = fmaxf(mx, x);
        }
      }
    }
    mx = max_groups(mx);  // over the four lane groups: lane swaps, no LDS
    const bool up = mx > m_run + 8.f;  // false while mx is -inf
    if (__any(up)) {
      const float m_new = up ? mx : m_run;
      // o and l are still zero while the reference is -inf
      const float a = (up && m_run != -INFINITY) ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= a;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= a;
      m_run = m_new;
    }
    // exp2 of -inf (masked key) is +0; a reference that is still -inf means
    // every key so far was masked, and then all weights are 0.
    const float mref = m_run == -INFINITY ? INFINITY : m_run;
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(s[mt][i] - mref);
        s[mt][i] = e;
        psum += e;
      }
    l_run += psum;

    // k-slots of lane group g in step k2: keys 32k2+4g..+3, then 32k2+16+4g..+3.
#pragma unroll
    for (int k2 = 0; k2 < TK / 32; ++k2) {
      u32x4_t pb;
      pb[0] = pack_bf16x2_hw(s[2 * k2][0], s[2 * k2][1]);
      pb[1] = pack_bf16x2_hw(s[2 * k2][2], s[2 * k2][3]);
      pb[2] = pack_bf16x2_hw(s[2 * k2 + 1][0], s[2 * k2 + 1][1]);
      pb[3] = pack_bf16x2_hw(s[2 * k2 + 1][2], s[2 * k2 + 1][3]);
      const uint16_t* vb = vt + (32 * k2 + 4 * g + (r16 >> 2)) * VP + 4 * (r16 & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2_t lo = lds_read_tr16(vb + 16 * dt);
        const u32x2_t hi = lds_read_tr16(vb + 16 * VP + 16 * dt);
        const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
        o[dt] = mfma16x16x32(va, pb, o[dt]);
      }
    }
    __syncthreads();
  }

  // Lane partial sums cover this lane's keys only; sum over lane groups.
  const float l_tot = sum_groups(l_run);
  if (nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = out + (qrow * HT + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t*>(op + 16 * dt) = o[dt] * inv;
    if (lse && g == 0) lse[qrow * HT + head] = (m_run + __log2f(l_tot)) * kLn2;
  } else {
    // The split's output normalised by its own sum (|O / l| <= max |V|),
    // stored in fp16 after a power-of-two scaling 2^-sh that keeps the
    // head's largest value below 2^15 (sh = 0, no scaling, unless |V|
    // exceeds fp16's range).  The record holds the multiplier 2^sh; the
    // merge weights the split by 2^(m - M) l and that multiplier.
    const int64_t pr = qrow * nsplit + split;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] *= inv;
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[dt][i]));
    }
    amax = max_groups(amax);  // the head's values sit in its four lane groups
    const int ex = int((__float_as_uint(amax) >> 23) & 0xffu) - 127;  // amax in [2^ex, 2^(ex+1))
    const int sh = max(0, ex - 14);                                   // <= 113 for finite values
    const float down = __uint_as_float(uint32_t(127 - sh) << 23);     // 2^-sh
    _Float16* op = part_o + (pr * HT + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4_t v = o[dt] * down;
      *reinterpret_cast<f16x4_t*>(op + 16 * dt) =
          f16x4_t{_Float16(v[0]), _Float16(v[1]), _Float16(v[2]), _Float16(v[3])};
    }
    if (g == 0)
      *reinterpret_cast<f32x4_t*>(part_ml + (pr * HT + head) * 4) =
          f32x4_t{m_run, l_tot, __uint_as_float(uint32_t(127 + sh) << 23), 0.f};
  }
}

template <int D, int NW, bool SPARSE, bool STREAM>
__global__ __launch_bounds__(64 * NW, 2) void attn_mfma_kernel(AttnK a) {
  __shared__ AttnLds<D> lds;
  __shared__ int32_t sidx[SPARSE ? kSparseChunkMax : 1];  // this chunk's compressed indices
  attn_mfma_body<D, NW, SPARSE, STREAM>(a, blockIdx.x, blockIdx.y, lds, sidx, blockIdx.z);
}

// A sparse and a dense query set in one launch (e.g. the CSA and HCA
// branches of one decode step): a 1-D grid whose first s.nsplit * rows_s
// workgroups take the sparse (query, chunk) pairs and the rest the dense
// ones.  Both roles share one set of LDS buffers.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_pair_kernel(AttnK s, int64_t rows_s, AttnK d) {
  __shared__ AttnLds<D> lds;
  __shared__ int32_t sidx[kSparseChunkMax];
  const int64_t id = blockIdx.x;
  const int64_t ns = int64_t(s.nsplit) * rows_s;
  if (id < ns) {
    const int64_t row = idiv(id, s.nsplit);
    attn_mfma_body<D, NW, true, true>(s, int(id - row * s.nsplit), row, lds, sidx);
  } else {
    const int64_t row = idiv(id - ns, d.nsplit);
    attn_mfma_body<D, NW, false, true>(d, int(id - ns - row * d.nsplit), row, lds, sidx);
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
                                                        float* __restrict__ part_o, float* __restrict__ part_ml,
                                                        int R) {
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
  const int64_t b = idiv(qrow, nq);
  const int64_t p = q_pos[qrow];
  const int nw = int(imax64(0, imin64(window, p + 1)));
  const int64_t nc = SPARSE ? int64_t(k) : imin64(n, imax64(0, n_vis[qrow]));
  const int64_t total = nc + nw;
  const int64_t j_begin = int64_t(split) * chunk;
  const int64_t j_end = imin64(total, j_begin + chunk);
  const int32_t* idx_row = SPARSE ? idx + qrow * k : nullptr;
  const T* ckv_b = ckv + b * n * C;
  const T* raw_b = raw + b * (R ? int64_t(R) : L) * C;
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
      const T* src = j < j_end ? key_row<T, SPARSE>(j, nc, idx_row, ckv_b, n, raw_b, L, p, nw, C, R) : nullptr;
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
      const float l = lrun[h];
      const float v = l > 0.f ? acc[u] / l : 0.f;
      if (nsplit == 1) out[qrow * H * D + i] = v;
      else part_o[(qrow * nsplit + split) * H * D + i] = v;  // normalised, as the MFMA kernel's (fp32 here)
    }
  }
  for (int h = tid; h < H; h += 256) {
    if (nsplit == 1) {
      if (lse) lse[qrow * H + h] = (mrun[h] + __log2f(lrun[h])) * kLn2;
    } else {
      float* rec = part_ml + ((qrow * nsplit + split) * H + h) * 4;  // (max, sum, multiplier 1, 0)
      rec[0] = mrun[h];
      rec[1] = lrun[h];
      rec[2] = 1.f;
      rec[3] = 0.f;
    }
  }
}

// Combines per-chunk partials, each stored as its normalised output
// u_s = O_s / l_s divided by a power-of-two multiplier c_s (PT: fp16 from
// the bf16 MFMA kernels, fp32 with c_s = 1 from the vector kernel) with a
// record (m_s, l_s, c_s, 0): o = sum_s w_s c_s (u_s / c_s) with weights
// w_s = 2^(m_s - M) l_s / sum_t 2^(m_t - M) l_t.  Needs nsplit <= 4 *
// kMergeRegs and a head shape merge_fast() accepts.
constexpr int kMergeRegs = 16;
constexpr int kMergeMaxSplit = 4 * kMergeRegs;

// Arguments of one merge (one query set's partials).
template <typename PT>
struct MergeK {
  const PT* part_o;
  const float* part_ml;
  int nsplit;
  float* out;
  float* lse;
};

static bool merge_fast(int h, int d, int nsplit) {
  return d % 64 == 0 && d <= 256 && (h * d) % 256 == 0 && nsplit <= kMergeMaxSplit;
}

struct MergeLds {
  float w[4][kMergeMaxSplit];  // weight of split s for each head of the group
  f32x4_t red[4][64];
};

// One workgroup merges 256 consecutive outputs [e0, e0 + 256) of row qrow
// (256 / D heads; d % 4 == 0 and h * d % 256 == 0).  Lane l of every wave
// holds outputs e0 + 4l .. 4l + 3 (one head), and wave g sums splits
// g, g + 4, ...: all partial loads and, in wave 0, the heads' (m_s, l_s)
// loads are issued before anything waits, so the merge is one memory round
// trip.  Wave 0 turns (m_s, l_s) into per-split weights (exp2(m_s - M) l_s /
// den with M the heads' largest m_s), the waves weight their partials, and
// the four group sums are added through LDS in group order.
// 4 consecutive partial values as loaded (Vec4<PT>::type) and as fp32.  The
// merge keeps the loaded vectors until every load is issued: converting
// each one as it arrives lets the compiler reuse one register pair and wait
// for every load in turn.
template <typename PT> struct Vec4;
template <> struct Vec4<float> { typedef f32x4_t type; };
template <> struct Vec4<_Float16> { typedef f16x4_t type; };
HATTN_DEV f32x4_t to_f32x4(f32x4_t v) { return v; }
HATTN_DEV f32x4_t to_f32x4(f16x4_t h) { return f32x4_t{float(h[0]), float(h[1]), float(h[2]), float(h[3])}; }

template <typename PT>
HATTN_DEV void attn_merge_body(const MergeK<PT>& mk, int H, int D, int64_t qrow, int e0, MergeLds& sm) {
  const int nsplit = mk.nsplit;
  const int tid = threadIdx.x, lane = tid & 63, sg = tid >> 6;
  const int hpg = 256 / D;            // heads in the group
  const int h0 = e0 / D;
  const int hl = (4 * lane) / D;      // this lane's head within the group
  const int64_t pos = int64_t(H) * D;
  typedef typename Vec4<PT>::type V4;
  const PT* __restrict__ po = mk.part_o + qrow * nsplit * pos + e0 + 4 * lane;
  V4 ov[kMergeRegs];
#pragma unroll
  for (int i = 0; i < kMergeRegs; ++i) {
    const int s = sg + 4 * i;
    ov[i] = s < nsplit ? __builtin_nontemporal_load(reinterpret_cast<const V4*>(po + s * pos)) : V4{0, 0, 0, 0};
  }
  if (sg == 0) {
    const float* __restrict__ ml = mk.part_ml + (qrow * nsplit * H + h0) * 4;
    const int64_t mls = int64_t(H) * 4;
    f32x4_t v[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
      v[hh] = hh < hpg && lane < nsplit ? *reinterpret_cast<const f32x4_t*>(ml + lane * mls + 4 * hh)
                                        : f32x4_t{-INFINITY, 0.f, 1.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (hh < hpg) {
        const float M = wave_max(v[hh][0]);
        float den = v[hh][0] != -INFINITY ? exp2f(v[hh][0] - M) * v[hh][1] : 0.f;
        den = wave_sum(den);
        const float inv = den > 0.f ? 1.f / den : 0.f;
        if (lane < nsplit)
          sm.w[hh][lane] = v[hh][0] == -INFINITY ? 0.f : exp2f(v[hh][0] - M) * v[hh][1] * inv * v[hh][2];
        if (lane == 0 && mk.lse) mk.lse[qrow * H + h0 + hh] = (M + __log2f(den)) * kLn2;
      }
    }
  }
  __syncthreads();
  f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMergeRegs; ++i) {
    const int s = sg + 4 * i;
    if (s < nsplit) {
      const float w = sm.w[hl][s];
      const f32x4_t v = to_f32x4(ov[i]);
#pragma unroll
      for (int c = 0; c < 4; ++c) num[c] = fmaf(w, v[c], num[c]);
    }
  }
  sm.red[sg][lane] = num;
  __syncthreads();
  if (sg == 0) {
    f32x4_t r;
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = sm.red[0][lane][c] + sm.red[1][lane][c] + sm.red[2][lane][c] + sm.red[3][lane][c];
    *reinterpret_cast<f32x4_t*>(mk.out + qrow * H * D + e0 + 4 * lane) = r;
  }
}

template <typename PT>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeK<PT> mk, int H, int D) {
  __shared__ MergeLds sm;
  attn_merge_body(mk, H, D, blockIdx.y, blockIdx.x * 256, sm);
}

// Two query sets' merges in one launch: rows [0, rows_a) of grid y are set
// a, the rest set b (same head count and size).
template <typename PT>
__global__ __launch_bounds__(256) void attn_merge_pair_kernel(MergeK<PT> a, int64_t rows_a, MergeK<PT> b, int H,
                                                              int D) {
  __shared__ MergeLds sm;
  const int64_t y = blockIdx.y;
  if (y < rows_a) attn_merge_body(a, H, D, y, blockIdx.x * 256, sm);
  else attn_merge_body(b, H, D, y - rows_a, blockIdx.x * 256, sm);
}

// Same combination for any head size or split count: one thread per output,
// each looping over all splits.
template <typename PT>
__global__ __launch_bounds__(256) void attn_merge_any_kernel(const PT* __restrict__ part_o,
                                                             const float* __restrict__ part_ml, int nsplit, int H,
                                                             int D, float* __restrict__ out, float* __restrict__ lse) {
  const int64_t qrow = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= H * D) return;
  const int h = e / D, c = e % D;
  const float* ml = part_ml + (qrow * nsplit * H + h) * 4;
  const int64_t mls = int64_t(H) * 4;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[s * mls]);
  float num = 0.f, den = 0.f;
  const PT* po = part_o + qrow * nsplit * H * D + e;
  const int64_t pos = int64_t(H) * D;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float ms = ml[s * mls];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M) * ml[s * mls + 1];
    den += w;
    num = fmaf(w * ml[s * mls + 2], float(po[s * pos]), num);
  }
  out[qrow * H * D + e] = den > 0.f ? num / den : 0.f;
  if (c == 0 && lse) lse[qrow * H + h] = (M + __log2f(den)) * kLn2;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
// bf16 MFMA shapes: 16, 32 or any multiple of 64 heads (up to 1,024; 64 per
// workgroup, head groups in grid z), d in {64, 128}.
static bool mfma_shape(const AttnArgs& a) {
  const int64_t lim = int64_t(1) << 31;  // (a ring of raw rows is never longer than L)
  const bool heads = a.h == 16 || a.h == 32 || (a.h % 64 == 0 && a.h <= 1024);
  return a.dtype == 1 && (a.d == 64 || a.d == 128) && heads && a.n * 2 * a.d < lim && a.L * 2 * a.d < lim &&
         (a.idx ? int64_t(a.k) : a.n) + a.window < lim;
}
static int head_groups(const AttnArgs& a) { return a.h > 64 ? a.h / 64 : 1; }

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
  const int tk = mfma_shape(a) ? 64 : 32;  // keys per tile
  const int64_t rows = a.bt * a.nq;
  const int64_t maxkeys = (a.idx ? int64_t(a.k) : a.n) + a.window;
  // MFMA kernel (two resident workgroups per CU): up to about 512
  // workgroups, one per resident slot, balances filling the chip against
  // the h*d*4 bytes that every extra chunk writes as a partial and the merge
  // reads back (measured: 480 beat 352 and 704 at batch 32).  Never a chunk
  // under 128 keys.
  const int64_t target_wg = mfma_shape(a) ? 512 : 1024;
  const int64_t hg = mfma_shape(a) ? head_groups(a) : 1;  // workgroups per (query, chunk)
  int64_t chunk = (rows * hg * maxkeys + target_wg - 1) / target_wg;
  chunk = std::max<int64_t>(chunk, 128);
  chunk = (chunk + tk - 1) / tk * tk;
  if (chunk >= maxkeys) chunk = (maxkeys + tk - 1) / tk * tk;
  if (mfma_shape(a) && a.idx) chunk = std::min<int64_t>(chunk, kSparseChunkMax);
  p.chunk = int(chunk);
  p.nsplit = int((maxkeys + chunk - 1) / chunk);
  if (p.nsplit > 1) {
    p.po_bytes = align256(size_t(rows) * p.nsplit * a.h * a.d * (mfma_shape(a) ? 2 : 4));  // fp16 from MFMA
    p.total = p.po_bytes + align256(size_t(rows) * p.nsplit * a.h * 4 * 4);  // 16-byte (m, l, c, 0) records
  }
  return p;
}

size_t attn_ws_bytes(const AttnArgs& a) { return plan_attn(a).total; }

static AttnK attn_k(const AttnArgs& a, const AttnPlan& pl, _Float16* po, float* pml) {
  return AttnK{(const uint16_t*)a.q, (const uint16_t*)a.ckv, a.n, a.idx, a.k, a.n_vis, (const uint16_t*)a.raw_kv,
               a.L, a.q_pos, a.window, a.scale * kLog2e, a.nq, pl.chunk, pl.nsplit, a.out, a.lse, po, pml,
               head_groups(a), a.raw_rows};
}

template <bool SPARSE>
static void launch_attn_mfma(const AttnArgs& a, const AttnPlan& pl, _Float16* po, float* pml, hipStream_t st) {
  const AttnK k = attn_k(a, pl, po, pml);
  dim3 grid(unsigned(pl.nsplit), unsigned(a.bt * a.nq), unsigned(head_groups(a)));
#define HATTN_ATTN(D, NH)                                                                     \
  do {                                                                                        \
    if (a.nq == 1) HATTN_LAUNCH((attn_mfma_kernel<D, NH, SPARSE, true>), grid, dim3(64 * NH), 0, st, k); \
    else HATTN_LAUNCH((attn_mfma_kernel<D, NH, SPARSE, false>), grid, dim3(64 * NH), 0, st, k);        \
  } while (0)
  const int nw = std::min(a.h, 64) / 16;  // waves per workgroup (16 heads each)
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
  HATTN_LAUNCH((attn_valu_kernel<T, SPARSE>), grid, dim3(256), smem, st, (const T*)a.q, (const T*)a.ckv, a.n,
                     a.idx, a.k, a.n_vis, (const T*)a.raw_kv, a.L, a.q_pos, a.window, sl2, a.nq, a.h, a.d, pl.chunk,
                     pl.nsplit, a.out, a.lse, po, pml, a.raw_rows);
}

// The merge of one query set whose partials (type PT) are at po / pml.
template <typename PT>
static void launch_merge(const AttnArgs& a, const AttnPlan& pl, PT* po, float* pml, hipStream_t st) {
  if (merge_fast(a.h, a.d, pl.nsplit))
    HATTN_LAUNCH((attn_merge_kernel<PT>), dim3(unsigned(a.h * a.d / 256), unsigned(a.bt * a.nq)), dim3(256), 0, st,
                 MergeK<PT>{po, pml, pl.nsplit, a.out, a.lse}, a.h, a.d);
  else
    HATTN_LAUNCH((attn_merge_any_kernel<PT>), dim3(unsigned((a.h * a.d + 255) / 256), unsigned(a.bt * a.nq)),
                 dim3(256), 0, st, po, pml, pl.nsplit, a.h, a.d, a.out, a.lse);
}

hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t st) {
  const AttnPlan pl = plan_attn(a);
  void* po = nullptr;  // fp16 partials from the MFMA kernels, fp32 from the vector kernel
  float* pml = nullptr;
  if (pl.nsplit > 1) {
    po = ws;
    pml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + pl.po_bytes);
  }
  const bool sparse = a.idx != nullptr;
  const bool mfma = mfma_shape(a);
  {
    LaunchScope ls(mfma ? (sparse ? "attn_sparse_mfma" : "attn_dense_mfma")
                        : (sparse ? "attn_sparse_valu" : "attn_dense_valu"),
                   st);
    _Float16* poh = static_cast<_Float16*>(po);
    float* pof = static_cast<float*>(po);
    if (mfma) {
      if (sparse) launch_attn_mfma<true>(a, pl, poh, pml, st);
      else launch_attn_mfma<false>(a, pl, poh, pml, st);
    } else if (a.dtype == 0) {
      if (sparse) launch_attn_valu<float, true>(a, pl, pof, pml, st);
      else launch_attn_valu<float, false>(a, pl, pof, pml, st);
    } else {
      if (sparse) launch_attn_valu<uint16_t, true>(a, pl, pof, pml, st);
      else launch_attn_valu<uint16_t, false>(a, pl, pof, pml, st);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  LaunchScope ls("attn_merge", st);
  if (mfma) launch_merge(a, pl, static_cast<_Float16*>(po), pml, st);
  else launch_merge(a, pl, static_cast<float*>(po), pml, st);
  return hipGetLastError();
}

// Sparse set s and dense set d in one attention launch and one merge launch
// (same bf16 MFMA head shape), each with its own workspace of
// attn_ws_bytes; any other combination runs the two launches one after the
// other.  Results equal launch_attn on each set.
hipError_t launch_attn_pair(const AttnArgs& s, void* ws_s, const AttnArgs& d, void* ws_d, hipStream_t st) {
  // (the paired launch streams K|V: one query per sequence, as in decode)
  if (!(mfma_shape(s) && mfma_shape(d) && s.idx && !d.idx && s.h == d.h && s.h <= 64 && s.d == d.d && s.nq == 1 &&
        d.nq == 1)) {
    hipError_t e = launch_attn(s, ws_s, st);
    return e != hipSuccess ? e : launch_attn(d, ws_d, st);
  }
  const AttnPlan ps = plan_attn(s), pd = plan_attn(d);
  auto parts = [](const AttnPlan& pl, void* ws, _Float16** po, float** pml) {
    *po = nullptr;
    *pml = nullptr;
    if (pl.nsplit > 1) {
      *po = reinterpret_cast<_Float16*>(ws);
      *pml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + pl.po_bytes);
    }
  };
  _Float16 *po_s, *po_d;
  float *pml_s, *pml_d;
  parts(ps, ws_s, &po_s, &pml_s);
  parts(pd, ws_d, &po_d, &pml_d);
  const AttnK ks = attn_k(s, ps, po_s, pml_s), kd = attn_k(d, pd, po_d, pml_d);
  const int64_t rows_s = s.bt * s.nq, rows_d = d.bt * d.nq;
  const dim3 grid(unsigned(int64_t(ps.nsplit) * rows_s + int64_t(pd.nsplit) * rows_d));
  {
    LaunchScope ls("attn_pair_mfma", st);
    const int nw = s.h / 16;
#define HATTN_PAIR(D, NH) HATTN_LAUNCH((attn_pair_kernel<D, NH>), grid, dim3(64 * NH), 0, st, ks, rows_s, kd)
    if (s.d == 128) {
      switch (nw) {
        case 1: HATTN_PAIR(128, 1); break;
        case 2: HATTN_PAIR(128, 2); break;
        default: HATTN_PAIR(128, 4); break;
      }
    } else {
      switch (nw) {
        case 1: HATTN_PAIR(64, 1); break;
        case 2: HATTN_PAIR(64, 2); break;
        default: HATTN_PAIR(64, 4); break;
      }
    }
#undef HATTN_PAIR
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool ms = ps.nsplit > 1, md = pd.nsplit > 1;
  const bool fast = merge_fast(s.h, s.d, ps.nsplit) && merge_fast(d.h, d.d, pd.nsplit);
  LaunchScope ls("attn_merge", st);
  const MergeK<_Float16> mks{po_s, pml_s, ps.nsplit, s.out, s.lse}, mkd{po_d, pml_d, pd.nsplit, d.out, d.lse};
  const unsigned gx = unsigned(s.h * s.d / 256);
  if (ms && md && fast) {
    HATTN_LAUNCH((attn_merge_pair_kernel<_Float16>), dim3(gx, unsigned(rows_s + rows_d)), dim3(256), 0, st, mks,
                 rows_s, mkd, s.h, s.d);
    return hipGetLastError();
  }
  for (int r = 0; r < 2; ++r) {
    const bool need = r == 0 ? ms : md;
    if (!need) continue;
    launch_merge(r == 0 ? s : d, r == 0 ? ps : pd, r == 0 ? po_s : po_d, r == 0 ? pml_s : pml_d, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hattn
