// Per-token cache maintenance of one compressed layer (decode): device code
// shared by the append kernel and the fused decode front kernel.
//
// [HCA] section 怎么压: an entry is the softmax(logit + position bias)-
// weighted sum of its window of raw rows; [HISA] section 02, first stage:
// one pooled representative (the mean) per block of B entries.
#pragma once

#include "common.h"

namespace hattn {

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  static HATTN_DEV void unpack(u32x4_t v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  static HATTN_DEV u32x4_t pack(const float* f) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  static HATTN_DEV void unpack(u32x4_t v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo(v[i]);
      f[2 * i + 1] = bf16hi(v[i]);
    }
  }
  static HATTN_DEV u32x4_t pack(const float* f) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};

// ---------------------------------------------------------------------------
// Per-token maintenance of one compressed layer in a decode step, one query
// (the newest token, at position p) per sequence:
//   workgroup 0: the visible count at p; if the token completes entry
//                e = (p - w + 1) / s, the softmax-weighted compression of
//                that window into ckv[e] (weights in LDS; row groups sum
//                their rows, the groups are added in a fixed order);
//   workgroup 1: if it does and block means are kept, the mean of the HISA
//                block holding e (entries past the last one count as zero).
// The same arithmetic as hattn_compress / hattn_hisa_pool / the visible
// count, in one launch instead of three.
// ---------------------------------------------------------------------------
constexpr int kAppNT = 256;  // threads per workgroup of the append kernel
constexpr int kAppUNR = 16;  // rows each thread has in flight

// Row u of a window of rows: base + u*ld, or, when the rows live in a ring
// of `wrap` rows whose row 0 sits at slot s0, base + ((s0 + u) % wrap)*ld.
HATTN_DEV int64_t win_row(int u, int s0, int wrap) { return wrap ? (s0 + u) % wrap : u; }

// Sums rows [0, n) of a [n][ld] matrix (16-byte slot cs, rows rg, rg + RG, ...)
// with per-row weights wt(u) into acc.  The first batch of rows is already in
// `first` (loaded before the weights were ready); later batches reuse it.
// Loads of a batch are all issued before any is used.  (s0, wrap): see
// win_row.
template <typename T, typename Wt>
HATTN_DEV void append_rows(const T* __restrict__ base, int64_t ld, int n, int rg, int RG, u32x4_t (&first)[kAppUNR],
                           Wt wt, float* acc, int s0 = 0, int wrap = 0) {
  constexpr int V = Vec16<T>::N;
  for (int u0 = rg; u0 < n; u0 += kAppUNR * RG) {
    if (u0 != rg) {
#pragma unroll
      for (int k = 0; k < kAppUNR; ++k) {
        const int u = u0 + k * RG;
        first[k] = u < n ? ld16_nt(base + win_row(u, s0, wrap) * ld) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < kAppUNR; ++k) {
      const int u = u0 + k * RG;
      if (u < n) {
        float f[V];
        Vec16<T>::unpack(first[k], f);
        const float pu = wt(u);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(pu, f[i], acc[i]);
      }
    }
  }
}

template <typename T>
HATTN_DEV void append_first(const T* __restrict__ base, int64_t ld, int n, int rg, u32x4_t (&first)[kAppUNR], int RG,
                            int s0 = 0, int wrap = 0) {
#pragma unroll
  for (int k = 0; k < kAppUNR; ++k) {
    const int u = rg + k * RG;
    first[k] = u < n ? ld16_nt(base + win_row(u, s0, wrap) * ld) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Per-token maintenance of one compressed layer: the launch arguments.
struct AppendK {
  const void* x;  // raw rows [bt][L][C], or a ring [bt][R][C]
  int64_t L;
  int C;
  const float* z;  // [bt][L], or a ring [bt][R]
  const float* bias;
  int w, s;
  void* y;  // entries [bt][N][C]
  int64_t N;
  int32_t* n_vis;
  const void* k_i;  // [bt][N][d_i] or NULL
  int d_i, B;
  float* reps;  // [bt][ceil(N/B)][d_i] or NULL
  int R = 0;    // 0: x and z hold all L rows; R > 0: row r at slot r % R
};

// The entry the token at p completes (-1 if none) and the visible count.
HATTN_DEV int64_t append_entry_of(const AppendK& a, int64_t p, int64_t* nv) {
  const int64_t pe = p >= a.w - 1 ? idiv(p - a.w + 1, a.s) : -1;  // entry ending at or before p
  *nv = pe + 1 > a.N ? a.N : pe + 1;
  return pe >= 0 && pe * a.s == p - a.w + 1 && pe < a.N ? pe : -1;
}

// Workgroup role "entry": the visible count and, when the token completes
// entry e, the softmax-weighted compression of its window into y[b][e].
template <typename T, int NT = kAppNT>
HATTN_DEV void append_entry_body(const AppendK& a, int64_t b, int64_t p, float* sm, float* red) {
  constexpr int V = Vec16<T>::N;
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const int C = a.C, w = a.w;
  int64_t nv;
  const int64_t e = append_entry_of(a, p, &nv);
  if (threadIdx.x == 0) a.n_vis[b] = int32_t(nv);
  if (e < 0) return;
  const int slots = C / V;
  const int RG = NT / slots;
  const int cs = threadIdx.x % slots, rg = threadIdx.x / slots;
  const int64_t t0 = e * a.s;
  // the window's rows: linear from row t0, or in the ring from slot t0 % R
  const int R = a.R;
  const int s0 = R ? int(t0 % R) : 0;
  const T* xb = R ? x + (b * R) * C + cs * V : x + (b * a.L + t0) * C + cs * V;
  const float* zb = a.z ? (R ? a.z + b * R : a.z + b * a.L + t0) : nullptr;
  // the window's first rows go out before the softmax weights are known
  u32x4_t first[kAppUNR];
  if (rg < RG) append_first(xb, C, w, rg, first, RG, s0, R);
  float* wt = sm;        // [w] logits, then softmax numerators
  float* part = sm + w;  // [RG][C] row-group partial sums
  for (int u = threadIdx.x; u < w; u += NT)
    wt[u] = (zb ? zb[win_row(u, s0, R)] : 0.f) + (a.bias ? a.bias[u] : 0.f);
  __syncthreads();
  if (threadIdx.x < kWave) {
    float mx = -INFINITY;
    for (int u = threadIdx.x; u < w; u += kWave) mx = fmaxf(mx, wt[u]);
    mx = wave_max(mx);
    float den = 0.f;
    for (int u = threadIdx.x; u < w; u += kWave) den += __expf(wt[u] - mx);
    den = wave_sum(den);
    if (threadIdx.x == 0) {
      red[0] = mx;
      red[1] = den;
    }
  }
  __syncthreads();
  const float mx = red[0], inv = 1.f / red[1];
  if (rg < RG) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    append_rows(xb, C, w, rg, RG, first, [&](int u) { return __expf(wt[u] - mx); }, acc, s0, R);
#pragma unroll
    for (int i = 0; i < V; ++i) part[rg * C + cs * V + i] = acc[i];
  }
  __syncthreads();
  T* y = static_cast<T*>(a.y);
  for (int c = threadIdx.x; c < slots; c += NT) {
    float r[V];
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] = 0.f;
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int i = 0; i < V; ++i) r[i] += part[g * C + c * V + i];
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] *= inv;
    st16(y + (b * a.N + e) * C + c * V, Vec16<T>::pack(r));
  }
}

// Workgroup role "block mean": the mean of the HISA block holding the
// completed entry (entries past the last one count as zero).
template <typename T, int NT = kAppNT>
HATTN_DEV void append_mean_body(const AppendK& a, int64_t b, int64_t p, float* sm) {
  constexpr int V = Vec16<T>::N;
  int64_t nv;
  const int64_t e = append_entry_of(a, p, &nv);
  if (e < 0 || !a.reps) return;
  const int B = a.B, d_i = a.d_i;
  const int64_t nb = idiv(a.N + B - 1, B);
  const int64_t j = idiv(e, B);
  const int64_t i0 = j * B;
  const int cnt = int(imin64(a.N, i0 + B) - i0);
  const int slots = d_i / V;
  const int RG = NT / slots;
  const int cs = threadIdx.x % slots, rg = threadIdx.x / slots;
  float* part = sm;  // [RG][d_i]
  if (rg < RG) {
    const T* kb = static_cast<const T*>(a.k_i) + (b * a.N + i0) * d_i + cs * V;
    u32x4_t first[kAppUNR];
    append_first(kb, d_i, cnt, rg, first, RG);
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    append_rows(kb, d_i, cnt, rg, RG, first, [](int) { return 1.f; }, acc);
#pragma unroll
    for (int i = 0; i < V; ++i) part[rg * d_i + cs * V + i] = acc[i];
  }
  __syncthreads();
  const float invb = 1.f / float(B);
  for (int c = threadIdx.x; c < d_i; c += NT) {
    float r = 0.f;
    for (int g = 0; g < RG; ++g) r += part[g * d_i + c];
    a.reps[(b * nb + j) * d_i + c] = r * invb;
  }
}

}  // namespace hattn
