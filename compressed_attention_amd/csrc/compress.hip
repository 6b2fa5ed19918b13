// Sequence-dimension KV compression, window visibility and HISA block pooling.
//
// Compression ([HCA] daiw.net "前代 · HCA：128 倍压缩后再做稠密注意力", section 怎么压):
// entry i of a sequence is the softmax(logit + position bias)-weighted sum of
// raw rows [i*s, i*s + w).  The kernel is a pure HBM stream: each thread owns
// 16 bytes of channels (8 bf16 or 4 fp32) of a run of consecutive entries and
// walks the window rows with fp32 accumulation; the window weights are
// recomputed per thread from the (cache-resident) logits, which costs w exps
// per w 16-byte loads.  When windows overlap (s < w) the rows shared with the
// previous entry of the run are kept in registers instead of being re-read.
#include <algorithm>
#include <type_traits>

#include "append.h"
#include "common.h"
#include "internal.h"

namespace hattn {

// Generic window: any w, s.  Thread = (sequence, run of entries, 16-byte slot).
// A second tensor compressed with the same weights as the first (the
// indexer keys of the entries, [bt][L][C2] -> [bt][N][C2]), or none (x2 ==
// nullptr, C2 == 0).  The kernels treat [x | x2] as one row of C + C2
// channels: a 16-byte slot past x's C channels belongs to x2.
template <typename T>
struct Second {
  const T* x2;
  T* y2;
  int C2;
};

// Source and destination of 16-byte slot cs of the virtual row, for
// sequence b: raw row 0 and entry 0 of that slot, and the row stride.
template <typename T>
HATTN_DEV void slot_of(const T* x, T* y, int C, const Second<T>& sec, int64_t b, int64_t L, int64_t N, int cs,
                       const T** xs, T** ys, int* ld) {
  constexpr int V = Vec16<T>::N;
  const int s1 = C / V;
  if (cs < s1) {
    *xs = x + b * L * C + cs * V;
    *ys = y + b * N * C + cs * V;
    *ld = C;
  } else {
    *xs = sec.x2 + b * L * sec.C2 + (cs - s1) * V;
    *ys = sec.y2 + b * N * sec.C2 + (cs - s1) * V;
    *ld = sec.C2;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void compress_generic_kernel(const T* __restrict__ x, const float* __restrict__ z,
                                                               const float* __restrict__ bias, T* __restrict__ y,
                                                               int64_t L, int C, int w, int s, int64_t N, int64_t e0,
                                                               int64_t runs_per_seq, int run, int64_t total,
                                                               Second<T> sec) {
  constexpr int V = Vec16<T>::N;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int slots = (C + sec.C2) / V;
  const int cs = int(t % slots);
  const int64_t rest = t / slots;
  const int64_t b = rest / runs_per_seq;
  const int64_t r = rest % runs_per_seq;
  const int64_t ebeg = e0 + r * run;
  const T* xb;
  T* yb;
  int ldc;
  slot_of(x, y, C, sec, b, L, N, cs, &xb, &yb, &ldc);
  const float* zb = z ? z + b * L : nullptr;
  for (int j = 0; j < run; ++j) {
    const int64_t e = ebeg + j;
    if (e >= N) break;
    const int64_t t0 = e * s;
    float mx = -INFINITY;
    for (int u = 0; u < w; ++u) {
      const float a = (zb ? zb[t0 + u] : 0.f) + (bias ? bias[u] : 0.f);
      mx = fmaxf(mx, a);
    }
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    float den = 0.f;
    for (int u = 0; u < w; ++u) {
      const float a = (zb ? zb[t0 + u] : 0.f) + (bias ? bias[u] : 0.f);
      const float p = __expf(a - mx);
      den += p;
      float f[V];
      Vec16<T>::unpack(ld16_nt(xb + (t0 + u) * ldc), f);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(p, f[i], acc[i]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] *= inv;
    st16(yb + e * ldc, Vec16<T>::pack(acc));
  }
}

// Overlapping windows with w = 2*s (CSA: 8 at stride 4): a thread walks a run
// of consecutive entries; the second half of entry e's window is the first
// half of entry e+1's, so each raw row is loaded once per run.
template <typename T, int S>
__global__ __launch_bounds__(256) void compress_overlap2_kernel(const T* __restrict__ x, const float* __restrict__ z,
                                                                const float* __restrict__ bias, T* __restrict__ y,
                                                                int64_t L, int C, int64_t N, int64_t e0, int64_t e1,
                                                                int64_t runs_per_seq, int run, int64_t total,
                                                                Second<T> sec) {
  constexpr int V = Vec16<T>::N;
  constexpr int W = 2 * S;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int slots = (C + sec.C2) / V;
  const int cs = int(t % slots);
  const int64_t rest = t / slots;
  const int64_t b = rest / runs_per_seq;
  const int64_t r = rest % runs_per_seq;
  const int64_t ebeg = e0 + r * run;
  const int64_t eend = imin64(e1, ebeg + run);
  if (ebeg >= eend) return;
  const T* xb;
  T* yb;
  int ldc;
  slot_of(x, y, C, sec, b, L, N, cs, &xb, &yb, &ldc);
  const float* zb = z ? z + b * L : nullptr;
  float bs[W];
#pragma unroll
  for (int u = 0; u < W; ++u) bs[u] = bias ? bias[u] : 0.f;

  // prev[] holds rows ebeg*S .. ebeg*S + S-1 (first half of the first window).
  float prev[S][V];
  float zprev[S];
#pragma unroll
  for (int u = 0; u < S; ++u) {
    Vec16<T>::unpack(ld16_nt(xb + (ebeg * S + u) * ldc), prev[u]);
    zprev[u] = zb ? zb[ebeg * S + u] : 0.f;
  }
  for (int64_t e = ebeg; e < eend; ++e) {
    float cur[S][V];
    float zcur[S];
    const int64_t t1 = e * S + S;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      Vec16<T>::unpack(ld16_nt(xb + (t1 + u) * ldc), cur[u]);
      zcur[u] = zb ? zb[t1 + u] : 0.f;
    }
    float a[W];
#pragma unroll
    for (int u = 0; u < S; ++u) {
      a[u] = zprev[u] + bs[u];
      a[S + u] = zcur[u] + bs[S + u];
    }
    float mx = a[0];
#pragma unroll
    for (int u = 1; u < W; ++u) mx = fmaxf(mx, a[u]);
    float den = 0.f;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const float p = __expf(a[u] - mx);
      den += p;
      const float* row = u < S ? prev[u] : cur[u - S];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(p, row[i], acc[i]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] *= inv;
    st16(yb + e * ldc, Vec16<T>::pack(acc));
#pragma unroll
    for (int u = 0; u < S; ++u) {
      zprev[u] = zcur[u];
#pragma unroll
      for (int i = 0; i < V; ++i) prev[u][i] = cur[u][i];
    }
  }
}

// Long windows (w >= 32, e.g. HCA's 128): one workgroup per (sequence,
// entry).  The window's softmax weights go through LDS; thread (row group
// rg, slot cs) sums rows rg, rg+RG, ... of its 16-byte slot, issuing all its
// loads before using any; the RG partial sums are then added through LDS
// in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void compress_window_kernel(const T* __restrict__ x, const float* __restrict__ z,
                                                              const float* __restrict__ bias, T* __restrict__ y,
                                                              int64_t L, int C, int w, int s, int64_t N, int64_t e0,
                                                              int64_t ne, Second<T> sec) {
  constexpr int V = Vec16<T>::N;
  extern __shared__ float wsm[];  // [w] weights, then [RG][C + C2] partial sums
  __shared__ float red[8];
  const int64_t e = e0 + blockIdx.x % ne;
  const int64_t b = blockIdx.x / ne;
  const int64_t t0 = e * s;
  const int CT = C + sec.C2;  // channels of the virtual row
  const int slots = CT / V;
  const int RG = 256 / slots;
  const int cs = threadIdx.x % slots, rg = threadIdx.x / slots;
  float mx = -INFINITY;
  for (int u = threadIdx.x; u < w; u += 256) {
    const float a = (z ? z[b * L + t0 + u] : 0.f) + (bias ? bias[u] : 0.f);
    wsm[u] = a;
    mx = fmaxf(mx, a);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float den = 0.f;
  for (int u = threadIdx.x; u < w; u += 256) {
    const float p = __expf(wsm[u] - mx);
    wsm[u] = p;
    den += p;
  }
  den = wave_sum(den);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[4 + (threadIdx.x >> 6)] = den;
  __syncthreads();
  den = red[4] + red[5] + red[6] + red[7];
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  const T* xs;
  T* ys;
  int ldc;
  slot_of(x, y, C, sec, b, L, N, cs, &xs, &ys, &ldc);
  const T* xb = xs + t0 * ldc;
  if (rg < RG) {
    int u = rg;
    for (; u + 3 * RG < w; u += 4 * RG) {
      u32x4_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = ld16_nt(xb + int64_t(u + j * RG) * ldc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f[V];
        Vec16<T>::unpack(v[j], f);
        const float p = wsm[u + j * RG];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(p, f[i], acc[i]);
      }
    }
    for (; u < w; u += RG) {
      float f[V];
      Vec16<T>::unpack(ld16_nt(xb + int64_t(u) * ldc), f);
      const float p = wsm[u];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(p, f[i], acc[i]);
    }
  }
  float* part = wsm + w;  // [RG][CT]
  if (rg < RG) {
#pragma unroll
    for (int i = 0; i < V; ++i) part[rg * CT + cs * V + i] = acc[i];
  }
  __syncthreads();
  const float inv = 1.f / den;
  for (int c = threadIdx.x; c < slots; c += 256) {
    float r[V];
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] = 0.f;
    for (int g2 = 0; g2 < RG; ++g2)
#pragma unroll
      for (int i = 0; i < V; ++i) r[i] += part[g2 * CT + c * V + i];
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] *= inv;
    const T* xo;
    T* yo;
    int ldo;
    slot_of(x, y, C, sec, b, L, N, c, &xo, &yo, &ldo);
    st16(yo + e * ldo, Vec16<T>::pack(r));
  }
}

template <typename T>
static hipError_t launch_compress_t(const void* x, int64_t bt, int64_t L, int C, const float* z, const float* bias,
                                    int w, int s, int64_t N, int64_t e0, int64_t e1, void* y, hipStream_t st,
                                    const void* x2 = nullptr, void* y2 = nullptr, int C2 = 0) {
  constexpr int V = Vec16<T>::N;
  const Second<T> sec{(const T*)x2, (T*)y2, x2 ? C2 : 0};
  const int slots = (C + sec.C2) / V;
  const int64_t ne = e1 - e0;
  if (ne <= 0 || bt <= 0) return hipSuccess;
  if (w == 2 * s && s == 4) {
    // Runs long enough to amortise the re-read first half, short enough to
    // keep many waves in flight.
    const int run = ne >= 16 * 1024 ? 16 : 1;
    const int64_t runs = (ne + run - 1) / run;
    const int64_t total = bt * runs * slots;
    LaunchScope ls("compress_overlap2", st);
    HATTN_LAUNCH((compress_overlap2_kernel<T, 4>), dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                       (const T*)x, z, bias, (T*)y, L, C, N, e0, e1, runs, run, total, sec);
    return hipGetLastError();
  }
  if (w >= 32 && slots <= 256) {
    const int RG = 256 / slots;
    const size_t smem = (size_t(w) + size_t(RG) * (C + sec.C2)) * 4;
    LaunchScope ls("compress_window", st);
    HATTN_LAUNCH((compress_window_kernel<T>), dim3(unsigned(bt * ne)), dim3(256), smem, st, (const T*)x, z, bias,
                       (T*)y, L, C, w, s, N, e0, ne, sec);
    return hipGetLastError();
  }
  const int run = 1;
  const int64_t runs = ne;
  const int64_t total = bt * runs * slots;
  LaunchScope ls("compress", st);
  HATTN_LAUNCH((compress_generic_kernel<T>), dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                     (const T*)x, z, bias, (T*)y, L, C, w, s, N, e0, runs, run, total, sec);
  return hipGetLastError();
}

hipError_t launch_compress(int dtype, const void* x, int64_t bt, int64_t L, int C, const float* z,
                           const float* bias, int w, int s, int64_t N, int64_t e0, int64_t e1, void* y,
                           hipStream_t st, const void* x2, void* y2, int C2) {
  if (dtype == 0) return launch_compress_t<float>(x, bt, L, C, z, bias, w, s, N, e0, e1, y, st, x2, y2, C2);
  return launch_compress_t<uint16_t>(x, bt, L, C, z, bias, w, s, N, e0, e1, y, st, x2, y2, C2);
}

// ---------------------------------------------------------------------------
// Compression with one logit per raw token and channel: each channel has its
// own softmax over the window.  Thread = (sequence, entry, 16-byte slot);
// one pass over the window rows with an online softmax per channel (the
// running maximum and sum are rescaled when the maximum grows).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void compress_channel_kernel(const T* __restrict__ x, const float* __restrict__ Z,
                                                               const float* __restrict__ bias, T* __restrict__ y,
                                                               int64_t L, int C, int w, int s, int64_t N, int64_t e0,
                                                               int64_t ne, int64_t total) {
  constexpr int V = Vec16<T>::N;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int slots = C / V;
  const int cs = int(t % slots);
  const int64_t rest = t / slots;
  const int64_t b = rest / ne;
  const int64_t e = e0 + rest % ne;
  const int64_t t0 = e * s;
  const T* xb = x + (b * L + t0) * C + cs * V;
  const float* zb = Z + (b * L + t0) * C + cs * V;
  float mx[V], den[V], acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    mx[i] = -INFINITY;
    den[i] = 0.f;
    acc[i] = 0.f;
  }
  for (int u = 0; u < w; ++u) {
    float f[V], a[V];
    Vec16<T>::unpack(ld16_nt(xb + int64_t(u) * C), f);
    const float bu = bias ? bias[u] : 0.f;
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const f32x4_t zz = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(zb + int64_t(u) * C + 4 * q));
#pragma unroll
      for (int i = 0; i < 4; ++i) a[4 * q + i] = zz[i] + bu;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float m_new = fmaxf(mx[i], a[i]);
      const float sc = __expf(mx[i] - m_new);  // 0 on the first row (mx = -inf)
      const float p = __expf(a[i] - m_new);
      den[i] = fmaf(den[i], sc, p);
      acc[i] = fmaf(acc[i], sc, p * f[i]);
      mx[i] = m_new;
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] /= den[i];
  st16(y + (b * N + e) * C + cs * V, Vec16<T>::pack(acc));
}

hipError_t launch_compress_channel(int dtype, const void* x, int64_t bt, int64_t L, int C, const float* Z,
                                   const float* bias, int w, int s, int64_t N, int64_t e0, int64_t e1, void* y,
                                   hipStream_t st) {
  const int V = dtype == 0 ? 4 : 8;
  const int64_t ne = e1 - e0;
  if (ne <= 0 || bt <= 0) return hipSuccess;
  const int64_t total = bt * ne * (C / V);
  LaunchScope ls("compress_channel", st);
  if (dtype == 0)
    HATTN_LAUNCH(compress_channel_kernel<float>, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                 (const float*)x, Z, bias, (float*)y, L, C, w, s, N, e0, ne, total);
  else
    HATTN_LAUNCH(compress_channel_kernel<uint16_t>, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st,
                 (const uint16_t*)x, Z, bias, (uint16_t*)y, L, C, w, s, N, e0, ne, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Visibility: entry i is visible at raw position p iff i*s + w - 1 <= p.
// ---------------------------------------------------------------------------
__global__ void visible_count_kernel(const int32_t* __restrict__ pos, int64_t count, int w, int s, int64_t n_entries,
                                     int32_t* __restrict__ n_vis) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= count) return;
  const int64_t p = pos[t];
  int64_t v = p < w - 1 ? 0 : (p - w + 1) / s + 1;
  if (v > n_entries) v = n_entries;
  n_vis[t] = int32_t(v);
}

hipError_t launch_visible_count(const int32_t* pos, int64_t count, int w, int s, int64_t n_entries, int32_t* n_vis,
                                hipStream_t st) {
  if (count <= 0) return hipSuccess;
  LaunchScope ls("visible_count", st);
  HATTN_LAUNCH(visible_count_kernel, dim3(unsigned((count + 255) / 256)), dim3(256), 0, st, pos, count, w, s,
                     n_entries, n_vis);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// HISA pooling ([HISA] my.qihongyi.cn/?p=787, section 第一阶段): block mean
// with a zero-padded short tail.  One workgroup per (sequence, block):
// thread (row group rg, 16-byte slot cs) sums rows rg, rg+RG, ... in fp32,
// then the RG partial sums are added through LDS in a fixed order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ k_i, int64_t n, int d, int B, int64_t nb,
                                                   int64_t j0, int64_t nj, float* __restrict__ reps) {
  constexpr int V = Vec16<T>::N;
  extern __shared__ float part[];  // [RG][d]
  const int64_t b = blockIdx.x / nj;
  const int64_t j = j0 + blockIdx.x % nj;
  const int slots = d / V;
  const int RG = 256 / slots;
  const int cs = threadIdx.x % slots, rg = threadIdx.x / slots;
  const int64_t i0 = j * B;
  const int cnt = int(imin64(n, i0 + B) - i0);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  if (rg < RG) {
    const T* base = k_i + (b * n + i0) * d + cs * V;
    int u = rg;
    for (; u + 3 * RG < cnt; u += 4 * RG) {
      u32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = ld16_nt(base + int64_t(u + q * RG) * d);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float f[V];
        Vec16<T>::unpack(v[q], f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += f[i];
      }
    }
    for (; u < cnt; u += RG) {
      float f[V];
      Vec16<T>::unpack(ld16_nt(base + int64_t(u) * d), f);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += f[i];
    }
#pragma unroll
    for (int i = 0; i < V; ++i) part[rg * d + cs * V + i] = acc[i];
  }
  __syncthreads();
  const float inv = 1.f / float(B);
  for (int c = threadIdx.x; c < d; c += 256) {
    float r = 0.f;
    for (int g2 = 0; g2 < RG; ++g2) r += part[g2 * d + c];
    reps[(b * nb + j) * d + c] = r * inv;
  }
}

hipError_t launch_pool(int dtype, const void* k_i, int64_t bt, int64_t n, int d_i, int B, int64_t j0, int64_t j1,
                       float* reps, hipStream_t st) {
  const int64_t nb = (n + B - 1) / B;
  const int64_t nj = j1 - j0;
  if (nj <= 0 || bt <= 0) return hipSuccess;
  LaunchScope ls("hisa_pool", st);
  const int V = dtype == 0 ? 4 : 8;
  const int RG = 256 / (d_i / V);
  const size_t smem = size_t(RG) * d_i * 4;
  if (dtype == 0) {
    HATTN_LAUNCH(pool_kernel<float>, dim3(unsigned(bt * nj)), dim3(256), smem, st, (const float*)k_i, n, d_i, B,
                       nb, j0, nj, reps);
  } else {
    HATTN_LAUNCH(pool_kernel<uint16_t>, dim3(unsigned(bt * nj)), dim3(256), smem, st, (const uint16_t*)k_i, n,
                       d_i, B, nb, j0, nj, reps);
  }
  return hipGetLastError();
}


// One launch for one or two layers, grid (roles, bt): layer a's entry, then
// (when a keeps block means) its block mean, then (when b_on) layer b's
// entry.  Both layers serve the same sequences and token positions.
template <typename T>
__global__ __launch_bounds__(kAppNT) void append_kernel(AppendK la, AppendK lb, int b_on,
                                                        const int32_t* __restrict__ q_pos) {
  extern __shared__ float sm[];
  __shared__ float red[2];
  const int64_t b = blockIdx.y;
  const int64_t p = q_pos[b];
  int role = blockIdx.x;
  if (!la.reps && role >= 1) role += 1;
  if (role == 0) append_entry_body<T>(la, b, p, sm, red);
  else if (role == 1) append_mean_body<T>(la, b, p, sm);
  else if (b_on) append_entry_body<T>(lb, b, p, sm, red);
}

static size_t append_lds_one(const AppendK& a, int V) {
  const size_t sm_c = size_t(a.w + (kAppNT / (a.C / V)) * a.C) * 4;
  const size_t sm_r = a.reps ? size_t(kAppNT / (a.d_i / V)) * a.d_i * 4 : 0;
  return std::max(sm_c, sm_r);
}

static hipError_t launch_append_k(int dtype, const AppendK& la, const AppendK* lb, int64_t bt,
                                  const int32_t* q_pos, hipStream_t st) {
  const int V = dtype == 0 ? 4 : 8;
  size_t smem = append_lds_one(la, V);
  if (lb) smem = std::max(smem, append_lds_one(*lb, V));
  const unsigned roles = 1u + (la.reps ? 1u : 0u) + (lb ? 1u : 0u);
  const AppendK none{};
  LaunchScope ls("decode_append", st);
  if (dtype == 0)
    HATTN_LAUNCH((append_kernel<float>), dim3(roles, unsigned(bt)), dim3(kAppNT), smem, st, la, lb ? *lb : none,
                 lb ? 1 : 0, q_pos);
  else
    HATTN_LAUNCH((append_kernel<uint16_t>), dim3(roles, unsigned(bt)), dim3(kAppNT), smem, st, la, lb ? *lb : none,
                 lb ? 1 : 0, q_pos);
  return hipGetLastError();
}

size_t append_lds_bytes(int dtype, int C, int w, int d_i, bool with_reps) {
  AppendK a{};
  a.C = C;
  a.w = w;
  a.d_i = d_i;
  a.reps = with_reps ? reinterpret_cast<float*>(16) : nullptr;
  return append_lds_one(a, dtype == 0 ? 4 : 8);
}

hipError_t launch_append(int dtype, const void* x, int64_t bt, int64_t L, int C, const float* z, const float* bias,
                         int w, int s, const int32_t* q_pos, void* y, int64_t N, int32_t* n_vis, const void* k_i,
                         int d_i, int B, float* reps, hipStream_t st, int raw_rows) {
  const AppendK la{x, L, C, z, bias, w, s, y, N, n_vis, k_i, d_i, B, reps, raw_rows};
  return launch_append_k(dtype, la, nullptr, bt, q_pos, st);
}

hipError_t launch_append_pair(int dtype, int64_t bt, const int32_t* q_pos, const void* x1, const float* z1,
                              const float* bias1, int w1, int s1, void* y1, int64_t N1, int32_t* n_vis1,
                              const void* k_i, int d_i, int B, float* reps, const void* x2, const float* z2,
                              const float* bias2, int w2, int s2, void* y2, int64_t N2, int32_t* n_vis2, int64_t L,
                              int C, hipStream_t st, int raw_rows) {
  const AppendK la{x1, L, C, z1, bias1, w1, s1, y1, N1, n_vis1, k_i, d_i, B, reps, raw_rows};
  const AppendK lb{x2, L, C, z2, bias2, w2, s2, y2, N2, n_vis2, nullptr, 0, 0, nullptr, raw_rows};
  return launch_append_k(dtype, la, &lb, bt, q_pos, st);
}

}  // namespace hattn
