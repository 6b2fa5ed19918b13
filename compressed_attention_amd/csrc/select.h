// Block-wide exact top-k selection over order-preserving 32-bit keys in LDS.
//
// Semantics (shared by every selection in the library): among the valid
// keys (key != 0), take the k largest; equal keys are taken in increasing
// position; the chosen positions are emitted in increasing position order.
// That is the same set as sorting by (score desc, position asc) and keeping
// the first k, emitted sorted by position.
//
// Method: a 3-pass MSB radix search (12, 10, 10 bits) with LDS histograms
// finds the threshold key T and how many keys equal to T are still needed;
// then each wave walks its contiguous segment of positions, and ballots plus
// per-wave prefix counts give every chosen element its output slot, so the
// result is deterministic and needs no sorting.
#pragma once

#include "common.h"

namespace hattn {

template <int NT>
struct SelectShared {
  uint32_t hist[4096];
  int red[NT / kWave + 2];
  int wsum[2][NT / kWave];
  uint32_t thr;
  int need_eq;
  int above;
  int digit;
};

// Loads n fp32 scores (16-byte aligned row) into LDS as order-preserving
// keys.  Every thread issues all its 16-byte loads before converting any, so
// a row costs one memory round trip instead of one per element.
template <int NT>
HATTN_DEV void load_score_keys(const float* __restrict__ src, int n, uint32_t* keys) {
  constexpr int UNR = 4;
  const int n4 = n & ~3;
  for (int base = threadIdx.x * 4; base < n4; base += NT * 4 * UNR) {
    f32x4_t v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * NT * 4;
      v[u] = i < n4 ? *reinterpret_cast<const f32x4_t*>(src + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * NT * 4;
      if (i < n4) {
        u32x4_t kv;
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = order_key(v[u][e]);
        *reinterpret_cast<u32x4_t*>(keys + i) = kv;
      }
    }
  }
  for (int i = n4 + threadIdx.x; i < n; i += NT) keys[i] = order_key(src[i]);
}

// Same for (key, position) candidate lists of n entries (16-byte aligned).
template <int NT>
HATTN_DEV void load_candidates(const uint32_t* __restrict__ ik, const int32_t* __restrict__ ip, int n, uint32_t* keys,
                               int32_t* pos) {
  constexpr int UNR = 2;
  const int n4 = n & ~3;
  for (int base = threadIdx.x * 4; base < n4; base += NT * 4 * UNR) {
    u32x4_t kv[UNR], pv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * NT * 4;
      kv[u] = i < n4 ? *reinterpret_cast<const u32x4_t*>(ik + i) : u32x4_t{0, 0, 0, 0};
      pv[u] = i < n4 ? *reinterpret_cast<const u32x4_t*>(ip + i) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + u * NT * 4;
      if (i < n4) {
        *reinterpret_cast<u32x4_t*>(keys + i) = kv[u];
        *reinterpret_cast<u32x4_t*>(pos + i) = pv[u];
      }
    }
  }
  for (int i = n4 + threadIdx.x; i < n; i += NT) {
    keys[i] = ik[i];
    pos[i] = ip[i];
  }
}

// Block-wide exclusive prefix sum of v (thread order); *total gets the sum.
template <int NT>
HATTN_DEV int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      const int t = red[w];
      red[w] = acc;
      acc += t;
    }
    red[NT / kWave] = acc;
  }
  __syncthreads();
  const int excl = x - v + red[wave];
  *total = red[NT / kWave];
  __syncthreads();
  return excl;
}

// Finds (thr, need_eq): select {key > thr} plus the first need_eq keys == thr.
// keys[0..n) in LDS.  If at most k keys are valid, thr = 0 and need_eq = 0.
template <int NT>
HATTN_DEV void radix_threshold(const uint32_t* keys, int n, int k, SelectShared<NT>& sh) {
  uint32_t prefix = 0, hmask = 0;
  int remaining = k;
  const int shifts[3] = {20, 10, 0};
  const int widths[3] = {12, 10, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nbins = 1 << widths[pass];
    for (int i = threadIdx.x; i < nbins; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & hmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    // Each thread sums a contiguous run of bins; a suffix scan locates the
    // bin where the count of larger keys first reaches `remaining`.
    const int per = nbins / NT;
    const int b0 = threadIdx.x * per;
    int c = 0;
    for (int j = 0; j < per; ++j) c += int(sh.hist[b0 + j]);
    int total;
    const int excl = block_exclusive_scan<NT>(c, sh.red, &total);
    const int suffix_incl = total - excl;  // keys in bins >= b0
    if (pass == 0 && total <= k) {
      // Every valid key is chosen.
      if (threadIdx.x == 0) {
        sh.thr = 0u;
        sh.need_eq = 0;
      }
      __syncthreads();
      return;
    }
    const int suffix_excl = suffix_incl - c;  // keys in bins above this run
    if (suffix_incl >= remaining && suffix_excl < remaining) {
      int cum = suffix_excl;
      for (int j = per - 1; j >= 0; --j) {
        const int h = int(sh.hist[b0 + j]);
        if (cum + h >= remaining) {
          sh.digit = b0 + j;
          sh.above = cum;
          break;
        }
        cum += h;
      }
    }
    __syncthreads();
    prefix |= uint32_t(sh.digit) << shift;
    hmask |= uint32_t(nbins - 1) << shift;
    remaining -= sh.above;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    sh.thr = prefix;
    sh.need_eq = remaining;
  }
  __syncthreads();
}

// Emits the chosen positions in increasing order.  emit(slot, i) is called
// once per chosen element i with its output slot; returns the number chosen.
template <int NT, typename Emit>
HATTN_DEV int emit_selected(const uint32_t* keys, int n, SelectShared<NT>& sh, Emit emit) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t thr = sh.thr;
  const int need_eq = sh.need_eq;
  const int seg = ((n + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int p0 = wave * seg;
  const int p1 = min(n, p0 + seg);
  int gt = 0, eq = 0;
  for (int base = p0; base < p1; base += kWave) {
    const int i = base + lane;
    const uint32_t key = i < p1 ? keys[i] : 0u;
    gt += __popcll(ballot(key > thr));
    eq += __popcll(ballot(key == thr && key != 0u));
  }
  if (lane == 0) {
    sh.wsum[0][wave] = gt;
    sh.wsum[1][wave] = eq;
  }
  __syncthreads();
  // Per-wave bases: equal keys and chosen elements in earlier waves.
  int eqb = 0, outb = 0, my_eq_base = 0, my_out_base = 0;
  for (int w = 0; w < NW; ++w) {
    const int g = sh.wsum[0][w], e = sh.wsum[1][w];
    const int take_eq = max(0, min(e, need_eq - eqb));
    if (w == wave) {
      my_eq_base = eqb;
      my_out_base = outb;
    }
    outb += g + take_eq;
    eqb += e;
  }
  const int chosen_total = outb;
  int eq_seen = my_eq_base;
  int out = my_out_base;
  for (int base = p0; base < p1; base += kWave) {
    const int i = base + lane;
    const uint32_t key = i < p1 ? keys[i] : 0u;
    const bool is_eq = key == thr && key != 0u;
    const uint64_t eqm = ballot(is_eq);
    const int eq_rank = eq_seen + mbcnt(eqm);
    const bool sel = key > thr || (is_eq && eq_rank < need_eq);
    const uint64_t sm = ballot(sel);
    if (sel) emit(out + mbcnt(sm), i);
    out += __popcll(sm);
    eq_seen += __popcll(eqm);
  }
  __syncthreads();
  return chosen_total;
}

}  // namespace hattn
