// Block-wide exact top-k selection over order-preserving 32-bit keys.
//
// Semantics (shared by every selection in the library): among the valid
// keys (key != 0), take the k largest; equal keys are taken in increasing
// position; the chosen positions are emitted in increasing position order.
// That is the same set as sorting by (score desc, position asc) and keeping
// the first k, emitted sorted by position.
//
// Layout: a row of n <= 16 * NT keys is cut into one contiguous segment per
// wave; lane l of a wave holds positions p0 + 64 * it + l (it < iters) in
// registers.  The keys are read once (from global memory or LDS) and stay in
// registers for every pass below.
//
// Method: an MSB radix search (12, 10, 10 bits) finds the threshold key T and
// how many keys equal to T are still needed.  Each pass adds the key digits
// into an LDS histogram; the threshold bin is then located in two levels (the
// 4-bin sums are added into 64 coarse bins, wave 0 scans the coarse bins and
// then the 64 fine bins of the chosen one, lanes reading adjacent words), so
// a pass costs three barriers.  Emission: per-wave counts of keys above /
// equal to T give every wave its output base; inside a wave, ballots give
// each chosen key its slot, so the result is deterministic and needs no
// sorting.
#pragma once

#include "common.h"

namespace hattn {

constexpr int kSelIT = 16;  // default keys per lane: rows of up to 16 * NT keys

template <int NT>
struct SelectShared {
  __align__(16) uint32_t hist[4096];
  uint32_t coarse[64];
  int wsum[2][NT / kWave];
  uint32_t thr;
  int need_eq;
  int above;
  int digit;
};

// This wave's contiguous segment of a row of n keys.
struct SelSeg {
  int p0, p1, iters;
};

template <int NT>
HATTN_DEV SelSeg wave_segment(int n) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const int seg = ((n + NW - 1) / NW + kWave - 1) / kWave * kWave;
  SelSeg s;
  s.p0 = wave * seg;
  s.p1 = min(n, s.p0 + seg);
  s.iters = s.p1 > s.p0 ? (s.p1 - s.p0 + kWave - 1) / kWave : 0;
  return s;
}

// Keys of the segment from fp32 scores in global memory (coalesced 4-byte
// loads, all issued before any is used); positions beyond the row read 0.
template <int IT>
HATTN_DEV void seg_keys_from_scores(const float* __restrict__ src, const SelSeg& sg, uint32_t (&kc)[IT]) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = sg.p0 + it * kWave + lane;
    v[it] = it < sg.iters && i < sg.p1 ? src[i] : 0.f;
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = sg.p0 + it * kWave + lane;
    kc[it] = it < sg.iters && i < sg.p1 ? order_key(v[it]) : 0u;
  }
}

// Keys of the segment from a u32 key array (LDS or global); 0 beyond the row.
template <int IT>
HATTN_DEV void seg_keys_from_u32(const uint32_t* src, const SelSeg& sg, uint32_t (&kc)[IT]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = sg.p0 + it * kWave + lane;
    kc[it] = it < sg.iters && i < sg.p1 ? src[i] : 0u;
  }
}

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

// Finds (thr, need_eq): select {key > thr} plus the first need_eq keys ==
// thr, over the keys every thread holds in kc[0..iters).  If at most k keys
// are valid, thr = 0 and need_eq = 0 (all valid keys); k <= 0 selects
// nothing.  Ends with a barrier; sh.thr / sh.need_eq are then readable.
template <int NT, int IT>
HATTN_DEV void radix_threshold(const uint32_t (&kc)[IT], int iters, int k, SelectShared<NT>& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  if (k <= 0) {
    if (threadIdx.x == 0) {
      sh.thr = 0xffffffffu;
      sh.need_eq = 0;
    }
    __syncthreads();
    return;
  }
  const u32x4_t z4 = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x * 4; i < 4096; i += NT * 4) *reinterpret_cast<u32x4_t*>(sh.hist + i) = z4;
  for (int i = threadIdx.x; i < 64; i += NT) sh.coarse[i] = 0u;
  __syncthreads();
  uint32_t prefix = 0, hmask = 0;
  int remaining = k;
  constexpr int kShift[3] = {20, 10, 0};
  constexpr int kWidth[3] = {12, 10, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass];
    const int nbins = 1 << kWidth[pass];
    // 1. histogram of this pass's digit over the keys that match the prefix
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      if (it < iters) {
        const uint32_t key = kc[it];
        if (key != 0u && (key & hmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nbins - 1)], 1u);
      }
    }
    __syncthreads();
    // 2. coarse bins: each holds 64 fine bins (16 quads)
    for (int q = threadIdx.x; q * 4 < nbins; q += NT) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sh.hist + 4 * q);
      const uint32_t sum = v[0] + v[1] + v[2] + v[3];
      if (sum) atomicAdd(&sh.coarse[q >> 4], sum);
    }
    __syncthreads();
    // 3. wave 0: crossing coarse bin, then crossing fine bin inside it
    if (wave == 0) {
      const int c = int(sh.coarse[lane]);
      int suf = c;  // keys in coarse bins >= lane
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int z = __shfl_down(suf, off);
        if (lane + off < kWave) suf += z;
      }
      const int total = __shfl(suf, 0);
      if (pass == 0 && total <= k) {
        if (lane == 0) sh.digit = -1;  // every valid key is chosen
      } else {
        const uint64_t cross = ballot(suf >= remaining && suf - c < remaining);
        const int cl = cross ? __ffsll((unsigned long long)cross) - 1 : 0;
        const int above_c = __shfl(suf - c, cl);
        const int f = int(sh.hist[cl * 64 + lane]);
        int fs = f;  // keys in fine bins >= lane inside coarse bin cl
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int z = __shfl_down(fs, off);
          if (lane + off < kWave) fs += z;
        }
        if (above_c + fs >= remaining && above_c + fs - f < remaining) {
          sh.digit = cl * 64 + lane;
          sh.above = above_c + fs - f;
        }
      }
      // clear for the next pass (this wave has finished reading both arrays)
      if (pass < 2) {
        for (int i = lane * 4; i < nbins; i += 4 * kWave) *reinterpret_cast<u32x4_t*>(sh.hist + i) = z4;
        sh.coarse[lane] = 0u;
      }
    }
    __syncthreads();
    const int digit = sh.digit;
    if (digit < 0) {
      __syncthreads();  // all threads have read sh.digit
      if (threadIdx.x == 0) {
        sh.thr = 0u;
        sh.need_eq = 0;
      }
      __syncthreads();
      return;
    }
    prefix |= uint32_t(digit) << shift;
    hmask |= uint32_t(nbins - 1) << shift;
    remaining -= sh.above;
  }
  if (threadIdx.x == 0) {
    sh.thr = prefix;
    sh.need_eq = remaining;
  }
  __syncthreads();
}

// Emits the chosen positions in increasing order from the same register
// keys.  emit(slot, i, key, it) is called once per chosen position i (held
// in kc[it] of the calling lane) with its output slot; returns the number
// chosen.  Does not end with a barrier.
template <int NT, int IT, typename Emit>
HATTN_DEV int emit_selected(const uint32_t (&kc)[IT], const SelSeg& sg, SelectShared<NT>& sh, Emit emit) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint32_t thr = sh.thr;
  const int need_eq = sh.need_eq;
  int gt = 0, eq = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    if (it < sg.iters) {
      gt += __popcll(ballot(kc[it] > thr));
      eq += __popcll(ballot(kc[it] == thr && kc[it] != 0u));
    }
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
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    if (it < sg.iters) {
      const uint32_t key = kc[it];
      const int i = sg.p0 + it * kWave + lane;
      const bool is_eq = key == thr && key != 0u;
      const uint64_t eqm = ballot(is_eq);
      const int eq_rank = eq_seen + mbcnt(eqm);
      const bool sel = key > thr || (is_eq && eq_rank < need_eq);
      const uint64_t sm = ballot(sel);
      if (sel) emit(out + mbcnt(sm), i, key, it);
      out += __popcll(sm);
      eq_seen += __popcll(eqm);
    }
  }
  return chosen_total;
}

}  // namespace hattn
