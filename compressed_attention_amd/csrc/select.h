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
// into an LDS histogram (pass 0 in words [0, 4096), pass 1 in [4096, 5120),
// pass 2 in [0, 1024), which pass 1 clears, so no pass waits for a clear).
// The threshold bin is then found without a further barrier: each thread
// owns a run of adjacent bins and publishes its wave's count; every wave
// reads the wave counts lane-parallel, picks the wave whose runs hold the
// crossing, re-reads that wave's runs, and locates the bin with DPP prefix
// sums and ballots.  Every thread thus knows the digit, and a pass costs two
// barriers.  Emission: per-wave counts of keys above / equal to T give every
// wave its output base (lane-parallel prefix sums over the waves); inside a
// wave, ballots give each chosen key its slot, so the result is
// deterministic and needs no sorting.
#pragma once

#include "common.h"

namespace hattn {

constexpr int kSelIT = 16;  // default keys per lane: rows of up to 16 * NT keys

template <int NT>
struct SelectShared {
  __align__(16) uint32_t hist[4096 + 1024];
  __align__(16) uint32_t wtot[NT / kWave];
  int wsum[2][NT / kWave];
};

// The selection's threshold: every key > thr, plus the first need_eq keys
// equal to thr (in position order).
struct SelThr {
  uint32_t thr;
  int need_eq;
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

// Raw fp32 scores of the segment (loads only; positions beyond the row read
// 0).  seg_keys_masked turns them into keys once they have arrived.
template <int IT>
HATTN_DEV void seg_load_scores(const float* __restrict__ src, const SelSeg& sg, float (&v)[IT]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = sg.p0 + it * kWave + lane;
    v[it] = it < sg.iters && i < sg.p1 ? src[i] : 0.f;
  }
}

// Keys of positions below nvalid; 0 (no candidate) elsewhere.
template <int IT>
HATTN_DEV void seg_keys_masked(const float (&v)[IT], const SelSeg& sg, int nvalid, uint32_t (&kc)[IT]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = sg.p0 + it * kWave + lane;
    kc[it] = it < sg.iters && i < sg.p1 && i < nvalid ? order_key(v[it]) : 0u;
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

// Zeroes the histogram.  A caller may do this early (e.g. while its key
// loads are in flight) and then pass CLEARED = true to radix_threshold; a
// barrier must separate the two.
template <int NT>
HATTN_DEV void select_clear(SelectShared<NT>& sh) {
  const u32x4_t z4 = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x * 4; i < 4096 + 1024; i += NT * 4) *reinterpret_cast<u32x4_t*>(sh.hist + i) = z4;
}

// This wave's index as a scalar (uniform) value.
HATTN_DEV int wave_index() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave); }

// Sum over the wave of x, in every lane.
HATTN_DEV uint32_t wave_total(uint32_t x) { return uint32_t(__builtin_amdgcn_readlane(int(wave_prefix_incl(x)), 63)); }

// Lowest set lane of a nonzero ballot, as a scalar.
HATTN_DEV int first_lane(uint64_t m) { return __builtin_amdgcn_readfirstlane(int(__builtin_ctzll(m))); }

// Finds the threshold over the keys every thread holds in kc[0..iters): the
// k largest valid keys are {key > thr} plus the first need_eq keys == thr.
// If at most k keys are valid, thr = 0 and need_eq = 0 (all valid keys);
// k <= 0 selects nothing.  Every thread returns the same value.  The
// histogram must be zero on entry (CLEARED: the caller cleared it and
// passed a barrier since; otherwise this clears it); it is left dirty.
// sh.wtot is reused by the next call only after that call's first barrier.
template <int NT, int IT, bool CLEARED = false>
HATTN_DEV SelThr radix_threshold(const uint32_t (&kc)[IT], int iters, int k, SelectShared<NT>& sh) {
  constexpr int NW = NT / kWave;
  static_assert(NT >= 256 && NT <= 1024 && 4096 % NT == 0, "runs of whole bins per thread");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  if (k <= 0) return SelThr{0xffffffffu, 0};
  if (!CLEARED) {
    __syncthreads();  // a previous selection may still be reading the histogram
    select_clear(sh);
    __syncthreads();
  }
  uint32_t prefix = 0, hmask = 0;
  uint32_t remaining = uint32_t(k);
  constexpr int kShift[3] = {20, 10, 0};
  constexpr int kWidth[3] = {12, 10, 10};
  constexpr int kBase[3] = {0, 4096, 0};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass];
    const int nbins = 1 << kWidth[pass];
    const int bpt = nbins / NT > 0 ? nbins / NT : 1;  // bins per owning thread
    uint32_t* hist = sh.hist + kBase[pass];
    // 1. histogram of this pass's digit over the keys that match the prefix
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      if (it < iters) {
        const uint32_t key = kc[it];
        if (key != 0u && (key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1u);
      }
    }
    __syncthreads();
    // 2. thread t owns bins [bpt*t, bpt*(t+1)) of this pass; wave totals.
    //    Pass 1 also clears pass 0's words, which pass 2 reuses.
    {
      uint32_t own = 0;
      if (bpt * int(threadIdx.x) < nbins)
        for (int j = 0; j < bpt; ++j) own += hist[bpt * threadIdx.x + j];
      if (pass == 1) {
        const u32x4_t z4 = {0u, 0u, 0u, 0u};
        for (int i = threadIdx.x * 4; i < 4096; i += NT * 4) *reinterpret_cast<u32x4_t*>(sh.hist + i) = z4;
      }
      const uint32_t incl = wave_prefix_incl(own);
      if (lane == kWave - 1) sh.wtot[wave] = incl;
    }
    __syncthreads();
    // 3. every wave: the crossing wave, then the crossing thread and bin
    const uint32_t wt = lane < NW ? sh.wtot[lane] : 0u;
    const uint32_t wincl = wave_prefix_incl(wt);
    const uint32_t total = uint32_t(__builtin_amdgcn_readlane(int(wincl), NW - 1));
    if (pass == 0 && total <= uint32_t(k)) return SelThr{0u, 0};  // every valid key is chosen
    const uint32_t above_w = total - wincl;  // keys in waves above lane w's wave
    const int wc = first_lane(ballot(lane < NW && above_w < remaining && above_w + wt >= remaining));
    const uint32_t above_wave = uint32_t(__builtin_amdgcn_readlane(int(above_w), wc));
    const int t = wc * kWave + lane;  // a thread of the crossing wave
    uint32_t c[4096 / 256];
    uint32_t own = 0;
#pragma unroll
    for (int j = 0; j < 4096 / 256; ++j) {
      c[j] = j < bpt && bpt * t < nbins ? hist[bpt * t + j] : 0u;
      own += c[j];
    }
    const uint32_t incl = wave_prefix_incl(own);
    const uint32_t tot_w = uint32_t(__builtin_amdgcn_readlane(int(incl), kWave - 1));
    const uint32_t above_run = above_wave + (tot_w - incl);
    const int lc = first_lane(ballot(above_run < remaining && above_run + own >= remaining));
    int digit = 0;
    uint32_t above = 0;
    {
      uint32_t cum = above_run;
#pragma unroll
      for (int j = 4096 / 256 - 1; j >= 0; --j) {
        if (j < bpt && cum < remaining && cum + c[j] >= remaining) {
          digit = bpt * t + j;
          above = cum;
        }
        cum += j < bpt ? c[j] : 0u;
      }
    }
    digit = __builtin_amdgcn_readlane(digit, lc);
    above = uint32_t(__builtin_amdgcn_readlane(int(above), lc));
    prefix |= uint32_t(digit) << shift;
    hmask |= uint32_t(nbins - 1) << shift;
    remaining -= above;
  }
  return SelThr{prefix, int(remaining)};
}

// One-wave variant for short rows (up to 64 * IT keys; lane l holds
// positions 64 * it + l): the same result as radix_threshold, found with
// four 8-bit passes over a 256-bin LDS histogram.  With one wave per
// workgroup a pass needs no cross-wave totals: lane l owns bins 4l..4l+3,
// and one DPP scan over the lanes locates the crossing bin.  The single
// wave's chain is longer than a workgroup's, so this pays off only when
// many rows keep the chip busy.  hist is this wave's 256 words of LDS; the
// workgroup must be this one wave (its barriers order the histogram's
// clears, adds and reads).
template <int IT>
HATTN_DEV SelThr wave_radix_threshold(const uint32_t (&kc)[IT], int k, uint32_t* hist) {
  const int lane = threadIdx.x & (kWave - 1);
  if (k <= 0) return SelThr{0xffffffffu, 0};
  uint32_t nval = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) nval += uint32_t(__popcll(ballot(kc[it] != 0u)));
  if (nval <= uint32_t(k)) return SelThr{0u, 0};  // every valid key is chosen
  uint32_t prefix = 0, hmask = 0, remaining = uint32_t(k);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    *reinterpret_cast<u32x4_t*>(hist + 4 * lane) = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t key = kc[it];
      if (key != 0u && (key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(hist + 4 * lane);
    const uint32_t own = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_prefix_incl(own);
    const uint32_t total = uint32_t(__builtin_amdgcn_readlane(int(incl), kWave - 1));
    const uint32_t above_run = total - incl;  // keys in the bins of higher lanes
    const int lc = first_lane(ballot(above_run < remaining && above_run + own >= remaining));
    int digit = 0;
    uint32_t above = 0;
    {
      uint32_t cum = above_run;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (cum < remaining && cum + c[j] >= remaining) {
          digit = 4 * lane + j;
          above = cum;
        }
        cum += c[j];
      }
    }
    digit = __builtin_amdgcn_readlane(digit, lc);
    above = uint32_t(__builtin_amdgcn_readlane(int(above), lc));
    prefix |= uint32_t(digit) << shift;
    hmask |= 255u << shift;
    remaining -= above;
    __syncthreads();  // every lane has read its bins before the next clear
  }
  return SelThr{prefix, int(remaining)};
}

// One-wave emission (positions 64 * it + lane, increasing): emit(slot, i,
// key) once per chosen position; returns the number chosen.
template <int IT, typename Emit>
HATTN_DEV int wave_emit_selected(const uint32_t (&kc)[IT], SelThr st, Emit emit) {
  const int lane = threadIdx.x & (kWave - 1);
  int out = 0, eq_seen = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t key = kc[it];
    const bool is_eq = key == st.thr && key != 0u;
    const uint64_t eqm = ballot(is_eq);
    const bool sel = key > st.thr || (is_eq && eq_seen + int(mbcnt(eqm)) < st.need_eq);
    const uint64_t sm = ballot(sel);
    if (sel) emit(out + int(mbcnt(sm)), kWave * it + lane, key);
    out += int(__popcll(sm));
    eq_seen += int(__popcll(eqm));
  }
  return out;
}

// Emits the chosen positions in increasing order from the same register
// keys.  emit(slot, i, key, it) is called once per chosen position i (held
// in kc[it] of the calling lane) with its output slot; returns the number
// chosen.  Does not end with a barrier.
template <int NT, int IT, typename Emit>
HATTN_DEV int emit_selected(const uint32_t (&kc)[IT], const SelSeg& sg, SelectShared<NT>& sh, SelThr st,
                            Emit emit) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const uint32_t thr = st.thr;
  const int need_eq = st.need_eq;
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
  // Per-wave bases, lane w standing for wave w: equal keys in earlier waves
  // (eqb), the equal keys wave w takes, and chosen keys in earlier waves.
  const int g = lane < NW ? sh.wsum[0][lane] : 0;
  const int e = lane < NW ? sh.wsum[1][lane] : 0;
  const int e_incl = int(wave_prefix_incl(uint32_t(e)));
  const int eqb = e_incl - e;
  const int take_eq = max(0, min(e, need_eq - eqb));
  const int out_incl = int(wave_prefix_incl(uint32_t(g + take_eq)));
  const int chosen_total = __builtin_amdgcn_readlane(out_incl, NW - 1);
  int eq_seen = wave > 0 ? __builtin_amdgcn_readlane(e_incl, wave - 1) : 0;
  int out = wave > 0 ? __builtin_amdgcn_readlane(out_incl, wave - 1) : 0;
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
