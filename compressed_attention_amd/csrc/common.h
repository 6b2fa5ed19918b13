// Device helpers shared by the hattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define HATTN_DEV __device__ __forceinline__

namespace hattn {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// bf16 is carried as raw 16-bit patterns (uint16_t) everywhere.
HATTN_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
HATTN_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
HATTN_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (finite inputs).
HATTN_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
HATTN_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}
// Same rounding with the gfx950 packed conversion instruction (one VALU op).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
HATTN_DEV uint32_t pack_bf16x2_hw(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// 2^x without the denormal-range fixups of exp2f (results below 2^-126
// flush to zero, which only ever meets softmax weights that are negligible).
HATTN_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map fp32 -> uint32: a < b (as reals) <=> key(a) < key(b).
// -0.0 is folded onto +0.0 (equal scores).  Key 0 is never produced by a
// non-NaN value and is used as the "no candidate" sentinel.
HATTN_DEV uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
HATTN_DEV float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Reduction of v over the wave, in every lane, without LDS: DPP moves inside
// each 16-lane row (lane pairs, lane quads, row halves, rows), then the
// gfx950 lane swaps across rows.  Every step combines two values in an
// order that is the same in the two lanes, so every lane ends with the same
// bits.
template <int CTRL>
HATTN_DEV float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <typename Op>
HATTN_DEV float wave_reduce(float v, Op op) {
  v = op(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = op(v, dpp_move<0x141>(v));  // row_half_mirror: the other quad of the half row
  v = op(v, dpp_move<0x140>(v));  // row_mirror: the other half of the row
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));  // row pairs
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));  // wave halves
}
HATTN_DEV float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
HATTN_DEV float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

// a / b for 0 <= a and 0 < b: a 32-bit division when both fit (a row index
// over a per-sequence count), the 64-bit expansion only otherwise.
HATTN_DEV int64_t idiv(int64_t a, int64_t b) {
  return ((uint64_t(a) | uint64_t(b)) >> 32) == 0 ? int64_t(uint32_t(a) / uint32_t(b)) : a / b;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts (1, 2, 4,
// 8) scan each row of 16 lanes in registers, then the three lower row
// totals are read out as scalars and added.  No LDS round trips (a
// __shfl-based scan costs six ds_bpermute latencies).
HATTN_DEV uint32_t wave_prefix_incl(uint32_t x) {
  int v = int(x);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = __lane_id() >> 4;
  v += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  return uint32_t(v);
}

// max(x, 0) as one integer max: every negative float and -0.0 compares below
// +0.0 as a signed integer.  (fmaxf would first canonicalise x, an extra
// instruction per element.)
HATTN_DEV float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Lane groups g = lane / 16 of a wave.  sum4_transpose: every lane holds
// four partial sums v0..v3; group g receives the sum of value g over the
// four groups (at the same position inside the group).  Three lane-swap
// VALU ops (gfx950 v_permlane32_swap / v_permlane16_swap), no LDS traffic.
HATTN_DEV float sum4_transpose(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows 0,1: v0 pairs; rows 2,3: v2 pairs
  const float B = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows 0,1: v1 pairs; rows 2,3: v3 pairs
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(B), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
// Sum of v over the four lane groups, in every lane.
HATTN_DEV float sum_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(A), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Maximum of v over the four lane groups, in every lane (two lane swaps).
HATTN_DEV float max_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float A = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(A), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Number of lanes below this one whose bit is set in mask.
HATTN_DEV int mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

HATTN_DEV uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// 16-byte global load/store helpers.
HATTN_DEV u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
HATTN_DEV void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
HATTN_DEV u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

HATTN_DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// MFMA 16x16x32 bf16 -> fp32 (gfx950).  Lane l holds A[l%16][8*(l/16)..+7],
// B[8*(l/16)..+7][l%16]; D[4*(l/16)+i][l%16] in element i.
HATTN_DEV f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// MFMA 32x32x16 bf16 -> fp32 (on gfx950 twice the rate per FLOP of the
// 16x16x32 form).  Lane l holds A[l%32][8*(l/32)..+7], B[8*(l/32)..+7][l%32];
// element v of the result is D[8*(v/4) + 4*(l/32) + v%4][l%32].
HATTN_DEV f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// gfx950 LDS transpose read: within each group of 16 lanes, lane i receives
// element i of each of the four 16-element rows formed by concatenating the
// group's 8-byte chunks (lane j's chunk holds elements 4(j%4)..4(j%4)+3 of
// row j/4).  Pointing lane j at row (kb + j/4), column (c0 + 4(j%4)) of a
// row-major bf16 tile yields rows kb..kb+3 of column c0 + i in lane i.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
HATTN_DEV u32x2_t lds_read_tr16(const uint16_t* p) {
  const i16x4_t v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

HATTN_DEV float to_float(float x) { return x; }
HATTN_DEV float to_float(uint16_t x) { return bf16_to_f32(x); }

HATTN_DEV int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
HATTN_DEV int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

}  // namespace hattn
