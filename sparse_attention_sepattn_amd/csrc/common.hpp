// Shared device-side helpers of libsepattn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sepattn.h"

namespace sepattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kQTile = SEPATTN_QTILE;
constexpr int kKTile = SEPATTN_KTILE;
constexpr int kQF = SEPATTN_QTILE_FIELDS;

// Separator id set passed by value in kernel arguments.
struct SepSet {
  int n;
  int32_t ids[SEPATTN_MAX_SEP_IDS];
};

__device__ __forceinline__ bool is_separator(const SepSet& s, int32_t tok) {
  bool hit = false;
  for (int i = 0; i < s.n; ++i) hit |= (s.ids[i] == tok);
  return hit;
}

// bf16 <-> f32 (round to nearest even), bit-level so the rounding is explicit.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// two floats -> packed pair of bf16 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions over the lane pair (l, l ^ 32) in registers: v_permlane32_swap
// of (x, x) yields [x_lo, x_lo] and [x_hi, x_hi] (lower / upper 32 lanes).
__device__ __forceinline__ float pair_max(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work-item order that keeps contiguous runs of logical items on one XCD:
// workgroups are dealt round-robin to the 8 XCDs by launch index, so item
// `g - base` of a segment [base, base + n) is renumbered so that each XCD
// receives one contiguous range of logical indices.  Bijective on [0, n).
__device__ __forceinline__ int xcd_local_index(int g, int base, int n) {
  constexpr int kXcd = 8;
  const int c = g % kXcd;                         // this workgroup's XCD
  const int first = ((c - base) % kXcd + kXcd) % kXcd;  // first segment offset on XCD c
  int before = 0;                                 // items of the segment on XCDs < c
  for (int x = 0; x < c; ++x) {
    const int f = ((x - base) % kXcd + kXcd) % kXcd;
    before += f < n ? (n - f + kXcd - 1) / kXcd : 0;
  }
  return before + ((g - base) - first) / kXcd;
}

// Sequence b and query head h of query-major work column x in [0, B*Hq).
// Workgroups are dealt to the 8 XCDs round-robin by launch index and each XCD
// has its own L2: the columns are ordered so that the query heads of one
// (sequence, kv head) are B*Hkv columns apart, which puts them all on one
// XCD whenever B*Hkv and B*Hq are multiples of 8 (then the XCD of a column
// is its (sequence, kv head) mod 8).  The K/V tiles those heads share are then
// read from HBM once per XCD instead of once per head.
__device__ __forceinline__ void query_column(int x, int B, int Hq, int Hkv, int& b, int& h) {
  const int BG = B * Hkv, grp = Hq / Hkv;
  const int bg = x % BG, j = x / BG;
  b = bg / Hkv;
  h = (bg - b * Hkv) * grp + j;
}

}  // namespace sepattn
