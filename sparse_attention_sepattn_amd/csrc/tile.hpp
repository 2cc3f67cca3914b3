// MFMA traits and LDS tile loaders shared by the attention kernels.
//
// Formulation.  A workgroup owns 128 query rows (4 waves x 32 rows).  Scores
// are computed transposed, S^T = K Q^T, with v_mfma 32x32 (keys on the M axis,
// queries on the N axis), so each lane holds one query column and the softmax
// statistics of that query stay in the lane (plus its partner 32 lanes away).
// The output is accumulated transposed as well, O^T = V^T P^T, so P^T feeds the
// MFMA B operand straight from the score registers; only V has to be stored
// transposed in LDS.  The MFMA contraction index may be permuted freely as long
// as both operands use the same permutation: the transposed V tile is written
// in the key order the score registers hold ("kpos").
#pragma once

#include "common.hpp"

namespace sepattn {

template <typename T>
struct Traits;

template <>
struct Traits<__bf16> {
  static constexpr int EPL = 8;    // operand elements per lane per MFMA
  static constexpr int KSTEP = 16; // MFMA contraction depth
  static constexpr int VEC = 8;    // elements per 16-byte chunk
  static constexpr int KPAD = 8;   // LDS row padding of the K tile (elements)
  static constexpr int VPAD = 8;   // LDS row padding of the transposed V tile
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mfma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Traits<float> {
  static constexpr int EPL = 1;
  static constexpr int KSTEP = 2;
  static constexpr int VEC = 4;
  static constexpr int KPAD = 4;
  static constexpr int VPAD = 4;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mfma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Key held by accumulator element i (0..15) of a 32x32 MFMA result in lane
// half hh (lane / 32): rows 8*(i/4) + 4*hh + i%4.
__device__ __forceinline__ int acc_row(int i, int hh) { return ((i >> 2) << 3) + (hh << 2) + (i & 3); }

// Column of tile key r (0..63) in the transposed V tile.
template <int EPL>
__device__ __forceinline__ int kpos_of(int r) {
  const int kb2 = r >> 5, rr = r & 31;
  const int idx = ((rr >> 3) << 2) | (rr & 3);
  const int hh = (rr >> 2) & 1;
  return 32 * kb2 + (idx / EPL) * (2 * EPL) + hh * EPL + (idx % EPL);
}

template <typename T, int D>
struct TileGeom {
  static constexpr int KSTR = D + Traits<T>::KPAD;          // K tile row stride (elements)
  static constexpr int VSTR = kKTile + Traits<T>::VPAD;     // V^T tile row stride (elements)
  static constexpr int K_ELEMS = kKTile * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int CH = D / Traits<T>::VEC;             // 16-byte chunks per row
};

// Source row of tile row r: a gathered anchor (anchor list entry base + r,
// valid below `limit`) or a plain key tile (row base + r, valid below S).
struct RowSrc {
  const int32_t* anchor;  // nullptr for a plain key tile
  int base;
  int limit;
  __device__ __forceinline__ int row(int r) const {
    const int x = base + r;
    if (x >= limit) return -1;
    return anchor ? anchor[x] : x;
  }
};

// K tile -> Ks[r][c] (row-major, padded).  Invalid rows are zero.
template <typename T, int D, int NT>
__device__ __forceinline__ void load_k_tile(T* __restrict__ Ks, const T* __restrict__ Kg, RowSrc src,
                                            int tid) {
  typedef TileGeom<T, D> G;
  constexpr int VEC = Traits<T>::VEC;
  for (int u = tid; u < kKTile * G::CH; u += NT) {
    const int r = u / G::CH, cc = u % G::CH;
    const int row = src.row(r);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row >= 0) val = *(const u32x4*)(Kg + (size_t)row * D + cc * VEC);
    *(u32x4*)(Ks + r * G::KSTR + cc * VEC) = val;
  }
}

// V tile -> Vt[d][kpos(r)] (transposed, padded).  Invalid rows are zero.
template <typename T, int D, int NT>
__device__ __forceinline__ void load_vt_tile(T* __restrict__ Vt, const T* __restrict__ Vg, RowSrc src,
                                             int tid) {
  typedef TileGeom<T, D> G;
  if constexpr (Traits<T>::EPL == 8) {
    // unit = (group gi of 8 keys that are adjacent in kpos order, chunk cc)
    for (int u = tid; u < 8 * G::CH; u += NT) {
      const int gi = u & 7, cc = u >> 3;
      const int kb2 = gi >> 2, sl = (gi >> 1) & 1, hh = gi & 1;
      u32x4 rows[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = 32 * kb2 + 16 * sl + 4 * hh + jj + (jj >= 4 ? 4 : 0);
        const int row = src.row(r);
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row >= 0) val = *(const u32x4*)(Vg + (size_t)row * D + cc * 8);
        rows[jj] = val;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x0 = rows[2 * w][e >> 1], x1 = rows[2 * w + 1][e >> 1];
          out[w] = (e & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
        }
        *(u32x4*)(Vt + (cc * 8 + e) * G::VSTR + 8 * gi) = out;
      }
    }
  } else {
    for (int u = tid; u < kKTile * G::CH; u += NT) {
      const int r = u / G::CH, cc = u % G::CH;
      const int row = src.row(r);
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      if (row >= 0) val = *(const f32x4*)((const float*)Vg + (size_t)row * D + cc * 4);
      const int kp = kpos_of<1>(r);
#pragma unroll
      for (int e = 0; e < 4; ++e) ((float*)Vt)[(cc * 4 + e) * G::VSTR + kp] = val[e];
    }
  }
}

}  // namespace sepattn
