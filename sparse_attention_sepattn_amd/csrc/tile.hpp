// MFMA traits, LDS tile loaders and operand readers shared by the attention
// kernels.
//
// Formulation.  A query-major workgroup owns 128 query rows (4 waves x 32
// rows).  Scores are computed transposed, S^T = K Q^T, with v_mfma 32x32
// (keys on the M axis, queries on the N axis), so each lane holds one query
// column and the softmax statistics of that query stay in the lane (plus its
// partner 32 lanes away).  The output is accumulated transposed as well,
// O^T = V^T P^T, so P^T feeds the MFMA B operand straight from the score
// registers.  The A operand V^T is read from the row-major V tile in LDS with
// the gfx950 transpose read (ds_read_b64_tr_b16): within each 16-lane group,
// output lane 4a+c receives element c of the 8-byte chunks addressed by lanes
// a, 4+a, 8+a, 12+a.  Addressing row r0+4h+(s>>2), column c0+16*(g&1)+4*(s&3)
// from source lane s of group g therefore gives output lane l the column
// c0+(l&31) of rows r0+4h+k, k = 0..3: the A operand of X^T for a row-major X.
// The MFMA contraction index may be permuted freely as long as both operands
// use the same permutation; the rows read here follow the order the score
// registers hold keys in (acc_row below).  fp32 tiles need no transpose read:
// one element per lane is a plain LDS read.
//
// Every tile is stored row-major in LDS (16-byte chunks XOR-swizzled by row,
// see TileGeom) and loaded through registers so the next tile's global loads
// are in flight while the current tile computes.
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
  static constexpr int PAD = 8;    // LDS row padding (elements)
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
  static constexpr int PAD = 4;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mfma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Row held by accumulator element i (0..15) of a 32x32 MFMA result in lane
// half hh (lane / 32): 8*(i/4) + 4*hh + i%4.
__device__ __forceinline__ int acc_row(int i, int hh) { return ((i >> 2) << 3) + (hh << 2) + (i & 3); }

// 16-byte chunks of a row are stored XOR-swizzled by the row index (no
// padding).  The row-major read of 16 consecutive rows at one chunk (one
// 256-byte LDS phase) touches distinct banks:
//   >= 16 chunks per row: c ^ f(r), f bijective on r % 16;
//   8 chunks per row (two rows per 256-byte bank line): c ^ g(r) with g
//   bijective on (r >> 1) % 8.
// The transpose read (32 lanes x 8 bytes = 4 rows x 64 bytes per phase) meets
// 2-way conflicts on two of its rows.  A swizzle free of them for both reads
// exists (XOR on the higher chunk bits), but it no longer commutes with the
// constant chunk offsets of the read sites, so every site needs its own
// address register; measured, that cost more than the conflicts.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3); }
__device__ __forceinline__ int swz8(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 1) | ((x >> 1) & 1) | (x & 4);
}

template <typename T, int D>
struct TileGeom {
  static constexpr int VEC = Traits<T>::VEC;
  static constexpr int CH = D / VEC;       // 16-byte chunks per row
  static constexpr int ELEMS = kKTile * D; // one 64-row tile
  // element offset of (row, col) in a swizzled tile
  static __device__ __forceinline__ int at(int row, int col) {
    const int f = CH >= 16 ? swz16(row) : swz8(row);
    return row * D + (((col / VEC) ^ f) & (CH - 1)) * VEC + (col % VEC);
  }
};

// Source row of tile row r: a gathered anchor (anchor list entry base + r,
// valid below `limit`) or a plain key/query tile (row base + r, valid below
// `limit`).
struct RowSrc {
  const int32_t* anchor;  // nullptr for a plain tile
  int base;
  int limit;
  __device__ __forceinline__ int row(int r) const {
    const int x = base + r;
    if (x >= limit) return -1;
    return anchor ? anchor[x] : x;
  }
};

// The rows of one 64-row tile of a [rows, D] tensor that thread tid fetches:
// NU 16-byte chunks, unit u in row tid/CH + (NT/CH)*u, chunk tid%CH, so
// consecutive lanes take consecutive chunks of a row.
template <typename T, int D, int NT>
struct TileRows {
  typedef TileGeom<T, D> G;
  static constexpr int NU = kKTile * G::CH / NT;
  static_assert(NU * NT == kKTile * G::CH, "tile must split evenly over the workgroup");

  static __device__ __forceinline__ int row_of(int tid, int u) { return tid / G::CH + (NT / G::CH) * u; }

  // source rows of this thread's units (anchor tiles read the anchor list)
  __device__ __forceinline__ static void rows(int* out, RowSrc src, int tid) {
#pragma unroll
    for (int u = 0; u < NU; ++u) out[u] = src.row(row_of(tid, u));
  }
};

// A 64-row tile loaded straight from global memory into LDS
// (buffer_load_dwordx4 ... lds: lane l of a wave writes 16 bytes at
// M0 + 16*l), so no registers hold the tile in flight.  A wave's instruction
// u fills 1 KB of LDS, the rows TileRows::row_of gives its lanes; each lane
// fetches the global chunk that the swizzle puts at its LDS position.  Rows
// with srow < 0 use an offset past the buffer's size, which the hardware
// range check turns into zeros.  Completion is counted by vmcnt: the caller
// waits (s_waitcnt vmcnt) before the barrier that publishes the tile.
template <typename T, int D, int NT>
struct TileDMA {
  typedef TileGeom<T, D> G;
  typedef TileRows<T, D, NT> R;
  static constexpr int NU = R::NU;
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t src, unsigned src_bytes, const int* srow,
                                               T* tile, int tid) {
    // the wave index is uniform: read it into a scalar so the LDS destination
    // (M0) of every load is a scalar value, not a per-lane one read back
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int pos = tid % G::CH;  // 16-byte position of this lane in its LDS row
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = R::row_of(tid, u);
      const int f = G::CH >= 16 ? swz16(r) : swz8(r);
      const int c = (pos ^ f) & (G::CH - 1);
      const unsigned off = srow[u] >= 0 ? (unsigned)(srow[u] * D + c * Traits<T>::VEC) * (unsigned)sizeof(T)
                                        : src_bytes;
      T* dst = tile + (w * 1024 + u * NT * 16) / (int)sizeof(T);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
    }
  }
  // A tile of 64 consecutive rows: `src` starts at the tile's first row and
  // ends where the tensor ends, so rows past the end read zeros; the offsets
  // are the per-thread constants of tile_unit_offset, and only the resource
  // (scalar) changes from tile to tile.
  static __device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t src, const unsigned* uoff, T* tile,
                                                    int tid) {
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      T* dst = tile + (w * 1024 + u * NT * 16) / (int)sizeof(T);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, uoff[u], 0, 0,
                                               0);
    }
  }
};

// Byte offset, within a tile of consecutive rows, of the 16-byte chunk that
// thread tid's unit u loads (TileDMA's layout): a per-thread constant.
template <typename T, int D, int NT>
__device__ __forceinline__ unsigned tile_unit_offset(int tid, int u) {
  typedef TileGeom<T, D> G;
  const int r = TileRows<T, D, NT>::row_of(tid, u);
  const int f = G::CH >= 16 ? swz16(r) : swz8(r);
  const int c = ((tid % G::CH) ^ f) & (G::CH - 1);
  return (unsigned)(r * D + c * Traits<T>::VEC) * (unsigned)sizeof(T);
}

// A 128-row block of bf16 output held transposed in MFMA accumulators (wave
// w: rows 32w .. 32w+31, lane = row within those 32; acc[db] element i =
// column 32db + acc_row(i, lane / 32), times `scale`) goes out as whole rows:
// the waves write their rows into two 64-row tiles (A: rows 0..63, B: rows
// 64..127, swizzled like every tile), then every thread stores the 16-byte
// chunks that a tile load (TileDMA) would have brought into its LDS slots, so
// consecutive lanes store consecutive chunks of a row.  row_dst(r) gives the
// destination of block row r (nullptr: not stored).  The caller's barrier
// must precede the call (both tiles free); the tiles are overwritten.
template <int D, int NT, typename RowDst>
__device__ __forceinline__ void store_rows_via_lds(__bf16* tileA, __bf16* tileB, const f32x16* acc, float scale,
                                                   RowDst row_dst, const unsigned* uoff, int tid) {
  typedef TileGeom<__bf16, D> G;
  typedef TileRows<__bf16, D, NT> R;
  constexpr int NDB = D / 32;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave, hh = lane >> 5;
  __bf16* own = w < 2 ? tileA : tileB;
  const int row = 32 * (w & 1) + (lane & 31);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * db + 8 * r4 + 4 * hh;
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[db][4 * r4 + 0] * scale, acc[db][4 * r4 + 1] * scale);
      pk[1] = pack_bf16x2(acc[db][4 * r4 + 2] * scale, acc[db][4 * r4 + 3] * scale);
      *(u32x2*)(own + G::at(row, d0)) = pk;
    }
  }
  __syncthreads();
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const __bf16* src = half == 0 ? tileA : tileB;
#pragma unroll
    for (int u = 0; u < R::NU; ++u) {
      const int r = R::row_of(tid, u);
      __bf16* d = row_dst(kKTile * half + r);
      const u32x4 v = *(const u32x4*)(src + (w * 1024 + u * NT * 16) / 2 + lane * 8);
      if (d) *(u32x4*)(d + uoff[u] / 2 - (size_t)r * D) = v;
    }
  }
}

// Buffer resource over `bytes` bytes from `base` (raw, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}
// Waits for this wave's outstanding vector-memory loads, LDS-bound ones included.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0), other counters untouched

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
}

// A operand of X^T for MFMA step `sl` over the 32-row block `k2` of a
// row-major swizzled LDS tile X: lane (m = lane&31, h = lane>>5) gets column
// c0 + m of the rows the score accumulators hold for that step.
// bf16 (16 rows per step): rows 32*k2 + 16*sl + 8*(j/4) + 4h + j%4, j = 0..7.
// fp32 (2 rows per step):  row 32*k2 + acc_row(sl, h).
template <typename T, int D>
__device__ __forceinline__ typename Traits<T>::frag read_xt(const T* X, int k2, int sl, int c0, int lane) {
  typedef TileGeom<T, D> G;
  if constexpr (Traits<T>::EPL == 8) {
    const int grp = lane >> 4, s = lane & 15;
    const int h = grp >> 1;
    const int col = c0 + 16 * (grp & 1) + 4 * (s & 3);
    const int row = 32 * k2 + 16 * sl + 4 * h + (s >> 2);
    const s16x4 lo = lds_read_tr16(X + G::at(row, col));
    const s16x4 hi = lds_read_tr16(X + G::at(row + 8, col));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  } else {
    return X[G::at(32 * k2 + acc_row(sl, lane >> 5), c0 + (lane & 31))];
  }
}

// A operand of X (row-major) for the contraction over columns: lane (row
// m = lane&31 of the 32-row block `rb`, h) gets columns c*KSTEP + EPL*h ..
template <typename T, int D>
__device__ __forceinline__ typename Traits<T>::frag read_x(const T* X, int rb, int c, int lane) {
  typedef TileGeom<T, D> G;
  constexpr int EPL = Traits<T>::EPL;
  const int row = 32 * rb + (lane & 31);
  const int col = c * Traits<T>::KSTEP + EPL * (lane >> 5);
  return *(const typename Traits<T>::frag*)(X + G::at(row, col));
}

// Bits [lo, hi] of a 64-bit word (lo, hi clamped to [0, 63]; empty if hi < lo).
__device__ __forceinline__ uint64_t bit_range(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 63 ? 63 : hi;
  if (hi < lo) return 0ull;
  return (~0ull >> (63 - hi)) & (~0ull << lo);
}

// Masking of one accumulator element by bit `pos` of a lane's visibility
// word: v_bfe_i32 sign-extends the 1-bit field to an all-ones / all-zero
// mask; a bitfield insert then keeps the value or puts -inf in its place.
__device__ __forceinline__ uint32_t bit_mask(uint32_t w, int pos) {
  return (uint32_t)__builtin_amdgcn_sbfe((int)w, pos, 1);
}
__device__ __forceinline__ float keep_or_neg_inf(float x, uint32_t m) {
  return __uint_as_float((__float_as_uint(x) & m) | (~m & 0xFF800000u));
}
// Bit position, within a lane's 32-row (or 32-key) block, of accumulator
// element i once the block's word is shifted right by 4 * (lane / 32).
__device__ __forceinline__ constexpr int acc_bit(int i) { return ((i >> 2) << 3) + (i & 3); }

// Keys c0 .. c0+63 of the band that query row iq sees (bit r = key c0 + r):
// keys in [lo, min(iq, S-1)] that are initial (< a) or separators (sepbits),
// plus the window [max(lo, iq - n + 1), min(iq, S-1)].
__device__ __forceinline__ uint64_t band_visible(int iq, int c0, int lo, int S, int a, int n,
                                                 uint64_t sepbits) {
  const int hi = (iq < S - 1 ? iq : S - 1) - c0;
  const int w0 = (lo > iq - n + 1 ? lo : iq - n + 1) - c0;
  return bit_range(w0, hi) | ((sepbits | bit_range(0, a - 1 - c0)) & bit_range(lo - c0, hi));
}

// B operand of step s from a 32x32 score accumulator: elements s*EPL..+EPL.
template <typename T>
__device__ __forceinline__ typename Traits<T>::frag acc_frag(const f32x16& a, int s);

template <>
__device__ __forceinline__ bf16x8 acc_frag<__bf16>(const f32x16& a, int s) {
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (__bf16)a[s * 8 + j];
  return f;
}

template <>
__device__ __forceinline__ float acc_frag<float>(const f32x16& a, int s) {
  return a[s];
}

}  // namespace sepattn
