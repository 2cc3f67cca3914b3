// Backward of SepLLM separator-sparse attention over the same kept tiles as
// the forward (training from scratch uses the separator mask in every layer:
// "How SepLLM Reorchestrates the Language Model for Speed and Efficiency",
// beiduofen.top, "The Mechanics of Compression"; atlas.scime.ai, "Approach").
//
// With P the masked softmax of scale*QK^T (recomputed from the forward's LSE),
//   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO * O)_i,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// dK/dV summed over the query heads of each kv group.
//
// Launches:
//   dQ       : query-major dQ over the forward's schedule, one workgroup per
//              query tile and head; each row's D = rowsum(dO * O) is computed
//              from its O and dO rows here and stored with log2(e) LSE for
//              the next kernel;
//   main     : one grid of two kinds of independent work items, so the long
//              anchor reductions run beside the short items instead of alone:
//     anchor dK/dV -- key-major over gathered anchor tiles (128 anchors per
//              workgroup), every query row at or after each anchor (an
//              initial token or a separator is seen by every later row); the
//              query tiles are split into chunks by the shapes and, with more
//              than one chunk, each (anchor tile, chunk) stores its fp32
//              partial in its own slot, else the workgroup stores the rows;
//     band dK/dV -- key-major over 128-key tiles of the local band for the
//              keys that are not anchors; a workgroup owns and stores its rows;
//   finalize : (several chunks only) anchor rows sum their slots and are stored.
//
// Key-major formulation: S = Q K^T with queries on the MFMA M axis and the
// workgroup's keys on the N axis (lanes), so dV^T = dO^T P and dK^T = Q^T dS
// take P and dS straight from the score registers; the transposed operands
// dO^T and Q^T are read from the row-major LDS tiles with the transpose read.
// Query-major (dQ): S^T = K Q^T as in the forward, dP^T = V dO^T,
// dQ^T = K^T dS^T.
#include <type_traits>

#include <algorithm>

#include "internal.hpp"
#include "tile.hpp"

namespace sepattn {

constexpr int kBwdThreads = 256;
constexpr int kKeysPerWG = 128;  // 4 waves x 32 keys

// Workgroups per CU the register budget of the main kernel targets: the
// d=128 and fp32 kernels keep more operands resident (key fragments and
// dK/dV accumulators) than fit two waves per SIMD.
#ifndef SEPATTN_BWD_OCC
#define SEPATTN_BWD_OCC 2
#endif
#ifndef SEPATTN_BWD_OCC128
#define SEPATTN_BWD_OCC128 1
#endif
template <typename T, int D>
constexpr int bwd_occupancy() {
  return sizeof(T) == 2 ? (D == 64 ? SEPATTN_BWD_OCC : SEPATTN_BWD_OCC128) : 1;
}
// Anchor work items aimed at, by head size: more items spread the anchor
// columns wider but write more fp32 partial slots.  Chosen by measurement on
// MI355X (8x12 heads of 2048 at d=64; 8 kv heads of 8192 and 32768 at
// d=128, where the anchor columns carry most of the backward's work and the
// time is not monotonic in the chunk count).
#ifndef SEPATTN_ANCHOR_MAX_TILES
#define SEPATTN_ANCHOR_MAX_TILES 40  // longest anchor chunk, in query tiles
#endif
#ifndef SEPATTN_ANCHOR_ITEMS64
#define SEPATTN_ANCHOR_ITEMS64 256
#endif
#ifndef SEPATTN_ANCHOR_ITEMS128
#define SEPATTN_ANCHOR_ITEMS128 1024
#endif
// Waves per SIMD of the dQ kernel, and whether it uses the lean form (the
// 32-key halves one after the other, K/V operands read in groups of 4, D
// subtracted per score) that fits two waves per SIMD at d=128.
#ifndef SEPATTN_DQ_OCC128
#define SEPATTN_DQ_OCC128 2
#endif
#ifndef SEPATTN_DQ_OCC64
#define SEPATTN_DQ_OCC64 3
#endif
#ifndef SEPATTN_DQ_LEAN64
#define SEPATTN_DQ_LEAN64 1
#endif
template <typename T, int D>
constexpr int dq_occupancy() {
  return sizeof(T) == 2 ? (D == 64 ? SEPATTN_DQ_OCC64 : SEPATTN_DQ_OCC128) : 1;
}
template <typename T, int D>
constexpr bool dq_lean() {
  return sizeof(T) == 2 ? (D == 64 ? SEPATTN_DQ_LEAN64 != 0 : true) : true;
}
#ifndef SEPATTN_FIN_BLOCKS
#define SEPATTN_FIN_BLOCKS 1024  // finalize workgroups in all (before the per-(b, kv head) floor of one)
#endif
#ifndef SEPATTN_DQ_INTERLEAVE
#define SEPATTN_DQ_INTERLEAVE 1  // interleaved order when both 32-key halves of a tile are live
#endif

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* LD;  // [B,Hq,SB,128]: per 64-row block, log2(e)*LSE then -D (zero past S); written by the dQ items
  float* dKa;   // [nchunk,B,Hkv,S,D] fp32 partials by chunk and anchor index (several chunks only)
  float* dVa;
  const uint8_t* is_sep;
  const int32_t* sep_prefix;
  const int32_t* anchor_pos;
  const int32_t* anchor_count;
  const int32_t* qtile;
  int B, Hq, Hkv, S, a, n, QT;
  int SB;                   // ceil(S / 64) row blocks of LD
  int nchunk, chunk_tiles;  // anchor work split: nchunk chunks of chunk_tiles query tiles
  int units;                // ceil(S / 128) key units per (sequence, kv head)
  int anchor_lanes;         // anchor work items per (sequence, kv head, chunk); each walks units
                            // lane, lane + anchor_lanes, ... until one has no anchor a query sees
  int anchor_stride;        // B * Hkv * nchunk rounded up to a multiple of 8: anchor items per lane
  int n_anchor_items, n_dq_items, n_band_items;
  float scale;
  float scale_log2;
};

// Split of the query tiles among anchor work items, from the shapes alone:
// aim at a number of (anchor tile, chunk, sequence, kv head) items that
// depends on the head size, guessing the anchor count from a separator
// density of 1/8; at most 16 chunks.
static void anchor_split(int B, int Hkv, int S, int QT, int d, int* nchunk, int* chunk_tiles) {
  const long units_guess = (4 + S / 8 + 127) / 128 + 1;
  const long target = d <= 64 ? SEPATTN_ANCHOR_ITEMS64 : SEPATTN_ANCHOR_ITEMS128;
  long n = (target + (long)B * Hkv * units_guess - 1) / ((long)B * Hkv * units_guess);
  if (n < 1) n = 1;
  // once the anchor columns are split, chunks of at most
  // SEPATTN_ANCHOR_MAX_TILES query tiles bound the longest anchor item
  if (n > 1) n = std::max(n, (long)(QT + SEPATTN_ANCHOR_MAX_TILES - 1) / SEPATTN_ANCHOR_MAX_TILES);
  if (n > 16) n = 16;  // the partial slots grow with the chunk count
  if (n > QT) n = QT;
  const int ct = (int)((QT + n - 1) / n);
  *chunk_tiles = ct;
  *nchunk = (QT + ct - 1) / ct;
}

// Double-buffered LDS tiles as separate arrays: each step names its buffer
// at compile time, so the compiler can tell a DMA into one buffer from the
// reads of the other and does not wait for that DMA before the reads.
template <typename T>
struct SmemBufs {
  T* a[2];      // Q tiles (dK/dV items), K tiles (dQ items)
  T* b[2];      // dO tiles, V tiles
  float* l[2];  // per-wave log2(e)*LSE and D copies (dK/dV items)
};
typedef std::integral_constant<int, 0> Buf0;
typedef std::integral_constant<int, 1> Buf1;

// ---------------------------------------------------------------------------
// key-major dK/dV of one key unit (128 keys) against a range of query tiles
// ---------------------------------------------------------------------------
template <typename T, int D, bool ANCHOR>
__device__ __forceinline__ bool dkdv_item(const BwdArgs& p, int b, int g, int unit, int chunk,
                                          const SmemBufs<T>& sm) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef TileRows<T, D, kBwdThreads> Regs;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NF = D / KSTEP;    // K/V fragments per lane
  constexpr int NDB = D / 32;      // 32-row blocks of dK^T / dV^T
  constexpr int SPB = 32 / KSTEP;  // MFMA steps over one 32-query block
  typedef TileDMA<T, D, kBwdThreads> DMA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so tests on it are scalar branches
  const int hh = lane >> 5;
  const int kc = lane & 31;
  const int grp = p.Hq / p.Hkv;
  int rb_begin, rb_end;  // 64-row query blocks [rb_begin, rb_end) the item steps through
  if constexpr (ANCHOR) {
    // Every row at or after an anchor's position sees it (an initial token or
    // a separator: through the gathered anchor tiles, or within its window
    // through the band), so the anchor items take the whole column of every
    // anchor and the band items leave anchors out.  The unit's rows start at
    // the block that holds its first anchor (position p0); a chunk is a range
    // of query tiles.
    const int a0 = unit * kKeysPerWG;
    const int p0 = a0 < p.S ? p.anchor_pos[(size_t)b * p.S + a0] : -1;
    if (p0 < 0) return false;  // past the last anchor, as are the units after it
    constexpr int BPQ = kQTile / kKTile;  // 64-row blocks per query tile
    rb_begin = max(p0 / kKTile, chunk * p.chunk_tiles * BPQ);
    rb_end = min(p.SB, (chunk + 1) * p.chunk_tiles * BPQ);
    // no row of this chunk sees the unit: nothing to add, and the finalize
    // never reads this chunk's slot for these anchors
    if (rb_begin >= rb_end) return true;
  } else {
    // rows [k0, k1 + n - 1]: the windows of the unit's keys
    const int k0 = unit * kKeysPerWG;
    const int k1 = min(k0 + kKeysPerWG - 1, p.S - 1);
    rb_begin = k0 / kKTile;
    rb_end = min(p.S - 1, k1 + p.n - 1) / kKTile + 1;
  }
  const int n_rb = max(0, rb_end - rb_begin);
  const int n_it = grp * n_rb;  // (query head, 64-row block)

  // this lane's key
  const int kidx = unit * kKeysPerWG + 32 * w + kc;  // key row (band) or anchor index (anchor)
  int krow;
  // (anchor-list entries past the anchor count are -1)
  if constexpr (ANCHOR) krow = kidx < p.S ? p.anchor_pos[(size_t)b * p.S + kidx] : -1;
  else krow = kidx < p.S ? kidx : -1;
  // band: anchors (initial tokens and separators) are the anchor items' keys
  const bool key_anchor =
      (!ANCHOR && krow >= 0) ? (krow < p.a || p.is_sep[(size_t)b * p.S + krow] != 0) : false;
  // rows [krow, q_hi] see this lane's key: every later row for an anchor,
  // the window for a band key
  const int q_hi = ANCHOR ? p.S - 1 : min(p.S - 1, krow + p.n - 1);
  const bool key_live = krow >= 0 && !key_anchor;

  const T* Kg = (const T*)p.k + (((size_t)b * p.Hkv + g) * p.S) * D;
  const T* Vg = (const T*)p.v + (((size_t)b * p.Hkv + g) * p.S) * D;

  // Step order.  Anchor items walk the row blocks from the chunk's last one
  // down, the query heads inside: every anchor unit of a (sequence, kv head,
  // chunk) then reads the same Q/dO tiles at the same step, while they run
  // side by side on one XCD, so a tile comes from HBM once for all of them
  // (they differ only in where they stop).  Band items: head by head.
  auto it_head = [&](int it) {
    if constexpr (ANCHOR) return g * grp + it % grp;
    else return g * grp + it / n_rb;
  };
  auto it_row0 = [&](int it) {
    if constexpr (ANCHOR) return (rb_end - 1 - it / grp) * kKTile;
    else return (rb_begin + it % n_rb) * kKTile;
  };
  const unsigned ldbytes = (unsigned)((size_t)p.SB * 2 * kKTile * sizeof(float));
  unsigned uoff[Regs::NU];
#pragma unroll
  for (int u = 0; u < Regs::NU; ++u) uoff[u] = tile_unit_offset<T, D, kBwdThreads>(tid, u);
  // Q and dO tiles of step `it` straight into LDS buffer B
  auto issue = [&](int it, auto B) {
    constexpr int buf = decltype(B)::value;
    const int h = it_head(it);
    const int r0 = it_row0(it);
    const size_t bh = (size_t)b * p.Hq + h;
    // consecutive rows r0 ..: a resource from row r0 to the end, constant offsets
    const size_t rbase = (bh * p.S + r0) * D;
    const unsigned rbytes = (unsigned)((size_t)(p.S - r0) * D * sizeof(T));
    DMA::issue_rows(buffer_rsrc((const T*)p.q + rbase, rbytes), uoff, sm.a[buf], tid);
    DMA::issue_rows(buffer_rsrc((const T*)p.dout + rbase, rbytes), uoff, sm.b[buf], tid);
    // this wave's own copy of the tile's 64 (log2(e)*LSE, -D) pairs: lanes
    // 0..31 carry the 512-byte block, lanes 32..63 read past the buffer
    // (zeros into the unused half of the wave's 1 KB slot)
    const unsigned off = lane < 32 ? (unsigned)((r0 / kKTile) * 2 * kKTile * 4 + lane * 16) : ldbytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(p.LD + bh * p.SB * 2 * kKTile, ldbytes),
                                             (__attribute__((address_space(3))) void*)(sm.l[buf] + w * 256),
                                             16, off, 0, 0, 0);
  };

  if (n_it > 0) issue(0, Buf0{});

  // this lane's key rows (a lane without a key reads row 0: its column is
  // masked out of every tile and never stored)
  frag kf[NF], vf[NF];
  {
    const int kr = krow >= 0 ? krow : 0;
#pragma unroll
    for (int c = 0; c < NF; ++c) {
      kf[c] = *(const frag*)(Kg + (size_t)kr * D + c * KSTEP + EPL * hh);
      vf[c] = *(const frag*)(Vg + (size_t)kr * D + c * KSTEP + EPL * hh);
    }
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // step `it` reads buffer B = it & 1
  auto step = [&](int it, auto B) {
    constexpr int buf = decltype(B)::value;
    T* Qb = sm.a[buf];
    T* dOb = sm.b[buf];
    float* lb = sm.l[buf] + w * 256;  // log2(e)*LSE of the tile's 64 rows
    float* db_ = lb + kKTile;         // then -D
    wait_vm_all();    // this wave's part of tile `it` (and its LSE/D copy) has landed in LDS
    __syncthreads();  // tile `it` visible; every wave is done with tile it-1's buffer
    const int r0 = it_row0(it);
    if (it + 1 < n_it) issue(it + 1, std::integral_constant<int, 1 - buf>{});

    // query-row range [ql, qh] of the rows that see this lane's key
    const int ql = key_live ? krow : 1;
    const int qh = key_live ? q_hi : 0;
    // every row of this 64-row chunk sees every key of the wave: skip the tests
    const bool full = __all(ql <= r0 && qh >= r0 + kKTile - 1);
    // bit r: row r0 + r sees this lane's key
    const uint64_t vis = full ? ~0ull : bit_range(ql - r0, qh - r0);
    // 32 rows that see no key of the wave add nothing (wave-uniform skip)
    bool live[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) live[mb] = full || __any((uint32_t)(vis >> (32 * mb)) != 0u);

    // S = Q K^T and dP = dO V^T for the 32-row block mb (operands first, then
    // the MFMAs back to back)
    auto scores = [&](int mb, f32x16& sacc, f32x16& pacc) {
      frag qq[NF], oo[NF];
#pragma unroll
      for (int c = 0; c < NF; ++c) {
        qq[c] = read_x<T, D>(Qb, mb, c, lane);
        oo[c] = read_x<T, D>(dOb, mb, c, lane);
      }
      sacc = f32x16{};
      // dP - D: the accumulation starts from -D of each row
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 n4 = *(const f32x4*)&db_[32 * mb + 8 * i4 + 4 * hh];
#pragma unroll
        for (int e = 0; e < 4; ++e) pacc[4 * i4 + e] = n4[e];
      }
#pragma unroll
      for (int c = 0; c < NF; ++c) {
        sacc = Tr::mfma(qq[c], kf[c], sacc);
        pacc = Tr::mfma(oo[c], vf[c], pacc);
      }
    };
    // P (masked exponents become -inf, so P = 0) and dS = P (dP - D), as MFMA
    // operands; rows are queries r0 + 32mb + acc_row(i), the column is this
    // lane's key (rows past S were loaded as zeros with zero LSE and D, so
    // they add nothing)
    auto probs = [&](int mb, f32x16& sacc, f32x16& pacc, frag* pf, frag* sf) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 l4 = *(const f32x4*)&lb[32 * mb + 8 * i4 + 4 * hh];
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[4 * i4 + e] = __builtin_fmaf(sacc[4 * i4 + e], p.scale_log2, -l4[e]);
      }
      if (!full) {  // wave-uniform
        const uint32_t vw = (uint32_t)(vis >> (32 * mb + 4 * hh));
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = keep_or_neg_inf(sacc[i], bit_mask(vw, acc_bit(i)));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(sacc[i]);
        sacc[i] = pv;
        pacc[i] = pv * pacc[i];  // pacc holds dP - D
      }
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl) {
        pf[sl] = acc_frag<T>(sacc, sl);
        sf[sl] = acc_frag<T>(pacc, sl);
      }
    };
    // dV^T += dO^T P ; dK^T += Q^T dS (per step: operands first, then MFMAs)
    auto grads = [&](int mb, const frag* pf, const frag* sf) {
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl) {
        frag ot[NDB], qt_[NDB];
#pragma unroll
        for (int dbk = 0; dbk < NDB; ++dbk) {
          ot[dbk] = read_xt<T, D>(dOb, mb, sl, 32 * dbk, lane);
          qt_[dbk] = read_xt<T, D>(Qb, mb, sl, 32 * dbk, lane);
        }
#pragma unroll
        for (int dbk = 0; dbk < NDB; ++dbk) {
          dv[dbk] = Tr::mfma(ot[dbk], pf[sl], dv[dbk]);
          dk[dbk] = Tr::mfma(qt_[dbk], sf[sl], dk[dbk]);
        }
      }
    };

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (!live[mb]) continue;
      f32x16 sacc, pacc;
      frag pf[SPB], sf[SPB];
      scores(mb, sacc, pacc);
      probs(mb, sacc, pacc, pf, sf);
      grads(mb, pf, sf);
    }
  };

  {
    int it = 0;
    for (; it + 1 < n_it; it += 2) {
      step(it, Buf0{});
      step(it + 1, Buf1{});
    }
    if (it < n_it) step(it, Buf0{});
  }

  // epilogue: this lane holds column kidx of dK^T / dV^T, rows d = 32db + acc_row(i).
  // A band key's column and, with one chunk, an anchor's are complete and
  // stored in the input type; with several chunks an anchor's column is an
  // fp32 partial in the chunk's slot, summed by the finalize kernel.
  if (!key_live) return true;
  float* ka = nullptr;
  float* va = nullptr;
  T* dkg = nullptr;
  T* dvg = nullptr;
  if (ANCHOR && p.nchunk > 1) {
    const size_t off = (((size_t)chunk * p.B + b) * p.Hkv + g) * p.S + kidx;
    ka = p.dKa + off * D;
    va = p.dVa + off * D;
  } else {
    dkg = (T*)p.dk + (((size_t)b * p.Hkv + g) * p.S + krow) * D;
    dvg = (T*)p.dv + (((size_t)b * p.Hkv + g) * p.S + krow) * D;
  }
#pragma unroll
  for (int dbk = 0; dbk < NDB; ++dbk)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * dbk + 8 * r4 + 4 * hh;
      const f32x4 kv4 = {dk[dbk][4 * r4] * p.scale, dk[dbk][4 * r4 + 1] * p.scale, dk[dbk][4 * r4 + 2] * p.scale,
                         dk[dbk][4 * r4 + 3] * p.scale};
      const f32x4 vv4 = {dv[dbk][4 * r4], dv[dbk][4 * r4 + 1], dv[dbk][4 * r4 + 2], dv[dbk][4 * r4 + 3]};
      if (ka) {
        *(f32x4*)(ka + d0) = kv4;
        *(f32x4*)(va + d0) = vv4;
      } else if constexpr (EPL == 8) {
        u32x2 pk, pv2;
        pk[0] = pack_bf16x2(kv4[0], kv4[1]);
        pk[1] = pack_bf16x2(kv4[2], kv4[3]);
        pv2[0] = pack_bf16x2(vv4[0], vv4[1]);
        pv2[1] = pack_bf16x2(vv4[2], vv4[3]);
        *(u32x2*)(dkg + d0) = pk;
        *(u32x2*)(dvg + d0) = pv2;
      } else {
        *(f32x4*)(dkg + d0) = kv4;
        *(f32x4*)(dvg + d0) = vv4;
      }
    }
  return true;
}

// ---------------------------------------------------------------------------
// query-major dQ of one query tile over the forward's schedule
// ---------------------------------------------------------------------------
// LEAN: fewer registers (the 32-key halves one after the other, K/V operands
// read in groups of 4), for a kernel that runs two waves per SIMD at d=128
template <typename T, int D, bool LEAN = false>
__device__ __forceinline__ void dq_item(const BwdArgs& p, int b, int h, int qi, const SmemBufs<T>& sm) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef TileRows<T, D, kBwdThreads> Regs;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NQF = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr int SPB = 32 / KSTEP;
  typedef TileDMA<T, D, kBwdThreads> DMA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so tests on it are scalar branches
  const int hh = lane >> 5;
  const int qc = lane & 31;
  const int g = h / (p.Hq / p.Hkv);

  // band tiles first (rows follow from q0 and n), gathered anchor tiles last
  const int q0 = qi * kQTile;
  const int lo = max(0, q0 - p.n + 1);
  const int kb = lo / kKTile, ke = min(q0 + kQTile - 1, p.S - 1) / kKTile;
  const int n_band = ke - kb + 1;
  const int n_anchor = p.qtile[((size_t)b * p.QT + qi) * kQF + 1];
  const int n_at = (n_anchor + kKTile - 1) / kKTile;
  const int n_tiles = n_band + n_at;

  const int iq = q0 + 32 * w + qc;
  const bool q_ok = iq < p.S;
  const size_t qoff = (((size_t)b * p.Hq + h) * p.S) * D;
  const T* Qg = (const T*)p.q + qoff;
  const T* dOg = (const T*)p.dout + qoff;
  const T* Kg = (const T*)p.k + (((size_t)b * p.Hkv + g) * p.S) * D;
  const T* Vg = (const T*)p.v + (((size_t)b * p.Hkv + g) * p.S) * D;
  const int32_t* anc = p.anchor_pos + (size_t)b * p.S;
  const uint8_t* sepf = p.is_sep + (size_t)b * p.S;

  auto src_of = [&](int t) {
    RowSrc r;
    if (t >= n_band) {
      r.anchor = anc;
      r.base = (t - n_band) * kKTile;
      r.limit = n_anchor;
    } else {
      r.anchor = nullptr;
      r.base = (kb + t) * kKTile;
      r.limit = p.S;
    }
    return r;
  };
  const unsigned kv_bytes = (unsigned)((size_t)p.S * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t Krs = buffer_rsrc(Kg, kv_bytes), Vrs = buffer_rsrc(Vg, kv_bytes);
  // Source rows of anchor tiles come from the anchor list; their loads are
  // issued one tile ahead (fetch), unconditionally with a clamped index, so
  // no step waits on them before it can issue its DMA (resolve).
  int arow[Regs::NU];
  auto fetch = [&](int t) {
    const RowSrc r = src_of(t);
#pragma unroll
    for (int u = 0; u < Regs::NU; ++u) arow[u] = anc[min(r.base + Regs::row_of(tid, u), r.limit - 1)];
  };
  auto resolve = [&](int t, int* rows) {
    const RowSrc r = src_of(t);
#pragma unroll
    for (int u = 0; u < Regs::NU; ++u) {
      const int x = r.base + Regs::row_of(tid, u);
      rows[u] = x < r.limit ? (r.anchor ? arow[u] : x) : -1;
    }
  };
  // K and V tiles of tile t straight into LDS buffer B (its separator
  // flags, for band tiles, into sflag).  Band tiles (consecutive rows) use
  // per-thread constant offsets into a buffer resource that starts at the
  // tile; anchor tiles take their rows from the list.
  unsigned uoff[Regs::NU];
#pragma unroll
  for (int u = 0; u < Regs::NU; ++u) uoff[u] = tile_unit_offset<T, D, kBwdThreads>(tid, u);
  int sflag = 0;
  auto issue = [&](int t, auto B) {
    constexpr int buf = decltype(B)::value;
    sflag = 0;
    if (t < n_band) {  // wave-uniform
      const int r0 = (kb + t) * kKTile;
      const unsigned bytes = (unsigned)((size_t)(p.S - r0) * D * sizeof(T));
      DMA::issue_rows(buffer_rsrc(Kg + (size_t)r0 * D, bytes), uoff, sm.a[buf], tid);
      DMA::issue_rows(buffer_rsrc(Vg + (size_t)r0 * D, bytes), uoff, sm.b[buf], tid);
      const int j = r0 + lane;
      sflag = j < p.S ? (int)sepf[j] : 0;
    } else {
      int rows[Regs::NU];
      resolve(t, rows);
      DMA::issue(Krs, kv_bytes, rows, sm.a[buf], tid);
      DMA::issue(Vrs, kv_bytes, rows, sm.b[buf], tid);
    }
  };
  // the anchor-list entries of anchor tiles only
  auto fetch_anchor = [&](int t) {
    if (t >= n_band) fetch(t);
  };

  issue(0, Buf0{});  // a band tile
  fetch_anchor(min(1, n_tiles - 1));

  frag qf[NQF], of[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) {
    if (q_ok) {
      qf[c] = *(const frag*)(Qg + (size_t)iq * D + c * KSTEP + EPL * hh);
      of[c] = *(const frag*)(dOg + (size_t)iq * D + c * KSTEP + EPL * hh);
    } else {
      qf[c] = frag{};
      of[c] = frag{};
    }
  }
  const float lse2 = q_ok ? p.lse[((size_t)b * p.Hq + h) * p.S + iq] * 1.4426950408889634f : 0.f;
  // D_i = rowsum(dO * O)_i of this lane's row: the lane pair (l, l ^ 32)
  // holds the row's two halves of dO; the same halves of O are loaded here
  float Di = 0.f;
  {
    const T* Og = (const T*)p.o + qoff;
#pragma unroll
    for (int c = 0; c < NQF; ++c) {
      const frag oo = q_ok ? *(const frag*)(Og + (size_t)iq * D + c * KSTEP + EPL * hh) : frag{};
      if constexpr (EPL == 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) Di += (float)of[c][e] * (float)oo[e];
      } else {
        Di += of[c] * oo;
      }
    }
    Di = pair_sum(Di);
  }
  // this row's (log2(e) LSE, -D) for the key-major items, which read them
  // per 64-row block (rows past S, up to the block's end, get zeros)
  if (hh == 0 && iq < p.SB * kKTile) {
    float* blk = p.LD + (((size_t)b * p.Hq + h) * p.SB + iq / kKTile) * (2 * kKTile);
    blk[iq % kKTile] = lse2;
    blk[kKTile + iq % kKTile] = -Di;
  }
  f32x16 negD;  // dP^T - D: every accumulation starts from -D of this lane's row
#pragma unroll
  for (int i = 0; i < 16; ++i) negD[i] = -Di;

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  const int wrow0 = q0 + 32 * w;
  const int wrow1 = min(wrow0 + 31, p.S - 1);

  // step t reads buffer B = t & 1
  auto step = [&](int t, auto B) {
    constexpr int buf = decltype(B)::value;
    T* K = sm.a[buf];
    T* V = sm.b[buf];
    const uint64_t sepbits = __ballot(sflag != 0);
    wait_vm_all();  // this wave's part of tile t has landed in LDS
    __syncthreads();
    if (t + 1 < n_tiles) {
      issue(t + 1, std::integral_constant<int, 1 - buf>{});
      fetch_anchor(min(t + 2, n_tiles - 1));
    }

    const bool anchor_tile = t >= n_band;
    bool full;
    uint64_t vis;
    if (anchor_tile) {
      const int nv = n_anchor - (t - n_band) * kKTile;
      full = nv >= kKTile;
      vis = bit_range(0, nv - 1);
    } else {
      const int c0 = (kb + t) * kKTile;
      full = c0 >= lo && c0 + kKTile - 1 <= wrow0 && wrow1 - c0 < p.n && c0 + kKTile - 1 < p.S;
      vis = band_visible(iq, c0, lo, p.S, p.a, p.n, sepbits);
    }
    // a 32-key half that no query of the wave sees is skipped (wave-uniform)
    bool live[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) live[k2] = full || __any((uint32_t)(vis >> (32 * k2)) != 0u);

    // rows past S have zero Q, dO, LSE and D, so their dS is zero unmasked.
    // S^T = K Q^T and dP^T = V dO^T for the 32-key half k2 (operands first,
    // then the MFMAs back to back)
    auto scores = [&](int k2, f32x16& sacc, f32x16& pacc) {
      constexpr int GRP = LEAN && NQF > 4 ? 4 : NQF;  // operands read per group
      sacc = f32x16{};
      if constexpr (LEAN) pacc = f32x16{};  // D subtracted per score below
      else pacc = negD;
#pragma unroll
      for (int c0 = 0; c0 < NQF; c0 += GRP) {
        frag kk[GRP], vv[GRP];
#pragma unroll
        for (int c = 0; c < GRP; ++c) {
          kk[c] = read_x<T, D>(K, k2, c0 + c, lane);
          vv[c] = read_x<T, D>(V, k2, c0 + c, lane);
        }
#pragma unroll
        for (int c = 0; c < GRP; ++c) {
          sacc = Tr::mfma(kk[c], qf[c0 + c], sacc);
          pacc = Tr::mfma(vv[c], of[c0 + c], pacc);
        }
      }
    };
    // dS^T = P^T (dP^T - D) as MFMA operands (masked exponents become -inf, so P = 0)
    auto dsfrags = [&](int k2, f32x16& sacc, f32x16& pacc, frag* sf) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = __builtin_fmaf(sacc[i], p.scale_log2, -lse2);
      if (!full) {  // wave-uniform
        const uint32_t vw = (uint32_t)(vis >> (32 * k2 + 4 * hh));
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = keep_or_neg_inf(sacc[i], bit_mask(vw, acc_bit(i)));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[i] = fast_exp2(sacc[i]) * (LEAN ? pacc[i] - Di : pacc[i]);  // dP^T - D
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl) sf[sl] = acc_frag<T>(pacc, sl);
    };
    // dQ^T += K^T dS^T with the K^T operands of the half read first
    auto dqmm = [&](int k2, const frag* sf) {
      if constexpr (LEAN) {
#pragma unroll
        for (int sl = 0; sl < SPB; ++sl) {
          frag kt[NDB];
#pragma unroll
          for (int db = 0; db < NDB; ++db) kt[db] = read_xt<T, D>(K, k2, sl, 32 * db, lane);
#pragma unroll
          for (int db = 0; db < NDB; ++db) dq[db] = Tr::mfma(kt[db], sf[sl], dq[db]);
        }
      } else {
        frag kt[SPB][NDB];
#pragma unroll
        for (int sl = 0; sl < SPB; ++sl)
#pragma unroll
          for (int db = 0; db < NDB; ++db) kt[sl][db] = read_xt<T, D>(K, k2, sl, 32 * db, lane);
#pragma unroll
        for (int sl = 0; sl < SPB; ++sl)
#pragma unroll
          for (int db = 0; db < NDB; ++db) dq[db] = Tr::mfma(kt[sl][db], sf[sl], dq[db]);
      }
    };

    if (SEPATTN_DQ_INTERLEAVE && !LEAN && live[0] && live[1]) {
      // half 1's scores enter the MFMA pipe before half 0's dQ products, and
      // half 1's exponentials overlap those products
      f32x16 s0, p0, s1, p1;
      frag sf0[SPB], sf1[SPB];
      scores(0, s0, p0);
      dsfrags(0, s0, p0, sf0);
      scores(1, s1, p1);
      dqmm(0, sf0);
      dsfrags(1, s1, p1, sf1);
      dqmm(1, sf1);
    } else {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        if (!live[k2]) continue;
        f32x16 sacc, pacc;
        frag sf[SPB];
        scores(k2, sacc, pacc);
        dsfrags(k2, sacc, pacc, sf);
        dqmm(k2, sf);
      }
    }
  };

  {
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, Buf0{});
      step(t + 1, Buf1{});
    }
    if (t < n_tiles) step(t, Buf0{});
  }

  if constexpr (EPL == 8) {
    // dQ goes out as whole rows through the first pair of tile buffers
    __syncthreads();  // every wave is done with the last tile's buffers
    T* dQb = (T*)p.dq + qoff + (size_t)q0 * D;
    const int nrows = p.S - q0;
    store_rows_via_lds<D, kBwdThreads>(sm.a[0], sm.b[0], dq, p.scale,
                                       [&](int r) { return r < nrows ? dQb + (size_t)r * D : nullptr; }, uoff, tid);
    return;
  }
  if (q_ok) {
    T* dQg = (T*)p.dq + qoff + (size_t)iq * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * hh;
        if constexpr (EPL == 8) {
          u32x2 pk;
          pk[0] = pack_bf16x2(dq[db][4 * r4 + 0] * p.scale, dq[db][4 * r4 + 1] * p.scale);
          pk[1] = pack_bf16x2(dq[db][4 * r4 + 2] * p.scale, dq[db][4 * r4 + 3] * p.scale);
          *(u32x2*)(dQg + d0) = pk;
        } else {
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = dq[db][4 * r4 + e] * p.scale;
          *(f32x4*)(dQg + d0) = ov;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// main: anchor dK/dV items, then dQ items (heaviest query tiles first), then
// band dK/dV items, in one 1-D grid
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(kBwdThreads, (bwd_occupancy<T, D>())) bwd_main_kernel(BwdArgs p) {
  typedef TileGeom<T, D> G;
  __shared__ __attribute__((aligned(16))) T smA0[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T smA1[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T smB0[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T smB1[G::ELEMS];
  __shared__ __attribute__((aligned(16))) float smL0[4 * 256];  // [wave][LSE x 64, D x 64, spare]
  __shared__ __attribute__((aligned(16))) float smL1[4 * 256];
  const SmemBufs<T> sm = {{smA0, smA1}, {smB0, smB1}, {smL0, smL1}};

  int x = blockIdx.x;
  const int BG = p.B * p.Hkv;
  if (x < p.n_anchor_items) {
    // lane-major so the first anchor units come first; a lane's items are
    // padded to a multiple of the 8 XCDs (anchor_stride), so that every lane
    // of one (sequence, kv head, chunk) runs on the same XCD.  Chunk-major
    // within a lane: the XCD of a group is (chunk * B*Hkv + bg) mod 8, so
    // with B*Hkv a multiple of 8 every XCD gets all chunks of its (sequence,
    // kv head)s; numbered bg-major instead, (bg * nchunk + chunk) mod 8, an
    // even chunk count gives each XCD only some chunk indices, and the later
    // chunks hold far more anchor work
    const int lane0 = x / p.anchor_stride;
    const int r = x - lane0 * p.anchor_stride;
    if (r >= BG * p.nchunk) return;
    const int chunk = r / BG;
    const int bg = r - chunk * BG;
    for (int unit = lane0; unit < p.units; unit += p.anchor_lanes) {
      if (!dkdv_item<T, D, true>(p, bg / p.Hkv, bg % p.Hkv, unit, chunk, sm)) break;
      __syncthreads();  // the next unit refills the tile buffers
    }
    return;
  }
  // band items: the units of one (sequence, kv head) share query tiles, so
  // keep each (sequence, kv head) on one XCD's L2
  const int li = xcd_local_index(blockIdx.x, p.n_anchor_items, p.n_band_items);
  const int bg = li / p.units;
  const int unit = li - bg * p.units;
  dkdv_item<T, D, false>(p, bg / p.Hkv, bg % p.Hkv, unit, 0, sm);
}

// dQ items, the first kernel of the backward: they also produce every row's
// D = rowsum(dO * O) (and log2(e) LSE) for the key-major items of the main
// kernel.  A kernel of their own also fits more waves per SIMD than the
// key-major items' registers allow.
template <typename T, int D>
__global__ void __launch_bounds__(kBwdThreads, (dq_occupancy<T, D>())) bwd_dq_kernel(BwdArgs p) {
  typedef TileGeom<T, D> G;
  __shared__ __attribute__((aligned(16))) T smA0[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T smA1[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T smB0[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T smB1[G::ELEMS];
  const SmemBufs<T> sm = {{smA0, smA1}, {smB0, smB1}, {nullptr, nullptr}};
  const int x = blockIdx.x;
  const int BH = p.B * p.Hq;
  const int qi = p.QT - 1 - x / BH;  // heaviest query tiles (most anchors) first
  int b, h;
  query_column(x % BH, p.B, p.Hq, p.Hkv, b, h);
  dq_item<T, D, dq_lean<T, D>()>(p, b, h, qi, sm);
}

// ---------------------------------------------------------------------------
// finalize (several anchor chunks only): anchor rows = sum of their partial
// slots, stored in the input type
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_finalize_kernel(BwdArgs p) {
  constexpr int TPR = D / 4;  // threads per row, 4 elements each
  const int bg = blockIdx.y;
  const int b = bg / p.Hkv;
  const int n_anchor = p.anchor_count[b];
  const int c4 = (threadIdx.x % TPR) * 4;
  const size_t cstride = (size_t)p.B * p.Hkv * p.S * D;
  // the anchor count is known on the device only: a fixed number of
  // workgroups per (sequence, kv head) strides over it
  for (int ai = blockIdx.x * (256 / TPR) + threadIdx.x / TPR; ai < n_anchor; ai += gridDim.x * (256 / TPR)) {
    const size_t off = ((size_t)bg * p.S + ai) * D + c4;
    const int krow = p.anchor_pos[(size_t)b * p.S + ai];
    // the chunks that hold a row at or after the anchor (earlier chunks'
    // slots were not written)
    const int cmin = min((krow / kQTile) / p.chunk_tiles, p.nchunk - 1);
    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    // the partials of 4 slots in flight at once (slots past the last re-read
    // it and are not added)
    for (int c0 = cmin; c0 < p.nchunk; c0 += 4) {
      f32x4 k4[4], v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t cc = (size_t)min(c0 + j, p.nchunk - 1);
        k4[j] = *(const f32x4*)(p.dKa + cc * cstride + off);
        v4[j] = *(const f32x4*)(p.dVa + cc * cstride + off);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool use = c0 + j < p.nchunk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk[e] += use ? k4[j][e] : 0.f;
          sv[e] += use ? v4[j][e] : 0.f;
        }
      }
    }
    const size_t o = ((size_t)bg * p.S + krow) * D + c4;
    if constexpr (sizeof(T) == 2) {
      *(u32x2*)((uint16_t*)p.dk + o) = u32x2{pack_bf16x2(sk[0], sk[1]), pack_bf16x2(sk[2], sk[3])};
      *(u32x2*)((uint16_t*)p.dv + o) = u32x2{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
    } else {
      *(f32x4*)((float*)p.dk + o) = sk;
      *(f32x4*)((float*)p.dv + o) = sv;
    }
  }
}

// ---------------------------------------------------------------------------

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d) {
  const int QT = (S + kQTile - 1) / kQTile;
  int nchunk, ct;
  anchor_split(B, Hkv, S, QT, d, &nchunk, &ct);
  const size_t SB = (S + kKTile - 1) / kKTile;
  // per-row (log2(e) LSE, -D); then, with several anchor chunks, one fp32
  // partial slot per chunk for dK and for dV
  return a256((size_t)B * Hq * SB * 2 * kKTile * 4) +
         (nchunk > 1 ? 2 * a256((size_t)nchunk * B * Hkv * S * d * 4) : 0);
}

template <typename T, int D>
static hipError_t launch_bwd_t(BwdArgs& a, hipStream_t stream, hipEvent_t* ev) {
  const int main_blocks = a.n_anchor_items + a.n_band_items;
  const int fin_rows_per_block = 256 / (D / 4);
  hipError_t e;
  if (ev && ev[0] && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3(a.n_dq_items), dim3(kBwdThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && ev[1] && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main_kernel<T, D>), dim3(main_blocks), dim3(kBwdThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && ev[2] && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  const int fin_x = std::max(1, std::min((a.S + fin_rows_per_block - 1) / fin_rows_per_block,
                                         SEPATTN_FIN_BLOCKS / (a.B * a.Hkv)));
  if (a.nchunk > 1) {
    hipLaunchKernelGGL((bwd_finalize_kernel<T, D>), dim3(fin_x, a.B * a.Hkv), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev && ev[3] && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, const AttnShape& sh, const sepattn_index& idx, void* dq,
                      void* dk, void* dv, void* ws, hipStream_t stream, hipEvent_t* ev) {
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  char* w = (char*)ws;
  a.SB = (sh.S + kKTile - 1) / kKTile;
  a.LD = (float*)w;
  w += a256((size_t)sh.B * sh.Hq * a.SB * 2 * kKTile * 4);
  a.QT = (sh.S + kQTile - 1) / kQTile;
  anchor_split(sh.B, sh.Hkv, sh.S, a.QT, sh.d, &a.nchunk, &a.chunk_tiles);
  a.dKa = a.nchunk > 1 ? (float*)w : nullptr;
  w += a.nchunk > 1 ? a256((size_t)a.nchunk * sh.B * sh.Hkv * sh.S * sh.d * 4) : 0;
  a.dVa = a.nchunk > 1 ? (float*)w : nullptr;
  a.is_sep = idx.is_sep;
  a.sep_prefix = idx.sep_prefix;
  a.anchor_pos = idx.anchor_pos;
  a.anchor_count = idx.anchor_count;
  a.qtile = idx.qtile;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.a = idx.a;
  a.n = idx.n < idx.S ? idx.n : idx.S;  // as the index builders store it
  a.units = (sh.S + kKeysPerWG - 1) / kKeysPerWG;
  a.anchor_lanes = std::min(a.units, std::max(2, sh.S / 2048));
  a.anchor_stride = (sh.B * sh.Hkv * a.nchunk + 7) / 8 * 8;
  a.n_anchor_items = a.anchor_lanes * a.anchor_stride;
  a.n_dq_items = sh.B * sh.Hq * a.QT;
  a.n_band_items = a.units * sh.B * sh.Hkv;
  a.scale = sh.scale;
  a.scale_log2 = sh.scale * 1.4426950408889634f;
  if (sh.dtype == SEPATTN_BF16) {
    if (sh.d == 64) return launch_bwd_t<__bf16, 64>(a, stream, ev);
    return launch_bwd_t<__bf16, 128>(a, stream, ev);
  }
  if (sh.d == 64) return launch_bwd_t<float, 64>(a, stream, ev);
  return launch_bwd_t<float, 128>(a, stream, ev);
}

}  // namespace sepattn
