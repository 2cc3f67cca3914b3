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
// Kernels, in launch order:
//   pre   : D_i = rowsum(dO * O)
//   dkdv<anchor>: key-major over gathered anchor tiles (128 anchors per
//           workgroup), the query tiles split into a few chunks; each (anchor
//           tile, chunk) stores its fp32 partial in its own slot (plain
//           stores, zeros when the chunk sees none of the anchors)
//   dkdv<band>  : key-major over 128-key tiles of the local band; each
//           workgroup owns its rows, adds the chunk partials of rows that are
//           anchors, scales and stores dK/dV in the input type
//   dq    : query-major, same schedule as the forward
//
// Key-major formulation: S = Q K^T with queries on the MFMA M axis and the
// workgroup's keys on the N axis (lanes), so dV^T = dO^T P and dK^T = Q^T dS
// take P and dS straight from the score registers; Q and dO are staged in LDS
// both row-major and transposed.  Query-major (dq): S^T = K Q^T as in the
// forward, dP^T = V dO^T, dQ^T = K^T dS^T with K transposed in LDS.
#include "internal.hpp"
#include "tile.hpp"

namespace sepattn {

constexpr int kBwdThreads = 256;

// Workgroups per CU the register budget targets: the d=128 and fp32 backward
// kernels keep more operands resident than fit two waves per SIMD.
template <typename T, int D>
constexpr int bwd_occupancy() {
  return (sizeof(T) == 2 && D == 64) ? 2 : 1;
}
constexpr int kKeysPerWG = 128;   // 4 waves x 32 keys

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
  float* Dvec;  // [B,Hq,S]
  float* dKa;   // [nchunk,B,Hkv,S,D] anchor partials, by chunk and anchor index
  float* dVa;
  const uint8_t* is_sep;
  const int32_t* sep_prefix;
  const int32_t* anchor_pos;
  const int32_t* qtile;
  int B, Hq, Hkv, S, a, n, QT;
  int nchunk, chunk_tiles;  // anchor work split: nchunk chunks of chunk_tiles query tiles
  float scale;
  float scale_log2;
};

// Split of the query tiles among anchor work items, from the shapes alone:
// aim at about 1024 (anchor tile, chunk, sequence, kv head) items, guessing
// the anchor count from a separator density of 1/8; at most 16 chunks.
static void anchor_split(int B, int Hkv, int S, int QT, int* nchunk, int* chunk_tiles) {
  const long units_guess = (4 + S / 8 + 127) / 128 + 1;
  long n = (1024 + (long)B * Hkv * units_guess - 1) / ((long)B * Hkv * units_guess);
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  if (n > QT) n = QT;
  const int ct = (int)((QT + n - 1) / n);
  *chunk_tiles = ct;
  *nchunk = (QT + ct - 1) / ct;
}

// ---------------------------------------------------------------------------
// pre: D = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdArgs p) {
  constexpr int VEC = Traits<T>::VEC;
  constexpr int TPR = D / VEC;  // threads per row
  const size_t rows = (size_t)p.B * p.Hq * p.S;
  const size_t row = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  if (row >= rows) return;
  float acc = 0.f;
  const T* orow = (const T*)p.o + row * D + sub * VEC;
  const T* grow = (const T*)p.dout + row * D + sub * VEC;
  if constexpr (VEC == 8) {
    const u32x4 a = *(const u32x4*)orow, b = *(const u32x4*)grow;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __uint_as_float(a[w] << 16) * __uint_as_float(b[w] << 16);
      acc += __uint_as_float(a[w] & 0xFFFF0000u) * __uint_as_float(b[w] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *(const f32x4*)orow, b = *(const f32x4*)grow;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += a[e] * b[e];
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (sub == 0) p.Dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// key-major dK/dV
// ---------------------------------------------------------------------------
template <typename T, int D, bool ANCHOR>
__global__ void __launch_bounds__(kBwdThreads, (bwd_occupancy<T, D>())) bwd_dkdv_kernel(BwdArgs p) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef TileRegs<T, D, kBwdThreads> Regs;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NF = D / KSTEP;    // K/V fragments per lane
  constexpr int NDB = D / 32;      // 32-row blocks of dK^T / dV^T
  constexpr int SPB = 32 / KSTEP;  // MFMA steps over one 32-query block

  __shared__ __attribute__((aligned(16))) T Qs[2][G::ELEMS];   // 64 query rows, row-major
  __shared__ __attribute__((aligned(16))) T dOs[2][G::ELEMS];
  __shared__ __attribute__((aligned(16))) float lse_s[2][kKTile];
  __shared__ __attribute__((aligned(16))) float dd_s[2][kKTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hh = lane >> 5;
  const int kc = lane & 31;

  const int bg = blockIdx.y;
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  const int grp = p.Hq / p.Hkv;
  const int32_t* qt = p.qtile + (size_t)b * p.QT * kQF;
  const int n_last = qt[(p.QT - 1) * kQF + 1];

  int unit, qi_begin, qi_end;  // key unit and query-tile range [qi_begin, qi_end)
  int chunk = 0;
  if constexpr (ANCHOR) {
    unit = blockIdx.x / p.nchunk;
    chunk = blockIdx.x - unit * p.nchunk;
    if (unit * kKeysPerWG >= n_last) return;  // no query sees these anchors; never read
    // first query tile whose anchor count exceeds this unit's first anchor
    int lo_t = 0, hi_t = p.QT - 1;
    while (lo_t < hi_t) {
      const int mid = (lo_t + hi_t) >> 1;
      if (qt[mid * kQF + 1] > unit * kKeysPerWG) hi_t = mid;
      else lo_t = mid + 1;
    }
    qi_begin = max(lo_t, chunk * p.chunk_tiles);
    qi_end = min(p.QT, (chunk + 1) * p.chunk_tiles);  // may be empty: the slot is then zero-filled
  } else {
    unit = blockIdx.x;
    const int k0 = unit * kKeysPerWG;
    const int k1 = min(k0 + kKeysPerWG - 1, p.S - 1);
    qi_begin = k0 / kQTile;
    qi_end = min(p.QT, (k1 + p.n - 1) / kQTile + 1);
  }
  const int n_q = max(0, qi_end - qi_begin);
  const int n_it = grp * n_q * 2;  // (query head, query tile, 64-row half)

  // this lane's key
  const int kidx = unit * kKeysPerWG + 32 * w + kc;  // key row (band) or anchor index (anchor)
  int krow;
  if constexpr (ANCHOR) krow = kidx < n_last ? p.anchor_pos[(size_t)b * p.S + kidx] : -1;
  else krow = kidx < p.S ? kidx : -1;
  const bool key_sep = (!ANCHOR && krow >= 0) ? (p.is_sep[(size_t)b * p.S + krow] != 0) : false;
  // band: rows that see this key through the window or because it is an anchor-type key
  const int q_hi = (krow < p.a || key_sep) ? p.S - 1 : min(p.S - 1, krow + p.n - 1);

  const T* Kg = (const T*)p.k + (((size_t)b * p.Hkv + g) * p.S) * D;
  const T* Vg = (const T*)p.v + (((size_t)b * p.Hkv + g) * p.S) * D;

  auto it_head = [&](int it) { return g * grp + it / (2 * n_q); };
  auto it_row0 = [&](int it) {
    const int r = it % (2 * n_q);
    return (qi_begin + (r >> 1)) * kQTile + (r & 1) * kKTile;
  };

  Regs rq, ro;
  float pf_lse = 0.f, pf_d = 0.f;
  auto issue = [&](int it) {
    const int h = it_head(it);
    const int r0 = it_row0(it);
    int rows[Regs::NU];
    Regs::rows(rows, RowSrc{nullptr, r0, p.S}, tid);
    rq.issue((const T*)p.q + (((size_t)b * p.Hq + h) * p.S) * D, rows, tid);
    ro.issue((const T*)p.dout + (((size_t)b * p.Hq + h) * p.S) * D, rows, tid);
    if (tid < kKTile) {
      const int r = r0 + tid;
      const size_t o = ((size_t)b * p.Hq + h) * p.S + r;
      pf_lse = r < p.S ? p.lse[o] * 1.4426950408889634f : 0.f;
      pf_d = r < p.S ? p.Dvec[o] : 0.f;
    }
  };
  if (n_it > 0) issue(0);

  frag kf[NF], vf[NF];
#pragma unroll
  for (int c = 0; c < NF; ++c) {
    if (krow >= 0) {
      kf[c] = *(const frag*)(Kg + (size_t)krow * D + c * KSTEP + EPL * hh);
      vf[c] = *(const frag*)(Vg + (size_t)krow * D + c * KSTEP + EPL * hh);
    } else {
      kf[c] = frag{};
      vf[c] = frag{};
    }
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    rq.store(Qs[buf], tid);
    ro.store(dOs[buf], tid);
    if (tid < kKTile) {
      lse_s[buf][tid] = pf_lse;
      dd_s[buf][tid] = pf_d;
    }
    __syncthreads();
    const int r0 = it_row0(it);
    const int qi = r0 / kQTile;
    if (it + 1 < n_it) issue(it + 1);

    // query-row range [ql, qh] of the rows r0 .. r0+63 that see this lane's key
    int ql, qh;
    if constexpr (ANCHOR) {
      const bool seen = krow >= 0 && kidx < qt[qi * kQF + 1];
      ql = seen ? 0 : 1;
      qh = seen ? p.S - 1 : 0;
    } else {
      const bool in_band = krow >= 0 && krow >= qt[qi * kQF + 0];
      ql = in_band ? krow : 1;
      qh = in_band ? q_hi : 0;
    }
    const T* Q = Qs[buf];
    const T* dO = dOs[buf];

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int c = 0; c < NF; ++c) {
        sacc = Tr::mfma(read_x<T, D>(Q, mb, c, lane), kf[c], sacc);
        pacc = Tr::mfma(read_x<T, D>(dO, mb, c, lane), vf[c], pacc);
      }
      // P and dS; rows are queries r0 + 32mb + acc_row(i), column is this lane's key
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int rl0 = 32 * mb + 8 * i4 + 4 * hh;
        const f32x4 l4 = *(const f32x4*)&lse_s[buf][rl0];
        const f32x4 d4 = *(const f32x4*)&dd_s[buf][rl0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          const int q = r0 + rl0 + e;
          const bool vis = q >= ql && q <= qh;
          const float pv = vis ? fast_exp2(sacc[i] * p.scale_log2 - l4[e]) : 0.f;
          sacc[i] = pv;
          pacc[i] = pv * (pacc[i] - d4[e]);
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl) {
        const frag pf = acc_frag<T>(sacc, sl);
        const frag sf = acc_frag<T>(pacc, sl);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dv[db] = Tr::mfma(read_xt<T, D>(dO, mb, sl, 32 * db, lane), pf, dv[db]);
          dk[db] = Tr::mfma(read_xt<T, D>(Q, mb, sl, 32 * db, lane), sf, dk[db]);
        }
      }
    }
  }

  // epilogue: this lane holds column kidx of dK^T / dV^T, rows d = 32db + acc_row(i)
  if constexpr (ANCHOR) {
    if (krow >= 0) {
      const size_t slot = (((size_t)chunk * p.B + b) * p.Hkv + g) * p.S + kidx;
      float* ka = p.dKa + slot * D;
      float* va = p.dVa + slot * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * db + 8 * r4 + 4 * hh;
          *(f32x4*)(ka + d0) = f32x4{dk[db][4 * r4] * p.scale, dk[db][4 * r4 + 1] * p.scale,
                                     dk[db][4 * r4 + 2] * p.scale, dk[db][4 * r4 + 3] * p.scale};
          *(f32x4*)(va + d0) = f32x4{dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
        }
    }
  } else {
    if (krow >= 0) {
      // is this key also an anchor that some query sees through the anchor path?
      const int n_init = p.a < p.S ? p.a : p.S;
      int ai = -1;
      if (krow < n_init) ai = krow;
      else if (key_sep) ai = n_init + p.sep_prefix[(size_t)b * (p.S + 1) + krow];
      const bool add = ai >= 0 && ai < n_last;
      const size_t cstride = (size_t)p.B * p.Hkv * p.S * D;  // between chunk slots
      const float* ka = p.dKa + (((size_t)b * p.Hkv + g) * p.S + (add ? ai : 0)) * D;
      const float* va = p.dVa + (((size_t)b * p.Hkv + g) * p.S + (add ? ai : 0)) * D;
      T* dkg = (T*)p.dk + (((size_t)b * p.Hkv + g) * p.S + krow) * D;
      T* dvg = (T*)p.dv + (((size_t)b * p.Hkv + g) * p.S + krow) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * db + 8 * r4 + 4 * hh;
          float kv4[4], vv4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv4[e] = dk[db][4 * r4 + e] * p.scale;
            vv4[e] = dv[db][4 * r4 + e];
          }
          if (add) {
            for (int c = 0; c < p.nchunk; ++c) {
              const f32x4 ak = *(const f32x4*)(ka + c * cstride + d0);
              const f32x4 av = *(const f32x4*)(va + c * cstride + d0);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                kv4[e] += ak[e];
                vv4[e] += av[e];
              }
            }
          }
          if constexpr (EPL == 8) {
            u32x2 pk, pv2;
            pk[0] = pack_bf16x2(kv4[0], kv4[1]);
            pk[1] = pack_bf16x2(kv4[2], kv4[3]);
            pv2[0] = pack_bf16x2(vv4[0], vv4[1]);
            pv2[1] = pack_bf16x2(vv4[2], vv4[3]);
            *(u32x2*)(dkg + d0) = pk;
            *(u32x2*)(dvg + d0) = pv2;
          } else {
            *(f32x4*)(dkg + d0) = f32x4{kv4[0], kv4[1], kv4[2], kv4[3]};
            *(f32x4*)(dvg + d0) = f32x4{vv4[0], vv4[1], vv4[2], vv4[3]};
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// query-major dQ over the forward's schedule
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(kBwdThreads, (bwd_occupancy<T, D>())) bwd_dq_kernel(BwdArgs p) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef TileRegs<T, D, kBwdThreads> Regs;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NQF = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr int SPB = 32 / KSTEP;

  __shared__ __attribute__((aligned(16))) T Ks[2][G::ELEMS];
  __shared__ __attribute__((aligned(16))) T Vs[2][G::ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hh = lane >> 5;
  const int qc = lane & 31;

  const int qi = p.QT - 1 - (int)blockIdx.y;
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / (p.Hq / p.Hkv);

  const int32_t* qt = p.qtile + ((size_t)b * p.QT + qi) * kQF;
  const int lo = qt[0], n_anchor = qt[1], kb = qt[2], ke = qt[3], q0 = qt[6];
  const int n_at = (n_anchor + kKTile - 1) / kKTile;
  const int n_tiles = n_at + ke - kb + 1;

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
    if (t < n_at) {
      r.anchor = anc;
      r.base = t * kKTile;
      r.limit = n_anchor;
    } else {
      r.anchor = nullptr;
      r.base = (kb + t - n_at) * kKTile;
      r.limit = p.S;
    }
    return r;
  };
  auto sep_flag = [&](int t) -> int {
    if (t < n_at) return 0;
    const int j = (kb + t - n_at) * kKTile + lane;
    return j < p.S ? (int)sepf[j] : 0;
  };

  Regs rk, rv;
  int rows[Regs::NU];
  Regs::rows(rows, src_of(0), tid);
  rk.issue(Kg, rows, tid);
  rv.issue(Vg, rows, tid);
  int sflag = sep_flag(0);
  if (n_tiles > 1) Regs::rows(rows, src_of(1), tid);

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
  const float Di = q_ok ? p.Dvec[((size_t)b * p.Hq + h) * p.S + iq] : 0.f;

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  const int wrow0 = q0 + 32 * w;
  const int wrow1 = min(wrow0 + 31, p.S - 1);

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    rk.store(Ks[buf], tid);
    rv.store(Vs[buf], tid);
    const uint64_t sepbits = __ballot(sflag != 0);
    __syncthreads();
    if (t + 1 < n_tiles) {
      rk.issue(Kg, rows, tid);
      rv.issue(Vg, rows, tid);
      sflag = sep_flag(t + 1);
      if (t + 2 < n_tiles) Regs::rows(rows, src_of(t + 2), tid);
    }
    const T* K = Ks[buf];
    const T* V = Vs[buf];

    const bool anchor_tile = t < n_at;
    bool full;
    uint64_t vis;
    if (anchor_tile) {
      const int nv = n_anchor - t * kKTile;
      full = nv >= kKTile;
      vis = bit_range(0, nv - 1);
    } else {
      const int c0 = (kb + t - n_at) * kKTile;
      full = c0 >= lo && c0 + kKTile - 1 <= wrow0 && wrow1 - c0 < p.n && c0 + kKTile - 1 < p.S;
      vis = band_visible(iq, c0, lo, p.S, p.a, p.n, sepbits);
    }
    vis >>= 4 * hh;
    full = full && q_ok;

    f32x16 ds[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int c = 0; c < NQF; ++c) {
        sacc = Tr::mfma(read_x<T, D>(K, k2, c, lane), qf[c], sacc);
        pacc = Tr::mfma(read_x<T, D>(V, k2, c, lane), of[c], pacc);
      }
      const uint32_t vw = q_ok ? (uint32_t)(vis >> (32 * k2)) : 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool on = full || ((vw >> (((i >> 2) << 3) + (i & 3))) & 1u);
        const float pv = on ? fast_exp2(sacc[i] * p.scale_log2 - lse2) : 0.f;
        ds[k2][i] = pv * (pacc[i] - Di);
      }
    }

    // dQ^T += K^T dS^T
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl) {
        const frag sf = acc_frag<T>(ds[k2], sl);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = Tr::mfma(read_xt<T, D>(K, k2, sl, 32 * db, lane), sf, dq[db]);
      }
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

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d) {
  const int QT = (S + kQTile - 1) / kQTile;
  int nchunk, ct;
  anchor_split(B, Hkv, S, QT, &nchunk, &ct);
  return a256((size_t)B * Hq * S * 4) + 2 * a256((size_t)nchunk * B * Hkv * S * d * 4);
}

template <typename T, int D>
static hipError_t launch_bwd_t(BwdArgs& a, hipStream_t stream, hipEvent_t* ev) {
  constexpr int TPR = D / Traits<T>::VEC;
  const size_t rows = (size_t)a.B * a.Hq * a.S;
  const int pre_blocks = (int)((rows + (256 / TPR) - 1) / (256 / TPR));
  const int units = (a.S + kKeysPerWG - 1) / kKeysPerWG;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(pre_blocks), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), dim3(units * a.nchunk, a.B * a.Hkv), dim3(kBwdThreads), 0,
                     stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false>), dim3(units, a.B * a.Hkv), dim3(kBwdThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3(a.B * a.Hq, a.QT), dim3(kBwdThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[4], stream)) != hipSuccess) return e;
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
  a.Dvec = (float*)w;
  w += a256((size_t)sh.B * sh.Hq * sh.S * 4);
  a.QT = (sh.S + kQTile - 1) / kQTile;
  anchor_split(sh.B, sh.Hkv, sh.S, a.QT, &a.nchunk, &a.chunk_tiles);
  a.dKa = (float*)w;
  w += a256((size_t)a.nchunk * sh.B * sh.Hkv * sh.S * sh.d * 4);
  a.dVa = (float*)w;
  a.is_sep = idx.is_sep;
  a.sep_prefix = idx.sep_prefix;
  a.anchor_pos = idx.anchor_pos;
  a.qtile = idx.qtile;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.a = idx.a;
  a.n = idx.n;
  a.QT = (sh.S + kQTile - 1) / kQTile;
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
