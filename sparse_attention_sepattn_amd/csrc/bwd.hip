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
//   pre   : D_i = rowsum(dO * O) and zeroing of the anchor accumulators
//   dkdv<anchor>: key-major over gathered anchor tiles (128 anchors per
//           workgroup), the query tiles that see them split into chunks; fp32
//           partials added atomically into an accumulator indexed by anchor
//   dkdv<band>  : key-major over 128-key tiles of the local band; each
//           workgroup owns its rows, adds the anchor partial of rows that are
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
constexpr int kKeysPerWG = 128;   // 4 waves x 32 keys
constexpr int kAnchorChunk = 16;  // query tiles per anchor work item

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
  float* dKa;   // [B,Hkv,S,D] by anchor index
  float* dVa;
  const uint8_t* is_sep;
  const int32_t* sep_prefix;
  const int32_t* anchor_pos;
  const int32_t* qtile;
  int B, Hq, Hkv, S, a, n, QT;
  float scale;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// pre: D = rowsum(dO * O); zero anchor accumulator rows below the last query
// tile's anchor count (the only anchors any row sees through the anchor path)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdArgs p) {
  constexpr int VEC = Traits<T>::VEC;
  constexpr int TPR = D / VEC;  // threads per row
  const size_t rows = (size_t)p.B * p.Hq * p.S;
  const size_t row = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  if (row < rows) {
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
  // zero anchor accumulators: grid-stride over (b, g, anchor row, d)
  const size_t stride = (size_t)gridDim.x * 256;
  const size_t total = (size_t)p.B * p.Hkv * p.S * D;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < total; x += stride) {
    const size_t bg = x / ((size_t)p.S * D);
    const int arow = (int)((x / D) % p.S);
    const int b = (int)(bg / p.Hkv);
    const int n_last = p.qtile[((size_t)b * p.QT + p.QT - 1) * kQF + 1];
    if (arow < n_last) {
      p.dKa[x] = 0.f;
      p.dVa[x] = 0.f;
    } else {
      // skip ahead to the first index of this thread's stride sequence that
      // lies in the next (b, g) slab (the loop adds the last stride)
      const size_t next = (bg + 1) * (size_t)p.S * D;
      const size_t k = (next - x + stride - 1) / stride;
      x += (k - 1) * stride;
    }
  }
}

// ---------------------------------------------------------------------------
// key-major dK/dV
// ---------------------------------------------------------------------------
template <typename T, int D, bool ANCHOR>
__global__ void __launch_bounds__(kBwdThreads) bwd_dkdv_kernel(BwdArgs p) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NF = D / KSTEP;   // K/V fragments per lane
  constexpr int NDB = D / 32;     // 32-row blocks of dK^T / dV^T
  constexpr int NPS = 32 / KSTEP; // MFMA steps over one 32-query block

  __shared__ __attribute__((aligned(16))) T Qs[G::K_ELEMS];   // 64 query rows, row-major
  __shared__ __attribute__((aligned(16))) T Qt[G::V_ELEMS];   // transposed
  __shared__ __attribute__((aligned(16))) T dOs[G::K_ELEMS];
  __shared__ __attribute__((aligned(16))) T dOt[G::V_ELEMS];
  __shared__ float lse_s[kKTile];
  __shared__ float dv_s[kKTile];

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

  int unit, qi_begin, qi_end;  // key unit and query-tile range [qi_begin, qi_end)
  if constexpr (ANCHOR) {
    const int nchunks = (p.QT + kAnchorChunk - 1) / kAnchorChunk;
    unit = blockIdx.x / nchunks;
    const int chunk = blockIdx.x - unit * nchunks;
    const int n_last = qt[(p.QT - 1) * kQF + 1];
    if (unit * kKeysPerWG >= n_last) return;
    // first query tile whose anchor count exceeds this unit's first anchor
    int lo_t = 0, hi_t = p.QT - 1;
    while (lo_t < hi_t) {
      const int mid = (lo_t + hi_t) >> 1;
      if (qt[mid * kQF + 1] > unit * kKeysPerWG) hi_t = mid;
      else lo_t = mid + 1;
    }
    qi_begin = max(lo_t, chunk * kAnchorChunk);
    qi_end = min(p.QT, (chunk + 1) * kAnchorChunk);
    if (qi_begin >= qi_end) return;
  } else {
    unit = blockIdx.x;
    const int k0 = unit * kKeysPerWG;
    const int k1 = min(k0 + kKeysPerWG - 1, p.S - 1);
    qi_begin = k0 / kQTile;
    qi_end = min(p.QT, (k1 + p.n - 1) / kQTile + 1);
  }

  // this lane's key
  const int kidx = unit * kKeysPerWG + 32 * w + kc;  // key row (band) or anchor index (anchor)
  int krow;
  if constexpr (ANCHOR) {
    const int n_last = qt[(p.QT - 1) * kQF + 1];
    krow = kidx < n_last ? p.anchor_pos[(size_t)b * p.S + kidx] : -1;
  } else {
    krow = kidx < p.S ? kidx : -1;
  }
  const bool key_sep = (!ANCHOR && krow >= 0) ? (p.is_sep[(size_t)b * p.S + krow] != 0) : false;

  const T* Kg = (const T*)p.k + (((size_t)b * p.Hkv + g) * p.S) * D;
  const T* Vg = (const T*)p.v + (((size_t)b * p.Hkv + g) * p.S) * D;
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

  for (int hg = 0; hg < grp; ++hg) {
    const int h = g * grp + hg;
    const T* Qg = (const T*)p.q + (((size_t)b * p.Hq + h) * p.S) * D;
    const T* dOg = (const T*)p.dout + (((size_t)b * p.Hq + h) * p.S) * D;
    const float* lse_g = p.lse + ((size_t)b * p.Hq + h) * p.S;
    const float* D_g = p.Dvec + ((size_t)b * p.Hq + h) * p.S;
    for (int qi = qi_begin; qi < qi_end; ++qi) {
      const int lo = qt[qi * kQF + 0];
      const int n_anchor = qt[qi * kQF + 1];
      if constexpr (ANCHOR) {
        if (unit * kKeysPerWG >= n_anchor) continue;  // uniform across the workgroup
      }
      for (int half = 0; half < 2; ++half) {
        const int r0 = qi * kQTile + half * kKTile;  // first query row of this 64-row chunk
        if (r0 >= p.S) break;
        __syncthreads();
        RowSrc src{nullptr, r0, p.S};
        load_k_tile<T, D, kBwdThreads>(Qs, Qg, src, tid);
        load_vt_tile<T, D, kBwdThreads>(Qt, Qg, src, tid);
        load_k_tile<T, D, kBwdThreads>(dOs, dOg, src, tid);
        load_vt_tile<T, D, kBwdThreads>(dOt, dOg, src, tid);
        if (tid < kKTile) {
          const int r = r0 + tid;
          lse_s[tid] = r < p.S ? lse_g[r] * 1.4426950408889634f : 0.f;
          dv_s[tid] = r < p.S ? D_g[r] : 0.f;
        }
        __syncthreads();

#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          f32x16 sacc = f32x16{}, pacc = f32x16{};
          const T* qrow = Qs + (32 * mb + kc) * G::KSTR + EPL * hh;
          const T* orow = dOs + (32 * mb + kc) * G::KSTR + EPL * hh;
#pragma unroll
          for (int c = 0; c < NF; ++c) {
            sacc = Tr::mfma(*(const frag*)(qrow + c * KSTEP), kf[c], sacc);
            pacc = Tr::mfma(*(const frag*)(orow + c * KSTEP), vf[c], pacc);
          }
          // P and dS; rows are queries r0 + 32mb + acc_row(i), column is this lane's key
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rl = 32 * mb + acc_row(i, hh);
            const int qrow_i = r0 + rl;
            bool vis;
            if constexpr (ANCHOR) {
              vis = krow >= 0 && kidx < n_anchor && qrow_i < p.S;
            } else {
              vis = krow >= 0 && qrow_i < p.S && krow >= lo && krow <= qrow_i &&
                    (krow < p.a || key_sep || qrow_i - krow < p.n);
            }
            const float pv = vis ? fast_exp2(sacc[i] * p.scale_log2 - lse_s[rl]) : 0.f;
            sacc[i] = pv;
            pacc[i] = pv * (pacc[i] - dv_s[rl]);
          }
          // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
          for (int s = 0; s < NPS; ++s) {
            frag pf, sf;
            if constexpr (EPL == 8) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                pf[j] = (__bf16)sacc[s * 8 + j];
                sf[j] = (__bf16)pacc[s * 8 + j];
              }
            } else {
              pf = sacc[s];
              sf = pacc[s];
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const int off = (32 * db + kc) * G::VSTR + 32 * mb + s * 2 * EPL + hh * EPL;
              dv[db] = Tr::mfma(*(const frag*)(dOt + off), pf, dv[db]);
              dk[db] = Tr::mfma(*(const frag*)(Qt + off), sf, dk[db]);
            }
          }
        }
      }
    }
  }

  // epilogue: this lane holds column kidx of dK^T / dV^T, rows d = 32db + acc_row(i)
  if constexpr (ANCHOR) {
    if (krow >= 0) {
      float* ka = p.dKa + (((size_t)b * p.Hkv + g) * p.S + kidx) * D;
      float* va = p.dVa + (((size_t)b * p.Hkv + g) * p.S + kidx) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dd = 32 * db + acc_row(i, hh);
          atomicAdd(ka + dd, dk[db][i] * p.scale);
          atomicAdd(va + dd, dv[db][i]);
        }
    }
  } else {
    if (krow >= 0) {
      // is this key also an anchor that some query sees through the anchor path?
      const int n_last = qt[(p.QT - 1) * kQF + 1];
      const int n_init = p.a < p.S ? p.a : p.S;
      int ai = -1;
      if (krow < n_init) ai = krow;
      else if (key_sep) ai = n_init + p.sep_prefix[(size_t)b * (p.S + 1) + krow];
      const bool add = ai >= 0 && ai < n_last;
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
            const f32x4 ak = *(const f32x4*)(ka + d0), av = *(const f32x4*)(va + d0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              kv4[e] += ak[e];
              vv4[e] += av[e];
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
__global__ void __launch_bounds__(kBwdThreads) bwd_dq_kernel(BwdArgs p) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NQF = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr int NPS = kKTile / KSTEP;

  __shared__ __attribute__((aligned(16))) T Ks[G::K_ELEMS];
  __shared__ __attribute__((aligned(16))) T Kt[G::V_ELEMS];
  __shared__ __attribute__((aligned(16))) T Vs[G::K_ELEMS];

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
    const bool anchor_tile = t < n_at;
    const int kt = kb + (t - n_at);
    RowSrc src;
    if (anchor_tile) {
      src.anchor = anc;
      src.base = t * kKTile;
      src.limit = n_anchor;
    } else {
      src.anchor = nullptr;
      src.base = kt * kKTile;
      src.limit = p.S;
    }
    __syncthreads();
    load_k_tile<T, D, kBwdThreads>(Ks, Kg, src, tid);
    load_vt_tile<T, D, kBwdThreads>(Kt, Kg, src, tid);
    load_k_tile<T, D, kBwdThreads>(Vs, Vg, src, tid);
    uint64_t sepbits = 0;
    if (!anchor_tile) {
      const int j = kt * kKTile + lane;
      sepbits = __ballot(j < p.S && sepf[j] != 0);
    }
    __syncthreads();

    bool full;
    if (anchor_tile) {
      full = (t + 1) * kKTile <= n_anchor;
    } else {
      const int c0 = kt * kKTile;
      full = c0 >= lo && c0 + kKTile - 1 <= wrow0 && wrow1 - c0 < p.n && c0 + kKTile - 1 < p.S;
    }

    f32x16 ds[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const T* krow = Ks + (32 * k2 + qc) * G::KSTR + EPL * hh;
      const T* vrow = Vs + (32 * k2 + qc) * G::KSTR + EPL * hh;
#pragma unroll
      for (int c = 0; c < NQF; ++c) {
        sacc = Tr::mfma(*(const frag*)(krow + c * KSTEP), qf[c], sacc);
        pacc = Tr::mfma(*(const frag*)(vrow + c * KSTEP), of[c], pacc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        bool vis = q_ok;
        if (!full) {
          const int r = 32 * k2 + acc_row(i, hh);
          if (anchor_tile) {
            vis = vis && (t * kKTile + r < n_anchor);
          } else {
            const int j = kt * kKTile + r;
            vis = vis && j < p.S && j >= lo && j <= iq &&
                  (j < p.a || ((sepbits >> r) & 1ull) || iq - j < p.n);
          }
        }
        const float pv = vis ? fast_exp2(sacc[i] * p.scale_log2 - lse2) : 0.f;
        ds[k2][i] = pv * (pacc[i] - Di);
      }
    }

    // dQ^T += K^T dS^T
#pragma unroll
    for (int s = 0; s < NPS; ++s) {
      const int k2 = s / (32 / KSTEP);
      const int sl = s % (32 / KSTEP);
      frag sf;
      if constexpr (EPL == 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sf[j] = (__bf16)ds[k2][sl * 8 + j];
      } else {
        sf = ds[k2][sl];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const frag kfr = *(const frag*)(Kt + (32 * db + qc) * G::VSTR + 32 * k2 + sl * 2 * EPL + hh * EPL);
        dq[db] = Tr::mfma(kfr, sf, dq[db]);
      }
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
  return a256((size_t)B * Hq * S * 4) + 2 * a256((size_t)B * Hkv * S * d * 4);
}

template <typename T, int D>
static hipError_t launch_bwd_t(BwdArgs& a, hipStream_t stream, hipEvent_t* ev) {
  constexpr int TPR = D / Traits<T>::VEC;
  const size_t rows = (size_t)a.B * a.Hq * a.S;
  const int pre_blocks = (int)((rows + (256 / TPR) - 1) / (256 / TPR));
  const int units = (a.S + kKeysPerWG - 1) / kKeysPerWG;
  const int nchunks = (a.QT + kAnchorChunk - 1) / kAnchorChunk;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(pre_blocks), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true>), dim3(units * nchunks, a.B * a.Hkv), dim3(kBwdThreads), 0,
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
  a.dKa = (float*)w;
  w += a256((size_t)sh.B * sh.Hkv * sh.S * sh.d * 4);
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
