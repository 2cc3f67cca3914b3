// Forward of SepLLM separator-sparse attention: block-sparse flash attention
// over the kept tiles of each 128-row query tile -- the key tiles
// kt_begin..kt_end of the local band (masked element-wise), then
// ceil(n_anchor/64) tiles of gathered anchors (initial tokens and separators
// below the window, visible to every row of the tile, so unmasked).  Online
// softmax in the base-2 domain, fp32 accumulation, P rounded to the input
// type for the second product.
//
// Mask: SepLLM summary on atlas.scime.ai, "Approach".  Output O = M(A, V, M_b)
// read as softmax renormalised over the kept keys ("How SepLLM Reorchestrates
// the Language Model for Speed and Efficiency", "SepLLM's Architecture").
#include <type_traits>

#include "internal.hpp"
#include "tile.hpp"

namespace sepattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const uint8_t* is_sep;
  const int32_t* anchor_pos;
  const int32_t* qtile;
  int B, Hq, Hkv, S, a, n, QT;
  float scale_log2;  // softmax scale * log2(e)
};

constexpr int kFwdThreads = 256;
// Lazy rescaling threshold (base-2 units): probabilities stay below 2^8.
constexpr float kLazy = 8.f;
#ifndef SEPATTN_FWD_SKIP
#define SEPATTN_FWD_SKIP 1  // skip 32-key halves no query of the wave sees
#endif
#ifndef SEPATTN_FWD_OCC
#define SEPATTN_FWD_OCC 4  // waves per SIMD the bf16 d=64 register budget targets (128 VGPRs, no spills)
#endif
#ifndef SEPATTN_FWD_QLDS
#define SEPATTN_FWD_QLDS 128  // smallest head size whose Q tile and O rows go through LDS (coalesced rows):
                              // at d=64 it measured no faster and its extra registers spill outside the loop
#endif
#ifndef SEPATTN_FWD_OCC128
#define SEPATTN_FWD_OCC128 2  // d=128: two workgroups fill the LDS (64 KB each)
#endif

template <typename T, int D>
__global__ void __launch_bounds__(kFwdThreads, sizeof(T) == 2 ? (D == 64 ? SEPATTN_FWD_OCC : SEPATTN_FWD_OCC128) : 1) fwd_kernel(FwdArgs p) {
  typedef Traits<T> Tr;
  typedef TileGeom<T, D> G;
  typedef TileRows<T, D, kFwdThreads> Regs;
  typedef typename Tr::frag frag;
  constexpr int EPL = Tr::EPL;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int NQF = D / KSTEP;   // Q fragments per lane
  constexpr int NDB = D / 32;      // 32-row blocks of O^T
  constexpr int SPB = 32 / KSTEP;  // MFMA steps per 32-key block
  typedef TileDMA<T, D, kFwdThreads> DMA;

  // double buffers as separate arrays, and each step names its buffer at
  // compile time: the compiler can then tell a DMA into one buffer from the
  // reads of the other and does not wait for the DMA before those reads
  __shared__ __attribute__((aligned(16))) T Ks0[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T Ks1[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T Vs0[G::ELEMS];
  __shared__ __attribute__((aligned(16))) T Vs1[G::ELEMS];
  auto kbuf = [&](auto B) -> T* {
    if constexpr (decltype(B)::value == 0) return Ks0;
    else return Ks1;
  };
  auto vbuf = [&](auto B) -> T* {
    if constexpr (decltype(B)::value == 0) return Vs0;
    else return Vs1;
  };
  constexpr std::integral_constant<int, 0> I0{};
  constexpr std::integral_constant<int, 1> I1{};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so tests on it are scalar branches
  const int hh = lane >> 5;
  const int qc = lane & 31;

  // heaviest query tiles (most anchors) are dispatched first
  const int qi = p.QT - 1 - (int)blockIdx.y;
  int b, h;
  query_column(blockIdx.x, p.B, p.Hq, p.Hkv, b, h);
  const int g = h / (p.Hq / p.Hkv);

  // Band tiles first (their rows follow from q0 and n), gathered anchor tiles
  // last, so the first loads do not wait for the index.
  const int q0 = qi * kQTile;
  const int lo = max(0, q0 - p.n + 1);
  const int kb = lo / kKTile, ke = min(q0 + kQTile - 1, p.S - 1) / kKTile;
  const int n_band = ke - kb + 1;
  const int n_anchor = p.qtile[((size_t)b * p.QT + qi) * kQF + 1];
  const int n_at = (n_anchor + kKTile - 1) / kKTile;
  const int n_tiles = n_band + n_at;

  const int iq = q0 + 32 * w + qc;  // this lane's query row
  const bool q_ok = iq < p.S;
  const T* Qg = (const T*)p.q + (((size_t)b * p.Hq + h) * p.S) * D;
  const T* Kg = (const T*)p.k + (((size_t)b * p.Hkv + g) * p.S) * D;
  const T* Vg = (const T*)p.v + (((size_t)b * p.Hkv + g) * p.S) * D;
  const unsigned kv_bytes = (unsigned)((size_t)p.S * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t Krs = buffer_rsrc(Kg, kv_bytes), Vrs = buffer_rsrc(Vg, kv_bytes);
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
  auto sep_flag = [&](int t) -> int {
    if (t >= n_band) return 0;
    const int j = (kb + t) * kKTile + lane;
    return j < p.S ? (int)sepf[j] : 0;
  };

  // Source rows of anchor tiles come from the anchor list.  Their loads are
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

  // tile t straight into LDS buffer B (its separator flags, for band tiles,
  // into sflag).  A band tile's rows are consecutive: its loads use
  // per-thread constant offsets into a buffer resource that starts at the
  // tile (scalar work per tile); an anchor tile's rows come from the list.
  unsigned uoff[Regs::NU];
#pragma unroll
  for (int u = 0; u < Regs::NU; ++u) uoff[u] = tile_unit_offset<T, D, kFwdThreads>(tid, u);
  int sflag = 0;
  auto issue = [&](int t, auto B) {
    if (t < n_band) {  // wave-uniform
      const int r0 = (kb + t) * kKTile;
      const unsigned bytes = (unsigned)((size_t)(p.S - r0) * D * sizeof(T));
      DMA::issue_rows(buffer_rsrc(Kg + (size_t)r0 * D, bytes), uoff, kbuf(B), tid);
      DMA::issue_rows(buffer_rsrc(Vg + (size_t)r0 * D, bytes), uoff, vbuf(B), tid);
    } else {
      int rows[Regs::NU];
      resolve(t, rows);
      DMA::issue(Krs, kv_bytes, rows, kbuf(B), tid);
      DMA::issue(Vrs, kv_bytes, rows, vbuf(B), tid);
    }
    sflag = sep_flag(t);
  };
  // the anchor-list entries of anchor tiles only
  auto fetch_anchor = [&](int t) {
    if (t >= n_band) fetch(t);
  };
  // prologue: tile 0 (a band tile) in flight, the anchor rows of tile 1 requested
  issue(0, I0);
  fetch_anchor(min(1, n_tiles - 1));

  frag qf[NQF];
#if SEPATTN_FWD_QLDS > 0
  if constexpr (EPL == 8 && D >= SEPATTN_FWD_QLDS) {
    // The query tile comes in through the second pair of tile buffers (free
    // until tile 1 is issued) as two 64-row tiles, with the same coalesced
    // row loads as K and V, and each wave reads its 32 rows' fragments back;
    // rows past the end read zeros.
    const int rest = p.S - q0;
    DMA::issue_rows(buffer_rsrc(Qg + (size_t)q0 * D, (unsigned)(rest * D * sizeof(T))), uoff, Ks1, tid);
    const unsigned hi = rest > kKTile ? (unsigned)((rest - kKTile) * D * sizeof(T)) : 0u;
    DMA::issue_rows(buffer_rsrc(Qg + (size_t)min(q0 + kKTile, p.S - 1) * D, hi), uoff, Vs1, tid);
    wait_vm_all();
    __syncthreads();
    const T* Qt = w < 2 ? Ks1 : Vs1;
#pragma unroll
    for (int c = 0; c < NQF; ++c) qf[c] = read_x<T, D>(Qt, w & 1, c, lane);
  } else
#endif
  {
#pragma unroll
    for (int c = 0; c < NQF; ++c) {
      if (q_ok) qf[c] = *(const frag*)(Qg + (size_t)iq * D + c * KSTEP + EPL * hh);
      else qf[c] = frag{};
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running max (base-2 domain), shared by the lane pair
  float l = 0.f;        // this lane's part of the running sum

  const int wrow0 = q0 + 32 * w;
  const int wrow1 = min(wrow0 + 31, p.S - 1);

  // tile t from buffer B = t & 1
  auto step = [&](int t, auto B) {
    constexpr int buf = decltype(B)::value;
    constexpr std::integral_constant<int, 1 - buf> NB{};
    const uint64_t sepbits = __ballot(sflag != 0);
    wait_vm_all();    // this wave's part of tile t has landed in LDS
    __syncthreads();  // tile t visible; every wave is done with tile t-1's buffer
    if (t + 1 < n_tiles) {
      issue(t + 1, NB);  // the next tile fills the other buffer
      fetch_anchor(min(t + 2, n_tiles - 1));
    }
    const T* K = kbuf(B);
    const T* V = vbuf(B);

    // visibility (partial tiles only; bit r of vis: key r of the tile is visible)
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
    for (int k2 = 0; k2 < 2; ++k2) live[k2] = full || !SEPATTN_FWD_SKIP || __any((uint32_t)(vis >> (32 * k2)) != 0u);

    // S^T = K Q^T for the live 32-key halves of the tile; each half's operands
    // are read into registers first so its MFMAs issue back to back
    // (a dead half's accumulators are never read: the max, the exponentials
    // and the second product all skip it)
    f32x16 sacc[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if (!live[k2]) continue;
      frag kk[NQF];
#pragma unroll
      for (int c = 0; c < NQF; ++c) kk[c] = read_x<T, D>(K, k2, c, lane);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int c = 0; c < NQF; ++c) acc = Tr::mfma(kk[c], qf[c], acc);
      if (!full) {  // wave-uniform
        const uint32_t vw = (uint32_t)(vis >> (32 * k2 + 4 * hh));
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = keep_or_neg_inf(acc[i], bit_mask(vw, acc_bit(i)));
      }
      sacc[k2] = acc;
    }

    // online softmax in base 2 on raw scores: p = 2^(s*c - m).  The running
    // max m only moves when a row's max grows by more than kLazy (so p stays
    // below 2^kLazy), which leaves the rescale of O out of most tiles.
    float mloc = -INFINITY;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if (!live[k2]) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[k2][i]);
    }
    mloc = pair_max(mloc) * p.scale_log2;  // scale > 0
    const bool grow = mloc > m + kLazy;
    if (__any(grow)) {  // wave-uniform
      // rows that grow rescale by 2^(m - mloc) (0 on their first visible tile,
      // m = -inf); the others keep factor 1 (also when m is still -inf)
      const float alpha = grow ? fast_exp2(m - mloc) : 1.f;
      m = grow ? mloc : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    const float m_use = m == -INFINITY ? 0.f : m;
    float ps[4] = {-0.f, -0.f, -0.f, -0.f};  // -0 + x = x exactly, so the first adds fold away
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if (!live[k2]) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(__builtin_fmaf(sacc[k2][i], p.scale_log2, -m_use));
        sacc[k2][i] = pv;
        ps[i & 3] += pv;
      }
    }
    l += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    // O^T += V^T P^T, one live 32-key half at a time with its V^T operands read first
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if (!live[k2]) continue;
      frag vv[SPB][NDB];
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl)
#pragma unroll
        for (int db = 0; db < NDB; ++db) vv[sl][db] = read_xt<T, D>(V, k2, sl, 32 * db, lane);
#pragma unroll
      for (int sl = 0; sl < SPB; ++sl) {
        const frag pf = acc_frag<T>(sacc[k2], sl);
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = Tr::mfma(vv[sl][db], pf, oacc[db]);
      }
    }
  };

  {
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, I0);
      step(t + 1, I1);
    }
    if (t < n_tiles) step(t, I0);
  }

  // normalise and store
  const float l_tot = pair_sum(l);
  const float inv = 1.f / l_tot;
#if SEPATTN_FWD_QLDS > 0
  if constexpr (EPL == 8 && D >= SEPATTN_FWD_QLDS) {
    // O goes out as whole rows: each wave puts its 32 rows into the first
    // pair of tile buffers (row-major, swizzled like every tile), then every
    // thread stores the 16-byte chunks a tile load would have brought in
    // from those rows (consecutive lanes, consecutive chunks of a row).
    __syncthreads();  // every wave is done with the last tile's buffers
    T* Ob = (T*)p.o + (((size_t)b * p.Hq + h) * p.S + q0) * D;
    const int nrows = p.S - q0;
    store_rows_via_lds<D, kFwdThreads>(Ks0, Vs0, oacc, inv, [&](int r) { return r < nrows ? Ob + (size_t)r * D : nullptr; },
                                       uoff, tid);
    if (q_ok && hh == 0) {
      // natural-log normaliser of the scaled scores
      p.lse[((size_t)b * p.Hq + h) * p.S + iq] = (m + fast_log2(l_tot)) * 0.69314718055994530942f;
    }
    return;
  }
#endif
  if (q_ok) {
    T* Og = (T*)p.o + (((size_t)b * p.Hq + h) * p.S + iq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * hh;
        if constexpr (EPL == 8) {
          u32x2 pk;
          pk[0] = pack_bf16x2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv);
          pk[1] = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
          *(u32x2*)(Og + d0) = pk;
        } else {
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = oacc[db][4 * r4 + e] * inv;
          *(f32x4*)(Og + d0) = ov;
        }
      }
    }
    if (hh == 0) {
      // natural-log normaliser of the scaled scores
      p.lse[((size_t)b * p.Hq + h) * p.S + iq] = (m + fast_log2(l_tot)) * 0.69314718055994530942f;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  dim3 grid(a.B * a.Hq, a.QT);
  hipLaunchKernelGGL((fwd_kernel<T, D>), grid, dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, const AttnShape& sh,
                      const sepattn_index& idx, void* o, float* lse, hipStream_t stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.is_sep = idx.is_sep;
  a.anchor_pos = idx.anchor_pos;
  a.qtile = idx.qtile;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.a = idx.a;
  a.n = idx.n < idx.S ? idx.n : idx.S;  // as the index builders store it
  a.QT = (sh.S + kQTile - 1) / kQTile;
  a.scale_log2 = sh.scale * 1.4426950408889634f;
  if (sh.dtype == SEPATTN_BF16) {
    if (sh.d == 64) return launch_fwd_t<__bf16, 64>(a, stream);
    return launch_fwd_t<__bf16, 128>(a, stream);
  }
  if (sh.d == 64) return launch_fwd_t<float, 64>(a, stream);
  return launch_fwd_t<float, 128>(a, stream);
}

}  // namespace sepattn
