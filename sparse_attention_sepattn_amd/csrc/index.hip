// Index builder: separator flags, separator prefix counts, the anchor list
// (initial tokens then separators, a stream compaction) and the per-tile
// schedule / block-sparsity classes of the SepLLM mask.
//
// The mask (SepLLM summary on atlas.scime.ai, "Approach"): query i sees key j
// iff j <= i and (j < a or tok[j] is a separator or i - j < n).
//
// Fixed-interval anchors (the FixLLM baseline the pages compare against:
// beiduofen.top, "Performance in the Spotlight"; atlas.scime.ai, "Surprising
// findings"): with interval m > 0 the membership test is j % m == m - 1 and
// no token ids are read; everything downstream is unchanged.
#include "internal.hpp"

namespace sepattn {

#ifndef SEPATTN_SCAN_THREADS
#define SEPATTN_SCAN_THREADS 1024
#endif
constexpr int kScanThreads = SEPATTN_SCAN_THREADS;
constexpr int kScanItems = 8;  // consecutive tokens per thread per chunk

// One workgroup per sequence.  Chunks of kScanThreads * kScanItems tokens are
// scanned in order with a running carry, so the result is deterministic.
__global__ void __launch_bounds__(kScanThreads)
index_scan_kernel(const int32_t* __restrict__ tok, int S, int a, SepSet sep, int interval,
                  uint8_t* __restrict__ is_sep, int32_t* __restrict__ sep_prefix,
                  int32_t* __restrict__ anchor_pos, int32_t* __restrict__ anchor_count) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wid = t / kWave;
  constexpr int kWaves = kScanThreads / kWave;
  __shared__ int wave_sum[kWaves];
  __shared__ int carry_sh;

  const int32_t* tk = tok ? tok + (size_t)b * S : nullptr;
  uint8_t* fl = is_sep + (size_t)b * S;
  int32_t* pre = sep_prefix + (size_t)b * (S + 1);
  int32_t* anc = anchor_pos + (size_t)b * S;
  const int n_init = a < S ? a : S;

  if (t == 0) carry_sh = 0;
  __syncthreads();

  for (int base = 0; base < S; base += kScanThreads * kScanItems) {
    const int j0 = base + t * kScanItems;
    // every token load is issued before any is used (clamped rows past S are
    // read but not counted)
    int32_t tv[kScanItems];
    if (interval <= 0) {
#pragma unroll
      for (int e = 0; e < kScanItems; ++e) tv[e] = tk[min(j0 + e, S - 1)];
    }
    // membership: ids outer, tokens inner, so each id is read once per chunk
    bool hit[kScanItems];
#pragma unroll
    for (int e = 0; e < kScanItems; ++e) hit[e] = interval > 0 && (j0 + e) % interval == interval - 1;
    if (interval <= 0) {
#pragma unroll 4
      for (int i = 0; i < sep.n; ++i) {
        const int32_t id = sep.ids[i];
#pragma unroll
        for (int e = 0; e < kScanItems; ++e) hit[e] |= tv[e] == id;
      }
    }
    int f[kScanItems];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kScanItems; ++e) {
      const int j = j0 + e;
      const int s = hit[e] ? 1 : 0;
      if (j < S) fl[j] = (uint8_t)s;
      f[e] = (j < S && j >= a) ? s : 0;  // separators counted from position a on
      cnt += f[e];
    }
    // inclusive scan of cnt across the wave
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) wave_sum[wid] = incl;
    __syncthreads();
    int wave_off = 0;
    int chunk_total = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int ws = wave_sum[w];
      wave_off += (w < wid) ? ws : 0;
      chunk_total += ws;
    }
    const int carry = carry_sh;
    int run = carry + wave_off + incl - cnt;  // exclusive prefix at j0
#pragma unroll
    for (int e = 0; e < kScanItems; ++e) {
      const int j = j0 + e;
      if (j < S) {
        pre[j] = run;
        if (j < n_init) anc[j] = j;
        else if (f[e]) anc[n_init + run] = j;
      }
      run += f[e];
    }
    __syncthreads();
    if (t == 0) carry_sh = carry + chunk_total;
    __syncthreads();
  }
  const int total = carry_sh;
  if (t == 0) {
    pre[S] = total;
    anchor_count[b] = n_init + total;
  }
  // pad the anchor list with -1
  for (int j = n_init + total + t; j < S; j += kScanThreads) anc[j] = -1;
}

// Visible entries of the mask in row i over key columns [c0, c1] (c1 < S),
// split so that a caller can keep many prefix loads in flight: `cnt` gets the
// window and initial-token part, and the separator part is
// pre[*hi_ix] - pre[*lo_ix] (both 0 when it is empty).
__device__ __forceinline__ void row_count_parts(int i, int c0, int c1, int a, int n, int* cnt, int* hi_ix,
                                                int* lo_ix) {
  const int hi = c1 < i ? c1 : i;
  const int w0 = (i - n + 1) > c0 ? (i - n + 1) : c0;
  int c = hi >= w0 ? hi - w0 + 1 : 0;  // window part (empty when hi < c0)
  const int e = hi < (i - n) ? hi : (i - n);  // last key outside the window
  const int ie = e < a - 1 ? e : a - 1;
  c += ie >= c0 ? ie - c0 + 1 : 0;  // initial tokens
  const int s0 = c0 > a ? c0 : a;
  const bool seps = e >= s0;  // separators in [s0, e]
  *cnt = c;
  *hi_ix = seps ? e + 1 : 0;
  *lo_ix = seps ? s0 : 0;
}

// Grid (QT, B): per query tile, its schedule fields and the class of every
// 128 x 64 tile in its row of the grid.
__global__ void __launch_bounds__(256)
index_tiles_kernel(int S, int a, int n, const int32_t* __restrict__ sep_prefix,
                   int32_t* __restrict__ qtile, uint8_t* __restrict__ tile_class) {
  const int qi = blockIdx.x;
  const int b = blockIdx.y;
  const int QT = gridDim.x;
  const int KT = (S + kKTile - 1) / kKTile;
  const int32_t* pre = sep_prefix + (size_t)b * (S + 1);
  const int q0 = qi * kQTile;
  const int q1 = min(q0 + kQTile - 1, S - 1);
  if (threadIdx.x == 0) {
    const int lo = max(0, q0 - n + 1);
    const int n_anchor = min(a, lo) + pre[lo];
    const int kb = lo / kKTile;
    const int ke = q1 / kKTile;
    int32_t* f = qtile + ((size_t)b * QT + qi) * kQF;
    f[0] = lo;
    f[1] = n_anchor;
    f[2] = kb;
    f[3] = ke;
    f[4] = (n_anchor + kKTile - 1) / kKTile + ke - kb + 1;
    f[5] = q1 - q0 + 1;
    f[6] = q0;
    f[7] = 0;
  }
  // 8 lanes per key tile, each counting 16 of the 128 rows
  uint8_t* cls = tile_class + ((size_t)b * QT + qi) * KT;
  const int sub = threadIdx.x & 7;
  for (int base = 0; base < KT; base += blockDim.x / 8) {
    const int kj = base + threadIdx.x / 8;
    const int c0 = kj * kKTile;
    const int c1 = min(c0 + kKTile - 1, S - 1);
    int total = 0;
    if (kj < KT && c0 <= q1) {
      if (c1 <= q0 - n) {
        // left of every row's window: each row sees the same keys of the
        // tile (its initial tokens and separators), so count one row
        if (sub == 0) {
          int c, hx, lx;
          row_count_parts(q0, c0, c1, a, n, &c, &hx, &lx);
          total = (q1 - q0 + 1) * (c + pre[hx] - pre[lx]);
        }
      } else {
        // the 16 rows of this lane (rows past the tile are not counted), all
        // of their prefix loads issued before any is used
        constexpr int R = kQTile / 8;
        int c[R], hx[R], lx[R], ph[R], pl[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = q0 + sub + 8 * r;
          row_count_parts(min(i, q1), c0, c1, a, n, &c[r], &hx[r], &lx[r]);
          if (i > q1) c[r] = hx[r] = lx[r] = 0;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          ph[r] = pre[hx[r]];
          pl[r] = pre[lx[r]];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < R; ++r) total += c[r] + ph[r] - pl[r];
      }
    }
    total += __shfl_xor(total, 1, 64);
    total += __shfl_xor(total, 2, 64);
    total += __shfl_xor(total, 4, 64);
    if (kj < KT && sub == 0) {
      const int full = (q1 - q0 + 1) * (c1 - c0 + 1);
      cls[kj] = total == 0 ? 0 : (total == full ? 2 : 1);
    }
  }
}

hipError_t launch_build_index(const int32_t* tok, int B, int S, const SepSet& sep, int interval, int a, int n,
                              const sepattn_index& idx, hipStream_t stream) {
  hipLaunchKernelGGL(index_scan_kernel, dim3(B), dim3(kScanThreads), 0, stream, tok, S, a, sep, interval,
                     idx.is_sep, idx.sep_prefix, idx.anchor_pos, idx.anchor_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int QT = (S + kQTile - 1) / kQTile;
  hipLaunchKernelGGL(index_tiles_kernel, dim3(QT, B), dim3(256), 0, stream, S, a, n,
                     idx.sep_prefix, idx.qtile, idx.tile_class);
  return hipGetLastError();
}

}  // namespace sepattn
