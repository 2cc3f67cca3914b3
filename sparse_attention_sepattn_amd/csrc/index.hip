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
//
// One launch, one workgroup per (query tile, sequence).  A workgroup counts
// the separators below its own tile itself (64-token blocks, one wave ballot
// each), so no workgroup waits for another: the prefix work is redundant
// across query tiles (the tokens stay in L2) but every workgroup starts at
// once.  What it writes:
//   * the schedule fields of its query tile and the class of every 128 x 64
//     tile in its row of the grid: tiles left of every row's window from the
//     block counts of the scan, tiles inside every row's window closed form,
//     the few tiles that cross the diagonal or a window's left edge row by
//     row from the block's 64-bit separator mask;
//   * flags, prefix counts and anchor-list entries of its own 128 positions;
//   * (last query tile) the totals and the -1 padding of the anchor list.
// The scan below a tile makes the whole launch O(S^2 / 8192) token reads
// (tile_class itself has S^2 / 8192 entries).  For long sequences
// (S >= SEPATTN_INDEX_TWO_PASS_S) a first launch counts the separators of
// every 128-position tile once (qtile field 7, two 16-bit counts per tile)
// and the second reads those counts instead of the tokens below its tile:
// 1/64 of the bytes, no id comparisons.
#include <stdlib.h>

#include "internal.hpp"

namespace sepattn {

#ifndef SEPATTN_INDEX_THREADS
#define SEPATTN_INDEX_THREADS 1024
#endif
constexpr int kIdxThreads = SEPATTN_INDEX_THREADS;
constexpr int kIdxWaves = kIdxThreads / kWave;
#ifndef SEPATTN_INDEX_TWO_PASS_S
#define SEPATTN_INDEX_TWO_PASS_S 16384  // sequence length from which the separator counts come from a first launch
#endif
#ifndef SEPATTN_INDEX_BATCH
#define SEPATTN_INDEX_BATCH 4
#endif
constexpr int kIdxBatch = SEPATTN_INDEX_BATCH;  // 64-token blocks per wave per pass
static_assert(kKTile == kWave, "one lane per key of a 64-key block");
static_assert(kQTile == 2 * kKTile, "a query tile spans two key blocks");

// bits [0, k) of a 64-bit mask (k clamped to [0, 64])
__device__ __forceinline__ uint64_t low_bits(int k) {
  return k <= 0 ? 0ull : (k >= 64 ? ~0ull : ((1ull << k) - 1ull));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Anchor-candidate bit of position j (separator id, or on the interval); the
// caller masks positions >= S.  `t` is the token at j (unused with an interval).
__device__ __forceinline__ bool candidate(int32_t t, int j, const SepSet& sep, int interval) {
  return interval > 0 ? j % interval == interval - 1 : is_separator(sep, t);
}

// Separators (from position a on) of the two 64-position blocks of query
// tile qi, packed into qtile field 7: low 16 bits the first block, high 16
// bits the second.  One wave per (query tile, sequence).
__global__ void __launch_bounds__(kWave)
index_counts_kernel(const int32_t* __restrict__ tok, int S, int a, SepSet sep, int interval,
                    int32_t* __restrict__ qtile) {
  const int QT = gridDim.x;
  const int qi = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int32_t* tk = tok ? tok + (size_t)b * S : nullptr;  // null with an interval
  const int j0 = qi * kQTile + lane, j1 = j0 + kKTile;
  const int32_t t0 = tk ? tk[min(j0, S - 1)] : 0, t1 = tk ? tk[min(j1, S - 1)] : 0;
  const uint64_t m0 = __ballot(j0 < S && j0 >= a && candidate(t0, j0, sep, interval));
  const uint64_t m1 = __ballot(j1 < S && j1 >= a && candidate(t1, j1, sep, interval));
  if (lane == 0) qtile[((size_t)b * QT + qi) * kQF + 7] = __popcll(m0) | (__popcll(m1) << 16);
}

// counts = 1: the block counts below the tile come from qtile field 7 (set
// by index_counts_kernel) instead of a scan of the tokens.
__global__ void __launch_bounds__(kIdxThreads)
index_kernel(int counts, const int32_t* __restrict__ tok, int S, int a, int n, SepSet sep, int interval,
             uint8_t* __restrict__ is_sep, int32_t* __restrict__ sep_prefix, int32_t* __restrict__ anchor_pos,
             int32_t* __restrict__ anchor_count, int32_t* __restrict__ qtile, uint8_t* __restrict__ tile_class) {
  const int QT = gridDim.x;
  const int qi = QT - 1 - (int)blockIdx.x;  // the longest scans first
  const int b = blockIdx.y;
  const int KT = (S + kKTile - 1) / kKTile;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int32_t* tk = tok ? tok + (size_t)b * S : nullptr;  // null with an interval
  uint8_t* cls = tile_class + ((size_t)b * QT + qi) * KT;
  const int q0 = qi * kQTile;
  const int q1 = min(q0 + kQTile - 1, S - 1);
  const int lo = max(0, q0 - n + 1);  // window start of the tile's first row
  const bool last = qi == QT - 1;
  const int n_init = min(a, S);
  // tiles [0, k_far) end before every row's window (64 kj + 63 <= q0 - n):
  // each row sees the same keys there, its initial tokens and separators
  const int k_far = q0 - n - (kKTile - 1) >= 0 ? (q0 - n - (kKTile - 1)) / kKTile + 1 : 0;

  // token loads of the later phases, issued before the scan so that their
  // latency overlaps it: this wave's first row-by-row tile, and (waves 0, 1)
  // the tile's own 128 positions.  Row-by-row tiles go to the waves from the
  // last one down, which have the least scan work on short sequences.
  const bool tok_ids = interval <= 0;
  const int wr = kIdxWaves - 1 - w;
  const int kj_first = k_far + wr;
  int32_t t_row = 0, t_s0 = 0, t_s1 = 0;
  if (tok_ids && kj_first <= q1 / kKTile) t_row = tk[min(kj_first * kKTile + lane, S - 1)];
  if (tok_ids && w < kQTile / kKTile) {
    t_s0 = tk[min(q0 + lane, S - 1)];
    t_s1 = tk[min(q0 + kKTile + lane, S - 1)];
  }

  // (1) separators at [a, q0) and [a, lo) (all of [a, S) in the last tile),
  // and the classes of the far-left tiles, block by block; the next pass's
  // tokens are loaded while this pass is counted
  const int nb = last ? KT : q0 / kKTile;
  int s_q0 = 0, s_lo = 0, s_all = 0;  // wave-uniform
  constexpr int kPass = kIdxWaves * kIdxBatch;
  int32_t tv[kIdxBatch];
  auto load_pass = [&](int base) {
#pragma unroll
    for (int e = 0; e < kIdxBatch; ++e) tv[e] = tk[min((base + e) * kKTile + lane, S - 1)];
  };
  if (counts) {
    // (1') the same sums from the per-block counts: blocks below q0 (all of
    // them in the last tile) and below lo; the block holding lo is counted
    // from its tokens (wave 0); far-left classes from the counts
    const int32_t* f7 = qtile + (size_t)b * QT * kQF + 7;
    const int kl = lo / kKTile;
    int c_q0 = 0, c_lo = 0, c_all = 0;
    for (int kj = (int)threadIdx.x; kj < nb; kj += kIdxThreads) {
      const int32_t pk = f7[(size_t)(kj >> 1) * kQF];
      const int cnt = (kj & 1) ? (pk >> 16) : (pk & 0xFFFF);
      c_all += cnt;
      c_q0 += kj * kKTile < q0 ? cnt : 0;
      c_lo += kj < kl ? cnt : 0;
      if (kj < k_far) {
        const int c0 = kj * kKTile;
        const int v = min(max(a - c0, 0), kKTile) + cnt;  // visible keys per row (full-width tile)
        cls[kj] = v == 0 ? 0 : (v == kKTile ? 2 : 1);
      }
    }
    s_q0 = wave_sum(c_q0);
    s_lo = wave_sum(c_lo);
    s_all = wave_sum(c_all);
    if (w == 0 && kl < nb) {
      const int c0 = kl * kKTile;
      const int j = c0 + lane;
      const int32_t t = tok_ids ? tk[min(j, S - 1)] : 0;
      s_lo += __popcll(__ballot(j < S && j >= a && candidate(t, j, sep, interval)) & low_bits(lo - c0));
    }
  }
  if (!counts && tok_ids && w * kIdxBatch < nb) load_pass(w * kIdxBatch);
  for (int base = w * kIdxBatch; !counts && base < nb; base += kPass) {
    bool hit[kIdxBatch];
    if (tok_ids) {
#pragma unroll
      for (int e = 0; e < kIdxBatch; ++e) hit[e] = false;
      // ids outer, so each id is read once per pass
#pragma unroll 4
      for (int i = 0; i < sep.n; ++i) {
        const int32_t id = sep.ids[i];
#pragma unroll
        for (int e = 0; e < kIdxBatch; ++e) hit[e] |= tv[e] == id;
      }
      if (base + kPass < nb) load_pass(base + kPass);
    } else {
#pragma unroll
      for (int e = 0; e < kIdxBatch; ++e) hit[e] = candidate(0, (base + e) * kKTile + lane, sep, interval);
    }
#pragma unroll
    for (int e = 0; e < kIdxBatch; ++e) {
      const int kj = base + e;
      const int c0 = kj * kKTile;
      const int j = c0 + lane;
      // separators counted from position a on
      const uint64_t m = __ballot(hit[e] && kj < nb && j < S && j >= a);
      const int cnt = __popcll(m);
      s_all += cnt;
      s_q0 += __popcll(m & low_bits(q0 - c0));
      s_lo += __popcll(m & low_bits(lo - c0));
      if (kj < k_far && lane == 0) {
        const int v = min(max(a - c0, 0), kKTile) + cnt;  // visible keys per row (full-width tile)
        cls[kj] = v == 0 ? 0 : (v == kKTile ? 2 : 1);
      }
    }
  }
  __shared__ int red[kIdxWaves][3];
  if (lane == 0) {
    red[w][0] = s_q0;
    red[w][1] = s_lo;
    red[w][2] = s_all;
  }

  // (2) classes of the tiles from k_far on: past the tile's last row 0,
  // inside every row's window and causal range 2 (closed form, all threads);
  // the rest row by row (one wave per tile)
  for (int kj = k_far + (int)threadIdx.x; kj < KT; kj += kIdxThreads) {
    const int c0 = kj * kKTile;
    const int c1 = min(c0 + kKTile - 1, S - 1);
    if (c0 > q1) cls[kj] = 0;
    else if (c0 >= q1 - n + 1 && c1 <= q0) cls[kj] = 2;
  }
  for (int kj = kj_first; kj <= q1 / kKTile; kj += kIdxWaves) {
    const int c0 = kj * kKTile;
    const int c1 = min(c0 + kKTile - 1, S - 1);
    if (c0 >= q1 - n + 1 && c1 <= q0) continue;  // written above
    const int j = c0 + lane;
    const int32_t t = !tok_ids ? 0 : (kj == kj_first ? t_row : tk[min(j, S - 1)]);
    const uint64_t keep = __ballot(j <= c1 && candidate(t, j, sep, interval)) | low_bits(a - c0);
    int total = 0;
#pragma unroll
    for (int r = 0; r < kQTile / kWave; ++r) {
      const int i = q0 + r * kWave + lane;
      if (i <= q1) {
        // keys of the tile row i sees: anchors or in its window, and j <= i
        const uint64_t vis = (keep | ~low_bits(i - n + 1 - c0)) & low_bits(min(c1, i) - c0 + 1);
        total += __popcll(vis);
      }
    }
    total = wave_sum(total);
    if (lane == 0) {
      const int full = (q1 - q0 + 1) * (c1 - c0 + 1);
      cls[kj] = total == 0 ? 0 : (total == full ? 2 : 1);
    }
  }

  __syncthreads();
  int pre_q0 = 0, pre_lo = 0, total = 0;
#pragma unroll
  for (int v = 0; v < kIdxWaves; ++v) {
    pre_q0 += red[v][0];
    pre_lo += red[v][1];
    total += red[v][2];
  }

  // (3) schedule fields of the query tile
  if (threadIdx.x == 0) {
    const int n_anchor = min(a, lo) + pre_lo;
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
  }

  // (4) flags, prefix counts and anchor entries of positions [q0, q1]: wave 0
  // the first 64, wave 1 the second (both need the first block's count)
  int32_t* pre = sep_prefix + (size_t)b * (S + 1);
  int32_t* anc = anchor_pos + (size_t)b * S;
  if (w < kQTile / kKTile && q0 + w * kKTile < S) {
    const int j0 = q0 + lane;
    const int j1 = q0 + kKTile + lane;
    const uint64_t raw0 = __ballot(j0 < S && candidate(t_s0, j0, sep, interval));
    const uint64_t raw1 = __ballot(j1 < S && candidate(t_s1, j1, sep, interval));
    const uint64_t cnt0 = raw0 & ~low_bits(a - q0);
    const uint64_t cnt1 = raw1 & ~low_bits(a - q0 - kKTile);
    if (!counts && w == 0 && lane == 0)
      qtile[((size_t)b * QT + qi) * kQF + 7] = __popcll(cnt0) | (__popcll(cnt1) << 16);
    const uint64_t raw = w ? raw1 : raw0;
    const uint64_t cm = w ? cnt1 : cnt0;
    const int j = w ? j1 : j0;
    if (j < S) {
      const int pj = pre_q0 + (w ? __popcll(cnt0) : 0) + __popcll(cm & low_bits(lane));
      is_sep[(size_t)b * S + j] = (uint8_t)((raw >> lane) & 1ull);
      pre[j] = pj;
      if (j < n_init) anc[j] = j;
      else if ((cm >> lane) & 1ull) anc[n_init + pj] = j;
    }
  }

  // (5) totals and the anchor list's padding
  if (last) {
    if (threadIdx.x == 0) {
      pre[S] = total;
      anchor_count[b] = n_init + total;
    }
    for (int j = n_init + total + (int)threadIdx.x; j < S; j += kIdxThreads) anc[j] = -1;
  }
}

hipError_t launch_build_index(const int32_t* tok, int B, int S, const SepSet& sep, int interval, int a, int n,
                              const sepattn_index& idx, hipStream_t stream) {
  const int QT = (S + kQTile - 1) / kQTile;
  // the length from which the counts come from a first launch; the
  // environment variable of the same name overrides the built-in value
  int two_pass = SEPATTN_INDEX_TWO_PASS_S;
  if (const char* e = getenv("SEPATTN_INDEX_TWO_PASS_S")) two_pass = atoi(e);
  const int counts = two_pass > 0 && S >= two_pass;
  if (counts) {
    hipLaunchKernelGGL(index_counts_kernel, dim3(QT, B), dim3(kWave), 0, stream, tok, S, a, sep, interval, idx.qtile);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(index_kernel, dim3(QT, B), dim3(kIdxThreads), 0, stream, counts, tok, S, a, n, sep, interval,
                     idx.is_sep, idx.sep_prefix, idx.anchor_pos, idx.anchor_count, idx.qtile, idx.tile_class);
  return hipGetLastError();
}

}  // namespace sepattn
