// SepCache update: append one token per sequence and, when usage reaches the
// capacity c, compress the Past Window into the Separator Cache.
//
// The four blocks ("How SepLLM Reorchestrates the Language Model for Speed and
// Efficiency", beiduofen.top, "SepLLM's Architecture: Composing Efficiency"):
// Initial (first a tokens), Separator (capacity s, atlas.scime.ai "Measured
// effects reported in the paper"), Window (its w newest tokens are the Local
// Window, older ones the Past Window).  Slots [0, L) hold Initial, Separator,
// Window in that order; rows are moved bit for bit.
//
// One workgroup per sequence: the compaction plan (which slot lands where) is
// built in LDS with a block scan over the Past Window's separator flags, and
// rows move in ascending destination order, one chunk at a time (all reads of
// a chunk finish before its writes; a destination never exceeds its source, so
// a later chunk's sources are never overwritten).
#include "internal.hpp"

namespace sepattn {

constexpr int kUpdThreads = 1024;
constexpr int kMoveUnits = 8;  // 16-byte units each thread holds per move chunk

__global__ void __launch_bounds__(256) cache_init_kernel(int c, int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ tok,
                                                         int32_t* __restrict__ state) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < c; i += blockDim.x) {
    pos[(size_t)b * c + i] = -1;
    tok[(size_t)b * c + i] = -1;
  }
  if (threadIdx.x < 4) state[b * 4 + threadIdx.x] = 0;
}

struct UpdArgs {
  void* k;
  void* v;
  int32_t* pos;
  int32_t* tok;
  int32_t* state;
  const void* k_new;
  const void* v_new;
  const int32_t* tok_new;
  int Hkv, d, c, a, s, w;
  SepSet sep;
};

__global__ void __launch_bounds__(kUpdThreads) cache_update_kernel(UpdArgs p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  constexpr int kWaves = kUpdThreads / 64;

  __shared__ int src_of[kMaxCacheCapacity];
  __shared__ int wave_sum[kWaves];
  __shared__ int st_sh[4];

  int32_t* st = p.state + b * 4;
  int32_t* posb = p.pos + (size_t)b * p.c;
  int32_t* tokb = p.tok + (size_t)b * p.c;
  const size_t row_elems = (size_t)p.d;                  // bf16 elements per row
  const size_t slice = (size_t)p.c * row_elems;          // one (b, g) slab
  uint16_t* K = (uint16_t*)p.k + (size_t)b * p.Hkv * slice;
  uint16_t* V = (uint16_t*)p.v + (size_t)b * p.Hkv * slice;

  if (tid < 4) st_sh[tid] = st[tid];
  __syncthreads();
  int n_init = st_sh[0], n_sep = st_sh[1], n_win = st_sh[2];
  const int t_seen = st_sh[3];
  const int slot = n_init + n_sep + n_win;

  // ---- append ----
  {
    const int chunks = p.d / 8;  // 16-byte chunks per row
    const u32x4* kn = (const u32x4*)((const uint16_t*)p.k_new + (size_t)b * p.Hkv * p.d);
    const u32x4* vn = (const u32x4*)((const uint16_t*)p.v_new + (size_t)b * p.Hkv * p.d);
    for (int u = tid; u < 2 * p.Hkv * chunks; u += kUpdThreads) {
      const int which = u / (p.Hkv * chunks);
      const int r = u - which * p.Hkv * chunks;
      const int g = r / chunks, cc = r - g * chunks;
      uint16_t* dst = (which ? V : K) + (size_t)g * slice + (size_t)slot * row_elems + cc * 8;
      *(u32x4*)dst = (which ? vn : kn)[(size_t)g * chunks + cc];
    }
    if (tid == 0) {
      posb[slot] = t_seen;
      tokb[slot] = p.tok_new[b];
    }
  }
  if (n_init < p.a) ++n_init;
  else ++n_win;
  const int L = slot + 1;

  if (L < p.c) {
    if (tid == 0) {
      st[0] = n_init;
      st[1] = n_sep;
      st[2] = n_win;
      st[3] = t_seen + 1;
    }
    return;
  }

  // ---- compress: plan ----
  __syncthreads();  // the appended row and its token id are visible below
  const int wb = n_init + n_sep;      // first Window slot
  const int npast = n_win - p.w;      // Past Window length (> 0 since c > a + s + w)
  // separators of the Past Window, in order, via a block scan of their flags
  int n_past_sep = 0;
  int* list = src_of + n_init;  // scratch: concat(old Sp, past separators) as source slots
  for (int i = tid; i < n_sep; i += kUpdThreads) list[i] = n_init + i;
  for (int base = 0; base < npast; base += kUpdThreads) {
    const int i = base + tid;
    const int f = (i < npast && is_separator(p.sep, tokb[wb + i])) ? 1 : 0;
    int incl = f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_sum[wid] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w2 = 0; w2 < kWaves; ++w2) {
      before += (w2 < wid) ? wave_sum[w2] : 0;
      total += wave_sum[w2];
    }
    if (f) list[n_sep + n_past_sep + before + incl - 1] = wb + i;
    n_past_sep += total;
    __syncthreads();
  }
  const int ns_all = n_sep + n_past_sep;
  const int drop = ns_all > p.s ? ns_all - p.s : 0;
  const int ns_keep = ns_all - drop;
  // shift the kept separators to the front of the list (ascending, in place)
  for (int base = 0; base < ns_keep; base += kUpdThreads) {
    const int i = base + tid;
    const int v = (i < ns_keep) ? list[drop + i] : 0;
    __syncthreads();
    if (i < ns_keep) list[i] = v;
    __syncthreads();
  }
  // the w newest Window rows follow
  for (int i = tid; i < p.w; i += kUpdThreads) list[ns_keep + i] = L - p.w + i;
  const int L_new = n_init + ns_keep + p.w;
  __syncthreads();

  // ---- compress: move rows (destinations [n_init, L_new)) ----
  const int chunks = p.d / 8;
  const int per_row = 2 * p.Hkv * chunks;  // 16-byte units of one slot over all (g, K/V)
  const int rows_per_chunk = (kUpdThreads * kMoveUnits) / per_row;  // >= 1 (host checks Hkv)
  for (int d0 = n_init; d0 < L_new; d0 += rows_per_chunk) {
    const int nrows = min(rows_per_chunk, L_new - d0);
    const int units = nrows * per_row;
    u32x4 buf[kMoveUnits];
    // reads
#pragma unroll
    for (int k = 0; k < kMoveUnits; ++k) {
      const int u = tid + k * kUpdThreads;
      if (u < units) {
        const int r = u / per_row, x = u - r * per_row;
        const int which = x / (p.Hkv * chunks), y = x - which * p.Hkv * chunks;
        const int g = y / chunks, cc = y - g * chunks;
        const uint16_t* src = (which ? V : K) + (size_t)g * slice + (size_t)src_of[d0 + r] * row_elems + cc * 8;
        buf[k] = *(const u32x4*)src;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMoveUnits; ++k) {
      const int u = tid + k * kUpdThreads;
      if (u < units) {
        const int r = u / per_row, x = u - r * per_row;
        const int which = x / (p.Hkv * chunks), y = x - which * p.Hkv * chunks;
        const int g = y / chunks, cc = y - g * chunks;
        uint16_t* dst = (which ? V : K) + (size_t)g * slice + (size_t)(d0 + r) * row_elems + cc * 8;
        *(u32x4*)dst = buf[k];
      }
    }
    __syncthreads();
  }

  // ---- positions and ids (all read before any write) ----
  int pv[kMaxCacheCapacity / kUpdThreads], tv[kMaxCacheCapacity / kUpdThreads];
#pragma unroll
  for (int k = 0; k < kMaxCacheCapacity / kUpdThreads; ++k) {
    const int dst = n_init + tid + k * kUpdThreads;
    if (dst < L_new) {
      pv[k] = posb[src_of[dst]];
      tv[k] = tokb[src_of[dst]];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kMaxCacheCapacity / kUpdThreads; ++k) {
    const int dst = n_init + tid + k * kUpdThreads;
    if (dst < L_new) {
      posb[dst] = pv[k];
      tokb[dst] = tv[k];
    } else if (dst < L) {
      posb[dst] = -1;
      tokb[dst] = -1;
    }
  }
  if (tid == 0) {
    st[0] = n_init;
    st[1] = ns_keep;
    st[2] = p.w;
    st[3] = t_seen + 1;
  }
}

// ---------------------------------------------------------------------------
// Prefill -> SepCache hand-off: the cache each sequence would hold after its
// P prompt tokens were streamed through the update above, built from the
// prompt's index (separator prefix counts from position a and the anchor
// list: initial tokens, then the separators in stream order).
//
// The Initial block is the first min(a, P) tokens; the Window is a suffix
// [ws, P) of the stream; the Separator block holds the last Sp separators
// before ws, Sp = min(s, #separators in [a, ws)).  With Sp separators held,
// usage reaches c when the Window holds c - a - Sp tokens, and the compression
// keeps the w newest, so ws advances by c - a - w - Sp (>= 1 since c > a+s+w);
// once Sp = s the step is constant and the rest is one division.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prefill_plan_kernel(int B, int P, int a, int s, int w, int c,
                                                           const int32_t* __restrict__ sep_prefix,
                                                           int32_t* __restrict__ state) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int32_t* pre = sep_prefix + (size_t)b * (P + 1);
  int n_init, sp = 0, ws;
  if (P <= a) {
    n_init = P;
    ws = P;
  } else {
    n_init = a;
    ws = a;
    while (true) {
      if (sp == s) {
        const long step = (long)c - a - w - s;
        const long first = (long)ws + (c - a - s) - 1;  // the token whose append fills the cache
        if (first <= P - 1) ws += (int)(((P - 1 - first) / step + 1) * step);
        break;
      }
      const long t = (long)ws + (c - a - sp) - 1;
      if (t > P - 1) break;
      ws += c - a - sp - w;  // now <= P - w, so pre[ws] is in range
      sp = min(s, pre[ws]);
    }
  }
  int32_t* st = state + b * 4;
  st[0] = n_init;
  st[1] = sp;
  st[2] = P - ws;
  st[3] = P;
}

constexpr int kPrefillSlots = 16;  // cache slots per copy workgroup

// Rows of the planned slots copied bit for bit; pos/tok written for every slot
// (-1 past the occupied ones).
__global__ void __launch_bounds__(256) prefill_copy_kernel(sepcache cache, const uint16_t* __restrict__ kin,
                                                           const uint16_t* __restrict__ vin,
                                                           const int32_t* __restrict__ tok_in, int P,
                                                           const int32_t* __restrict__ sep_prefix,
                                                           const int32_t* __restrict__ anchor_pos) {
  const int b = blockIdx.y;
  const int k0 = blockIdx.x * kPrefillSlots;
  const int32_t* st = cache.state + b * 4;
  const int n_init = st[0], sp = st[1], n_win = st[2];
  const int L = n_init + sp + n_win;
  const int ws = P - n_win;
  const int cnt = sep_prefix[(size_t)b * (P + 1) + ws];  // separators in [a, ws)
  const int a0 = min(cache.a, P);                          // separators start here in the anchor list
  __shared__ int src_sh[kPrefillSlots];
  if (threadIdx.x < kPrefillSlots) {
    const int k = k0 + threadIdx.x;
    int src = -1;
    if (k < L) {
      if (k < n_init) src = k;
      else if (k < n_init + sp) src = anchor_pos[(size_t)b * P + a0 + (cnt - sp) + (k - n_init)];
      else src = ws + (k - n_init - sp);
    }
    src_sh[threadIdx.x] = src;
    if (k < cache.c) {
      cache.pos[(size_t)b * cache.c + k] = src;
      cache.tok[(size_t)b * cache.c + k] = src >= 0 ? tok_in[(size_t)b * P + src] : -1;
    }
  }
  __syncthreads();
  const int cpr = cache.d / 8;  // 16-byte chunks per row
  const int per_slot = cache.Hkv * cpr;
  for (int u = threadIdx.x; u < kPrefillSlots * per_slot; u += 256) {
    const int sl = u / per_slot;
    const int r = u - sl * per_slot;
    const int h = r / cpr, ch = r - h * cpr;
    const int src = src_sh[sl];
    if (src < 0) continue;
    const size_t in = (((size_t)b * cache.Hkv + h) * P + src) * cache.d + 8 * ch;
    const size_t out = (((size_t)b * cache.Hkv + h) * cache.c + (k0 + sl)) * cache.d + 8 * ch;
    *(u32x4*)((uint16_t*)cache.k + out) = *(const u32x4*)(kin + in);
    *(u32x4*)((uint16_t*)cache.v + out) = *(const u32x4*)(vin + in);
  }
}

hipError_t launch_cache_prefill(const sepcache& c, const void* k, const void* v, const int32_t* tok, int P,
                                const sepattn_index& idx, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_plan_kernel, dim3((c.B + 255) / 256), dim3(256), 0, stream, c.B, P, c.a, c.s, c.w,
                     c.c, idx.sep_prefix, c.state);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_copy_kernel, dim3((c.c + kPrefillSlots - 1) / kPrefillSlots, c.B), dim3(256), 0,
                     stream, c, (const uint16_t*)k, (const uint16_t*)v, tok, P, idx.sep_prefix, idx.anchor_pos);
  return hipGetLastError();
}

hipError_t launch_cache_init(const sepcache& c, hipStream_t stream) {
  hipLaunchKernelGGL(cache_init_kernel, dim3(c.B), dim3(256), 0, stream, c.c, c.pos, c.tok, c.state);
  return hipGetLastError();
}

hipError_t launch_cache_update(const sepcache& c, const void* k_new, const void* v_new,
                               const int32_t* tok_new, const SepSet& sep, hipStream_t stream) {
  UpdArgs a;
  a.k = c.k;
  a.v = c.v;
  a.pos = c.pos;
  a.tok = c.tok;
  a.state = c.state;
  a.k_new = k_new;
  a.v_new = v_new;
  a.tok_new = tok_new;
  a.Hkv = c.Hkv;
  a.d = c.d;
  a.c = c.c;
  a.a = c.a;
  a.s = c.s;
  a.w = c.w;
  a.sep = sep;
  hipLaunchKernelGGL(cache_update_kernel, dim3(c.B), dim3(kUpdThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sepattn
