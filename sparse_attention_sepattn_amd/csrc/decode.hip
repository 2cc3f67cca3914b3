// SepCache decode: attention of each sequence's newest token over its
// compressed cache, with rotary positions assigned by cache slot.
//
// Positional shifting (project card on sourcepulse.org, "Limitations &
// Caveats"; atlas.scime.ai, "Measured effects reported in the paper"): slot k
// of the cache has position k and the query sits at the last slot.  Keys are
// stored without rotation and rotated here on load (rotate-half form, cos/sin
// table indexed by slot).
//
// Memory-bound: every cached K/V row of a (sequence, kv head) is read once per
// step and shared by the query heads of its group.  The slots are split into
// chunks of kDecChunk; one workgroup per (chunk, kv head, sequence) writes an
// unnormalised partial (max, sum, o) and a second kernel merges the chunks.
// Every load of a chunk is issued up front, unconditionally (rows past the
// chunk are clamped to its last row and never used, so no branch splits the
// loads and no wait lands between them), query first, then K pass by pass,
// then V; the rotary angles of later passes come from one angle addition
// per pass.  Cross-lane sums and maxima stay in registers (DPP, ds_swizzle,
// v_permlane32_swap).
#include <mutex>

#include "internal.hpp"

namespace sepattn {

constexpr int kDecThreads = 256;
#ifndef SEPATTN_DEC_CHUNK
#define SEPATTN_DEC_CHUNK 128
#endif
constexpr int kDecChunk = SEPATTN_DEC_CHUNK;

struct DecArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* state;
  const uint16_t* q;
  const float* cos;
  const float* sin;
  float* ws;
  uint16_t* o;
  int Hkv, Hq, c, nsplit;
  float scale_log2;
};

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& x, float* f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = __uint_as_float(x[w] << 16);
    f[2 * w + 1] = __uint_as_float(x[w] & 0xFFFF0000u);
  }
}


// Cross-lane reductions in registers (no LDS round trip):
//   DPP quad_perm [1,0,3,2] / [2,3,0,1] exchange with lane ^ 1 / lane ^ 2;
//   DPP row_ror:4 / row_ror:8 rotate within each 16-lane row;
//   ds_swizzle in bit mode (and 0x1f, xor 0x10) exchanges with lane ^ 16;
//   v_permlane32_swap exchanges the two 32-lane halves.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;
__device__ __forceinline__ float swz_xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float swz_xor4(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
}
// sum / max of a lane and lane ^ 32 (v_permlane32_swap of (x, x) gives the
// lower half's values in both halves and the upper half's in both halves)
__device__ __forceinline__ float halves_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over each aligned group of N lanes (N = 4 or 8), in every lane
template <int N>
__device__ __forceinline__ float group_sum(float a) {
  a += dpp<kQuadXor1>(a);
  a += dpp<kQuadXor2>(a);
  if constexpr (N == 8) a += swz_xor4(a);
  return a;
}
// all-lane sum / max over the wave: after the quad steps, row_ror:4 and then
// row_ror:8 add the other three quads of the row (whichever way the rotation
// runs), then the rows and the halves
__device__ __forceinline__ float wave_sum(float a) {
  a += dpp<kQuadXor1>(a);
  a += dpp<kQuadXor2>(a);
  a += dpp<kRowRor4>(a);
  a += dpp<kRowRor8>(a);
  a += swz_xor16(a);
  return halves_sum(a);
}
__device__ __forceinline__ float wave_max(float a) {
  a = fmaxf(a, dpp<kQuadXor1>(a));
  a = fmaxf(a, dpp<kQuadXor2>(a));
  a = fmaxf(a, dpp<kRowRor4>(a));
  a = fmaxf(a, dpp<kRowRor8>(a));
  a = fmaxf(a, swz_xor16(a));
  return halves_max(a);
}

#ifndef SEPATTN_DEC_OCC
#define SEPATTN_DEC_OCC 2
#endif
template <int D, int G>
__global__ void __launch_bounds__(kDecThreads, SEPATTN_DEC_OCC) decode_kernel(DecArgs p) {
  constexpr int H2 = D / 2;
  constexpr int LPS = D / 16;             // lanes per slot in the score phase (8 rotary pairs each)
  constexpr int SPP = kDecThreads / LPS;  // slots per score pass
  constexpr int NPASS = kDecChunk / SPP;  // score passes per chunk
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NSG = kDecThreads / CPR;  // slot groups in the P V phase
  constexpr int VPT = kDecChunk / NSG;    // value rows per thread
  constexpr int SGW = kWave / CPR;        // slot groups per wave
  constexpr int NW = kDecThreads / kWave;

  __shared__ __attribute__((aligned(16))) float qs[G][D];
  __shared__ float sc[G][kDecChunk];
  __shared__ __attribute__((aligned(16))) float red[NW][G][D];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int32_t* st = p.state + b * 4;
  const int L = st[0] + st[1] + st[2];
  const int s0 = split * kDecChunk;
  const size_t part_stride = (size_t)p.nsplit * (D + 2);
  float* part0 = p.ws + ((size_t)b * p.Hq + g * G) * part_stride + (size_t)split * (D + 2);

  if (s0 >= L) {
    if (tid < G) {
      part0[tid * part_stride + D] = -INFINITY;
      part0[tid * part_stride + D + 1] = 0.f;
    }
    return;
  }
  const int ns = min(kDecChunk, L - s0);
  const uint16_t* Kb = p.k + (((size_t)b * p.Hkv + g) * p.c) * D;
  const uint16_t* Vb = p.v + (((size_t)b * p.Hkv + g) * p.c) * D;

  // Loads are issued in the order they are consumed (query and its rotary
  // row, K pass by pass, then V): a wait for one load is a wait for every
  // load issued before it, so each phase only waits for its own data.
  constexpr int QPT = (G * H2 + kDecThreads - 1) / kDecThreads;  // query pairs per thread
  uint16_t xlb[QPT], xhb[QPT];  // raw bf16: converted after every load is out
  float qc[QPT], qsn[QPT];
#pragma unroll
  for (int r = 0; r < QPT; ++r) {
    const int u = min(tid + r * kDecThreads, G * H2 - 1);  // clamped: every load unconditional
    const int hg = u / H2, m = u - hg * H2;
    const uint16_t* qrow = p.q + ((size_t)b * p.Hq + g * G + hg) * D;
    xlb[r] = qrow[m];
    xhb[r] = qrow[m + H2];
    qc[r] = p.cos[(size_t)(L - 1) * H2 + m];
    qsn[r] = p.sin[(size_t)(L - 1) * H2 + m];
  }
  __builtin_amdgcn_sched_barrier(0);  // the query's loads go out first
  // rotary angles of this lane's 8 frequencies at its first slot, and the
  // rotation by SPP slots that carries them to the next pass (angle addition)
  const int sub = tid % LPS, sl = tid / LPS;
  f32x4 cs[2], sn[2], cstep[2], sstep[2];
  {
    const int slot0 = s0 + sl < L ? s0 + sl : L - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cs[h] = *(const f32x4*)(p.cos + (size_t)slot0 * H2 + 8 * sub + 4 * h);
      sn[h] = *(const f32x4*)(p.sin + (size_t)slot0 * H2 + 8 * sub + 4 * h);
      // table row SPP exists whenever it is used (ns > SPP implies c > SPP);
      // the row index is clamped so the load is unconditional
      const int srow = min(SPP, p.c - 1);
      cstep[h] = *(const f32x4*)(p.cos + (size_t)srow * H2 + 8 * sub + 4 * h);
      sstep[h] = *(const f32x4*)(p.sin + (size_t)srow * H2 + 8 * sub + 4 * h);
    }
  }
  // rows past the chunk are clamped to its last row (loaded, never used)
  u32x4 klo[NPASS], khi[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int j = min(ps * SPP + sl, ns - 1);
    klo[ps] = *(const u32x4*)(Kb + (size_t)(s0 + j) * D + 8 * sub);
    khi[ps] = *(const u32x4*)(Kb + (size_t)(s0 + j) * D + H2 + 8 * sub);
  }
  const int cc = tid % CPR, sg = tid / CPR;
  u32x4 vr[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int j = min(sg + NSG * k, ns - 1);
    vr[k] = *(const u32x4*)(Vb + (size_t)(s0 + j) * D + 8 * cc);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is in flight before the first use

  // the query of each head of the group, rotated at slot L-1
#pragma unroll
  for (int r = 0; r < QPT; ++r) {
    // clamped like the loads: extra threads rewrite the last pair with the same value
    const int u = min(tid + r * kDecThreads, G * H2 - 1);
    const int hg = u / H2, m = u - hg * H2;
    const float xl = bf16_bits_to_f32(xlb[r]), xh = bf16_bits_to_f32(xhb[r]);
    qs[hg][m] = xl * qc[r] - xh * qsn[r];
    qs[hg][m + H2] = xh * qc[r] + xl * qsn[r];
  }
  __syncthreads();

  // ---- scores: LPS lanes per slot, each rotating 8 (lo, hi) pairs ----
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    float kl[8], kh[8];
    bf16x8_to_f32(klo[ps], kl);
    bf16x8_to_f32(khi[ps], kh);
    float rl[8], rh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c1 = cs[e >> 2][e & 3], s1 = sn[e >> 2][e & 3];
      rl[e] = kl[e] * c1 - kh[e] * s1;
      rh[e] = kh[e] * c1 + kl[e] * s1;
    }
    float acc[G];
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      const f32x4 ql0 = *(const f32x4*)&qs[hg][8 * sub], ql1 = *(const f32x4*)&qs[hg][8 * sub + 4];
      const f32x4 qh0 = *(const f32x4*)&qs[hg][H2 + 8 * sub], qh1 = *(const f32x4*)&qs[hg][H2 + 8 * sub + 4];
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a += ql0[e] * rl[e] + qh0[e] * rh[e];
        a += ql1[e] * rl[4 + e] + qh1[e] * rh[4 + e];
      }
      a = group_sum<LPS>(a);
      acc[hg] = a;
    }
    const int j = ps * SPP + sl;
    if (sub == 0 && j < ns) {
#pragma unroll
      for (int hg = 0; hg < G; ++hg) sc[hg][j] = acc[hg] * p.scale_log2;
    }
    if (ps + 1 < NPASS) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 c0 = cs[h], sv = sn[h];
        cs[h] = c0 * cstep[h] - sv * sstep[h];
        sn[h] = sv * cstep[h] + c0 * sstep[h];
      }
    }
  }
  __syncthreads();

  // ---- chunk softmax per head (waves take heads in turn) ----
  {
    const int lane = tid & 63, wv = tid >> 6;
    for (int hg = wv; hg < G; hg += NW) {
      float mx = -INFINITY;
      for (int j = lane; j < ns; j += kWave) mx = fmaxf(mx, sc[hg][j]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int j = lane; j < ns; j += kWave) {
        const float e = fast_exp2(sc[hg][j] - mx);
        sc[hg][j] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        part0[hg * part_stride + D] = mx;
        part0[hg * part_stride + D + 1] = sum;
      }
    }
  }
  __syncthreads();

  // ---- o = sum_j p_j V_j from the value rows already in registers ----
  float acc[G][8];
#pragma unroll
  for (int hg = 0; hg < G; ++hg)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hg][e] = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int j = sg + NSG * k;
    if (j < ns) {
      float vv[8];
      bf16x8_to_f32(vr[k], vv);
#pragma unroll
      for (int hg = 0; hg < G; ++hg) {
        const float pj = sc[hg][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hg][e] += pj * vv[e];
      }
    }
  }
  // slot groups of one wave (lanes cc, cc + CPR, ...) in registers, then the
  // waves through LDS
#pragma unroll
  for (int hg = 0; hg < G; ++hg)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = acc[hg][e];
      if constexpr (CPR == 8) a += dpp<kRowRor8>(a);  // lane ^ 8 (a rotation by 8 of 16 lanes)
      a += swz_xor16(a);
      a = halves_sum(a);
      acc[hg][e] = a;
    }
  const int lane = tid & 63, wv = tid >> 6;
  if (lane < CPR) {
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      *(f32x4*)&red[wv][hg][8 * cc] = f32x4{acc[hg][0], acc[hg][1], acc[hg][2], acc[hg][3]};
      *(f32x4*)&red[wv][hg][8 * cc + 4] = f32x4{acc[hg][4], acc[hg][5], acc[hg][6], acc[hg][7]};
    }
  }
  static_assert(SGW * CPR == kWave, "slot groups must tile a wave");
  __syncthreads();
  for (int u = tid; u < G * D; u += kDecThreads) {
    const int hg = u / D, dd = u - hg * D;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) s += red[k][hg][dd];
    part0[hg * part_stride + dd] = s;
  }
}

// Merge the chunk partials of every (sequence, query head): one pass with a
// running maximum, the partials of 8 chunks loaded together.
template <int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(DecArgs p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int dd = threadIdx.x;
  const int32_t* st = p.state + b * 4;
  const int L = st[0] + st[1] + st[2];
  const int used = (L + kDecChunk - 1) / kDecChunk;
  const float* part = p.ws + (size_t)bh * p.nsplit * (D + 2);
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int s0 = 0; s0 < used; s0 += 8) {
    float m8[8], l8[8], o8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool ok = s0 + k < used;
      const float* ps = part + (size_t)(s0 + k) * (D + 2);
      m8[k] = ok ? ps[D] : -INFINITY;
      l8[k] = ok ? ps[D + 1] : 0.f;
      o8[k] = ok ? ps[dd] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < 8; ++k) Mn = fmaxf(Mn, m8[k]);
    // chunks that were empty or fully underflowed carry -inf / 0 and add nothing
    const float r = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
    num *= r;
    den *= r;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = m8[k] == -INFINITY ? 0.f : fast_exp2(m8[k] - Mn);
      num += w * o8[k];
      den += w * l8[k];
    }
    M = Mn;
  }
  // an empty cache (L = 0) has no chunk: its output is zero
  p.o[(size_t)bh * D + dd] = f32_to_bf16_bits(den > 0.f ? num / den : 0.f);
}

static int n_splits(int c) { return (c - 1 + kDecChunk - 1) / kDecChunk; }

size_t decode_workspace_bytes(const sepcache& c, int Hq) {
  const size_t n = (size_t)c.B * Hq * n_splits(c.c) * (c.d + 2) * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

template <int D, int G>
static hipError_t launch_decode_t(const DecArgs& a, int B, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  if (ev && ev[0] && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(a.nsplit, a.Hkv, B), dim3(kDecThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && ev[1] && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(B * a.Hq), dim3(D), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && ev[2] && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  return hipSuccess;
}

template <int D>
static hipError_t launch_decode_d(const DecArgs& a, int B, int G, hipStream_t stream, hipEvent_t* ev) {
  switch (G) {
    case 1: return launch_decode_t<D, 1>(a, B, stream, ev);
    case 2: return launch_decode_t<D, 2>(a, B, stream, ev);
    case 4: return launch_decode_t<D, 4>(a, B, stream, ev);
    case 8: return launch_decode_t<D, 8>(a, B, stream, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const sepcache& c, const void* q, int Hq, const float* rope_cos,
                         const float* rope_sin, float scale, void* o, void* ws, hipStream_t stream,
                         hipEvent_t* ev) {
  DecArgs a;
  a.k = (const uint16_t*)c.k;
  a.v = (const uint16_t*)c.v;
  a.state = c.state;
  a.q = (const uint16_t*)q;
  a.cos = rope_cos;
  a.sin = rope_sin;
  a.ws = (float*)ws;
  a.o = (uint16_t*)o;
  a.Hkv = c.Hkv;
  a.Hq = Hq;
  a.c = c.c;
  a.nsplit = n_splits(c.c);
  a.scale_log2 = scale * 1.4426950408889634f;
  const int G = Hq / c.Hkv;
  if (c.d == 64) return launch_decode_d<64>(a, c.B, G, stream, ev);
  return launch_decode_d<128>(a, c.B, G, stream, ev);
}

// ---------------------------------------------------------------------------
// Allocation-free decode: the chunk partials go to a fixed array in device
// memory instead of a caller workspace, for callers that cannot allocate
// (code under graph capture, tight serving loops).  Every GPU the library runs
// on holds its own copy of the array until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever passed to a kernel.  Every split of
// the decode kernel writes its partial before the merge reads it, so nothing
// needs clearing between calls; calls that overlap on one GPU share the array
// and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace

static hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_decode_noalloc(const sepcache& c, const void* q, int Hq, const float* rope_cos,
                                 const float* rope_sin, float scale, void* o, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_decode(c, q, Hq, rope_cos, rope_sin, scale, o, ws, stream, nullptr);
}

}  // namespace sepattn
