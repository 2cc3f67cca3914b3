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

template <int D, int G>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecArgs p) {
  constexpr int H2 = D / 2;
  constexpr int LPS = D / 16;             // lanes per slot in the score phase
  constexpr int SPP = kDecThreads / LPS;  // slots per pass
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NSG = kDecThreads / CPR;  // slot groups in the P V phase

  __shared__ float qs[G][D];
  __shared__ float sc[G][kDecChunk];
  __shared__ float red[NSG][G][D];

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

  // rotate the query at slot L-1
  for (int u = tid; u < G * H2; u += kDecThreads) {
    const int hg = u / H2, m = u - hg * H2;
    const uint16_t* qrow = p.q + ((size_t)b * p.Hq + g * G + hg) * D;
    const float xl = bf16_bits_to_f32(qrow[m]), xh = bf16_bits_to_f32(qrow[m + H2]);
    const float cs = p.cos[(size_t)(L - 1) * H2 + m], sn = p.sin[(size_t)(L - 1) * H2 + m];
    qs[hg][m] = xl * cs - xh * sn;
    qs[hg][m + H2] = xh * cs + xl * sn;
  }
  __syncthreads();

  const uint16_t* Kb = p.k + (((size_t)b * p.Hkv + g) * p.c) * D;
  const uint16_t* Vb = p.v + (((size_t)b * p.Hkv + g) * p.c) * D;

  // scores: LPS lanes per slot, each rotating 8 (lo, hi) pairs
  {
    const int sub = tid % LPS, sl = tid / LPS;
    for (int base = 0; base < ns; base += SPP) {
      const int j = base + sl;
      float acc[G];
#pragma unroll
      for (int hg = 0; hg < G; ++hg) acc[hg] = 0.f;
      if (j < ns) {
        const int slot = s0 + j;
        float kl[8], kh[8];
        bf16x8_to_f32(*(const u32x4*)(Kb + (size_t)slot * D + 8 * sub), kl);
        bf16x8_to_f32(*(const u32x4*)(Kb + (size_t)slot * D + H2 + 8 * sub), kh);
        const f32x4 c0 = *(const f32x4*)(p.cos + (size_t)slot * H2 + 8 * sub);
        const f32x4 c1 = *(const f32x4*)(p.cos + (size_t)slot * H2 + 8 * sub + 4);
        const f32x4 s0v = *(const f32x4*)(p.sin + (size_t)slot * H2 + 8 * sub);
        const f32x4 s1v = *(const f32x4*)(p.sin + (size_t)slot * H2 + 8 * sub + 4);
        float rl[8], rh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = e < 4 ? c0[e] : c1[e - 4];
          const float sn = e < 4 ? s0v[e] : s1v[e - 4];
          rl[e] = kl[e] * cs - kh[e] * sn;
          rh[e] = kh[e] * cs + kl[e] * sn;
        }
#pragma unroll
        for (int hg = 0; hg < G; ++hg) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) a += qs[hg][8 * sub + e] * rl[e] + qs[hg][H2 + 8 * sub + e] * rh[e];
          acc[hg] = a;
        }
      }
#pragma unroll
      for (int hg = 0; hg < G; ++hg) {
#pragma unroll
        for (int off = 1; off < LPS; off <<= 1) acc[hg] += __shfl_xor(acc[hg], off, 64);
      }
      if (sub == 0 && j < ns) {
#pragma unroll
        for (int hg = 0; hg < G; ++hg) sc[hg][j] = acc[hg] * p.scale_log2;
      }
    }
  }
  __syncthreads();

  // chunk softmax per head: one wave per head (G <= 8 heads over 4 waves)
  {
    const int lane = tid & 63, wv = tid >> 6;
    for (int hg = wv; hg < G; hg += kDecThreads / 64) {
      float mx = -INFINITY;
      for (int j = lane; j < ns; j += 64) mx = fmaxf(mx, sc[hg][j]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      float sum = 0.f;
      for (int j = lane; j < ns; j += 64) {
        const float e = fast_exp2(sc[hg][j] - mx);
        sc[hg][j] = e;
        sum += e;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
      if (lane == 0) {
        part0[hg * part_stride + D] = mx;
        part0[hg * part_stride + D + 1] = sum;
      }
    }
  }
  __syncthreads();

  // o = sum_j p_j V_j: thread (chunk cc, slot group sg)
  {
    const int cc = tid % CPR, sg = tid / CPR;
    float acc[G][8];
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hg][e] = 0.f;
    for (int j = sg; j < ns; j += NSG) {
      float vv[8];
      bf16x8_to_f32(*(const u32x4*)(Vb + (size_t)(s0 + j) * D + 8 * cc), vv);
#pragma unroll
      for (int hg = 0; hg < G; ++hg) {
        const float pj = sc[hg][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hg][e] += pj * vv[e];
      }
    }
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[sg][hg][8 * cc + e] = acc[hg][e];
  }
  __syncthreads();
  for (int u = tid; u < G * D; u += kDecThreads) {
    const int hg = u / D, dd = u - hg * D;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NSG; ++k) s += red[k][hg][dd];
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
  p.o[(size_t)bh * D + dd] = f32_to_bf16_bits(num / den);
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

}  // namespace sepattn
