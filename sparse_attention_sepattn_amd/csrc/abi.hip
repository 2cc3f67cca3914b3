// extern "C" entry points of libsepattn: argument checks on the host, then
// the launches of the kernels in index.hip, fwd.hip, bwd.hip, cache.hip and
// decode.hip.  Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include "internal.hpp"

using namespace sepattn;

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int to_status(hipError_t e) { return e == hipSuccess ? SEPATTN_OK : SEPATTN_EHIP; }

// Launch failures are read with hipGetLastError after each launch; an error
// an unrelated earlier HIP call left behind on this thread is cleared first
// so it is not reported as ours.
void forget_stale_error() { (void)hipGetLastError(); }

int make_sepset(const int32_t* sep_ids, int n_sep, SepSet* out) {
  if (n_sep < 0 || n_sep > SEPATTN_MAX_SEP_IDS) return SEPATTN_EINVAL;
  if (n_sep > 0 && !sep_ids) return SEPATTN_EINVAL;
  memset(out, 0, sizeof(*out));
  out->n = n_sep;
  for (int i = 0; i < n_sep; ++i) out->ids[i] = sep_ids[i];
  return SEPATTN_OK;
}

bool index_ok(const sepattn_index* idx, int B, int S) {
  return idx && idx->B == B && idx->S == S && idx->is_sep && idx->sep_prefix && idx->anchor_pos &&
         idx->anchor_count && idx->qtile && idx->tile_class && idx->a >= 0 && idx->n >= 1;
}

int check_attn(int B, int Hq, int Hkv, int S, int d, int dtype, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Hq % Hkv != 0 || !(isfinite(scale) && scale > 0.f))
    return SEPATTN_EINVAL;
  if (dtype != SEPATTN_F32 && dtype != SEPATTN_BF16) return SEPATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return SEPATTN_EUNSUPPORTED;
  // one (sequence, head) slice is addressed through 32-bit buffer offsets;
  // query tiles and (sequence, kv head) pairs are grid dimensions (<= 65535)
  if ((long long)S * d * (dtype == SEPATTN_F32 ? 4 : 2) >= (1ll << 31)) return SEPATTN_EUNSUPPORTED;
  if (S > kMaxGridDim * kQTile || (long long)B * Hkv > kMaxGridDim) return SEPATTN_EUNSUPPORTED;
  return SEPATTN_OK;
}

int check_cache(const sepcache* c) {
  if (!c || !c->k || !c->v || !c->pos || !c->tok || !c->state) return SEPATTN_EINVAL;
  if (c->B < 1 || c->Hkv < 1) return SEPATTN_EINVAL;
  if (c->Hkv > kMaxCacheHeads || c->B > kMaxGridDim) return SEPATTN_EUNSUPPORTED;
  if (c->d != 64 && c->d != 128) return SEPATTN_EUNSUPPORTED;
  if (c->a < 0 || c->s < 0 || c->w < 1) return SEPATTN_ECAPACITY;
  if ((long long)c->c <= (long long)c->a + c->s + c->w) return SEPATTN_ECAPACITY;
  if (c->c > kMaxCacheCapacity) return SEPATTN_ECAPACITY;
  return SEPATTN_OK;
}

}  // namespace

extern "C" {

const char* sepattn_strerror(int status) {
  switch (status) {
    case SEPATTN_OK: return "ok";
    case SEPATTN_EINVAL: return "invalid argument";
    case SEPATTN_EUNSUPPORTED:
      return "unsupported shape: dtype or head dimension (d must be 64 or 128), a slice of 2^31 bytes or more, "
             "a launch grid dimension above 65535, more than 128 SepCache kv heads, or a decode group "
             "Hq/Hkv other than 1, 2, 4, 8";
    case SEPATTN_ECAPACITY:
      return "invalid SepCache capacities (need a >= 0, s >= 0, w >= 1, c > a + s + w and c <= 8192)";
    case SEPATTN_EWORKSPACE: return "workspace too small";
    case SEPATTN_EHIP: return "HIP launch failed";
    case SEPATTN_ESCRATCH:
      return "input needs more than the library's fixed 16 MiB decode scratch (use sepcache_decode with a workspace)";
    default: return "unknown status";
  }
}

size_t sepattn_index_bytes(int B, int S) {
  if (B < 1 || S < 1) return 0;
  const size_t QT = (S + kQTile - 1) / kQTile, KT = (S + kKTile - 1) / kKTile;
  size_t n = 0;
  n += align256((size_t)B * S);                      // is_sep
  n += align256((size_t)B * (S + 1) * 4);            // sep_prefix
  n += align256((size_t)B * S * 4);                  // anchor_pos
  n += align256((size_t)B * 4);                      // anchor_count
  n += align256((size_t)B * QT * kQF * 4);           // qtile
  n += align256((size_t)B * QT * KT);                // tile_class
  return n;
}

int sepattn_index_bind(void* buf, size_t bytes, int B, int S, sepattn_index* idx) {
  if (!buf || !idx || B < 1 || S < 1) return SEPATTN_EINVAL;
  if (((uintptr_t)buf & 255) != 0) return SEPATTN_EINVAL;
  if (bytes < sepattn_index_bytes(B, S)) return SEPATTN_EWORKSPACE;
  const size_t QT = (S + kQTile - 1) / kQTile, KT = (S + kKTile - 1) / kKTile;
  char* p = (char*)buf;
  idx->B = B;
  idx->S = S;
  idx->a = 0;
  idx->n = 1;
  idx->is_sep = (uint8_t*)p;
  p += align256((size_t)B * S);
  idx->sep_prefix = (int32_t*)p;
  p += align256((size_t)B * (S + 1) * 4);
  idx->anchor_pos = (int32_t*)p;
  p += align256((size_t)B * S * 4);
  idx->anchor_count = (int32_t*)p;
  p += align256((size_t)B * 4);
  idx->qtile = (int32_t*)p;
  p += align256((size_t)B * QT * kQF * 4);
  idx->tile_class = (uint8_t*)p;
  return SEPATTN_OK;
}

int sepattn_build_index(const int32_t* token_ids, int B, int S, const int32_t* sep_ids, int n_sep,
                        int a, int n, sepattn_index* idx, void* stream) {
  if (!token_ids || !idx || B < 1 || S < 1 || a < 0 || n < 1) return SEPATTN_EINVAL;
  if (B > kMaxGridDim) return SEPATTN_EUNSUPPORTED;
  if (idx->B != B || idx->S != S || !idx->is_sep || !idx->sep_prefix || !idx->anchor_pos ||
      !idx->anchor_count || !idx->qtile || !idx->tile_class)
    return SEPATTN_EINVAL;
  SepSet sep;
  int st = make_sepset(sep_ids, n_sep, &sep);
  if (st != SEPATTN_OK) return st;
  idx->a = a;
  idx->n = n = n < S ? n : S;  // any n >= S keeps every j <= i: the same mask, no overflow in n-arithmetic
  forget_stale_error();
  return to_status(launch_build_index(token_ids, B, S, sep, 0, a, n, *idx, (hipStream_t)stream));
}

int sepattn_build_index_interval(int B, int S, int interval, int a, int n, sepattn_index* idx, void* stream) {
  if (!idx || B < 1 || S < 1 || interval < 1 || a < 0 || n < 1) return SEPATTN_EINVAL;
  if (B > kMaxGridDim) return SEPATTN_EUNSUPPORTED;
  if (idx->B != B || idx->S != S || !idx->is_sep || !idx->sep_prefix || !idx->anchor_pos ||
      !idx->anchor_count || !idx->qtile || !idx->tile_class)
    return SEPATTN_EINVAL;
  SepSet none;
  memset(&none, 0, sizeof(none));
  idx->a = a;
  idx->n = n = n < S ? n : S;
  forget_stale_error();
  return to_status(launch_build_index(nullptr, B, S, none, interval, a, n, *idx, (hipStream_t)stream));
}

int sepattn_fwd(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int S, int d,
                int dtype, float scale, const sepattn_index* idx, void* o, float* lse, void* stream) {
  int st = check_attn(B, Hq, Hkv, S, d, dtype, scale);
  if (st != SEPATTN_OK) return st;
  if (!q || !k || !v || !o || !lse || !index_ok(idx, B, S)) return SEPATTN_EINVAL;
  AttnShape sh{B, Hq, Hkv, S, d, dtype, scale};
  forget_stale_error();
  return to_status(launch_fwd(q, k, v, sh, *idx, o, lse, (hipStream_t)stream));
}

size_t sepattn_bwd_workspace(int B, int Hq, int Hkv, int S, int d, int dtype) {
  if (check_attn(B, Hq, Hkv, S, d, dtype, 1.0f) != SEPATTN_OK) return 0;
  return bwd_workspace_bytes(B, Hq, Hkv, S, d);
}

static int bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, int B, int Hq, int Hkv, int S, int d, int dtype, float scale,
                      const sepattn_index* idx, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                      void* stream, hipEvent_t* ev) {
  int st = check_attn(B, Hq, Hkv, S, d, dtype, scale);
  if (st != SEPATTN_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !index_ok(idx, B, S))
    return SEPATTN_EINVAL;
  if (!ws || ((uintptr_t)ws & 255) != 0) return SEPATTN_EINVAL;
  if (ws_bytes < bwd_workspace_bytes(B, Hq, Hkv, S, d)) return SEPATTN_EWORKSPACE;
  AttnShape sh{B, Hq, Hkv, S, d, dtype, scale};
  forget_stale_error();
  return to_status(launch_bwd(q, k, v, o, lse, dout, sh, *idx, dq, dk, dv, ws, (hipStream_t)stream, ev));
}

int sepattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, int B, int Hq, int Hkv, int S, int d, int dtype, float scale,
                const sepattn_index* idx, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                void* stream) {
  return bwd_common(q, k, v, o, lse, dout, B, Hq, Hkv, S, d, dtype, scale, idx, dq, dk, dv, ws, ws_bytes,
                    stream, nullptr);
}

int sepattn_bwd_profiled(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, int B, int Hq, int Hkv, int S, int d, int dtype, float scale,
                         const sepattn_index* idx, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                         void* stream, void* const* events, int n_events) {
  if (!events || n_events < kBwdLaunches + 1) return SEPATTN_EINVAL;
  return bwd_common(q, k, v, o, lse, dout, B, Hq, Hkv, S, d, dtype, scale, idx, dq, dk, dv, ws, ws_bytes,
                    stream, (hipEvent_t*)events);
}

int sepcache_init(const sepcache* cache, void* stream) {
  int st = check_cache(cache);
  if (st != SEPATTN_OK) return st;
  forget_stale_error();
  return to_status(launch_cache_init(*cache, (hipStream_t)stream));
}

int sepcache_update(const sepcache* cache, const void* k_new, const void* v_new,
                    const int32_t* tok_new, const int32_t* sep_ids, int n_sep, void* stream) {
  int st = check_cache(cache);
  if (st != SEPATTN_OK) return st;
  if (!k_new || !v_new || !tok_new) return SEPATTN_EINVAL;
  SepSet sep;
  st = make_sepset(sep_ids, n_sep, &sep);
  if (st != SEPATTN_OK) return st;
  forget_stale_error();
  return to_status(launch_cache_update(*cache, k_new, v_new, tok_new, sep, (hipStream_t)stream));
}

int sepcache_prefill(const sepcache* cache, const void* k, const void* v, const int32_t* tok, int P,
                     const sepattn_index* idx, void* stream) {
  int st = check_cache(cache);
  if (st != SEPATTN_OK) return st;
  if (!k || !v || !tok || !idx || P < 1) return SEPATTN_EINVAL;
  if (idx->B != cache->B || idx->S != P || idx->a != cache->a || !idx->sep_prefix || !idx->anchor_pos)
    return SEPATTN_EINVAL;
  forget_stale_error();
  return to_status(launch_cache_prefill(*cache, k, v, tok, P, *idx, (hipStream_t)stream));
}

size_t sepcache_decode_workspace(const sepcache* cache, int Hq) {
  if (check_cache(cache) != SEPATTN_OK || Hq < 1 || Hq % cache->Hkv != 0) return 0;
  return decode_workspace_bytes(*cache, Hq);
}

static int decode_common(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                         const float* rope_sin, float scale, void* o, void* ws, size_t ws_bytes,
                         void* stream, hipEvent_t* ev) {
  int st = check_cache(cache);
  if (st != SEPATTN_OK) return st;
  if (!q || !rope_cos || !rope_sin || !o || Hq < 1 || Hq % cache->Hkv != 0 || !(isfinite(scale) && scale > 0.f))
    return SEPATTN_EINVAL;
  const int G = Hq / cache->Hkv;
  if (G > kMaxDecodeGroup || (G & (G - 1)) != 0) return SEPATTN_EUNSUPPORTED;
  if (!ws || ((uintptr_t)ws & 255) != 0) return SEPATTN_EINVAL;
  if (ws_bytes < decode_workspace_bytes(*cache, Hq)) return SEPATTN_EWORKSPACE;
  forget_stale_error();
  return to_status(
      launch_decode(*cache, q, Hq, rope_cos, rope_sin, scale, o, ws, (hipStream_t)stream, ev));
}

int sepcache_decode(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                    const float* rope_sin, float scale, void* o, void* ws, size_t ws_bytes,
                    void* stream) {
  return decode_common(cache, q, Hq, rope_cos, rope_sin, scale, o, ws, ws_bytes, stream, nullptr);
}

int sepcache_decode_noalloc(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                            const float* rope_sin, float scale, void* o, void* stream) {
  int st = check_cache(cache);
  if (st != SEPATTN_OK) return st;
  if (!q || !rope_cos || !rope_sin || !o || Hq < 1 || Hq % cache->Hkv != 0 || !(isfinite(scale) && scale > 0.f))
    return SEPATTN_EINVAL;
  const int G = Hq / cache->Hkv;
  if (G > kMaxDecodeGroup || (G & (G - 1)) != 0) return SEPATTN_EUNSUPPORTED;
  if (decode_workspace_bytes(*cache, Hq) > kNoAllocScratchBytes) return SEPATTN_ESCRATCH;
  forget_stale_error();
  return to_status(launch_decode_noalloc(*cache, q, Hq, rope_cos, rope_sin, scale, o, (hipStream_t)stream));
}

int sepcache_decode_profiled(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                             const float* rope_sin, float scale, void* o, void* ws, size_t ws_bytes,
                             void* stream, void* const* events, int n_events) {
  if (!events || n_events < 3) return SEPATTN_EINVAL;
  return decode_common(cache, q, Hq, rope_cos, rope_sin, scale, o, ws, ws_bytes, stream,
                       (hipEvent_t*)events);
}

int sepattn_rope_table_host(double theta, int c, int d, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out || c < 1 || d < 2 || (d & 1) || !(theta > 0.0)) return SEPATTN_EINVAL;
  const int h = d / 2;
  for (int p = 0; p < c; ++p) {
    for (int m = 0; m < h; ++m) {
      const double f = pow(theta, -2.0 * (double)m / (double)d);
      const double ang = (double)p * f;
      cos_out[(size_t)p * h + m] = (float)cos(ang);
      sin_out[(size_t)p * h + m] = (float)sin(ang);
    }
  }
  return SEPATTN_OK;
}

}  // extern "C"
