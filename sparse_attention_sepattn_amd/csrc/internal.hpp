// Internal launcher declarations of libsepattn (host side of each .hip file).
#pragma once

#include "common.hpp"

namespace sepattn {

// Largest SepCache capacity c the update kernel plans in LDS.
constexpr int kMaxCacheCapacity = 8192;
// Largest kv-head count of a SepCache (one slot over all heads, K and V, must
// fit the update kernel's move chunk: 2 * Hkv * d * 2 bytes <= 1024 * 8 * 16).
constexpr int kMaxCacheHeads = 128;
// Largest number of query heads per kv head in decode.
constexpr int kMaxDecodeGroup = 8;
// grid y / z dimensions a launch may use (batch, query tiles, batch x kv heads)
constexpr int kMaxGridDim = 65535;

hipError_t launch_build_index(const int32_t* tok, int B, int S, const SepSet& sep, int interval, int a, int n,
                              const sepattn_index& idx, hipStream_t stream);

struct AttnShape {
  int B, Hq, Hkv, S, d, dtype;
  float scale;
};

hipError_t launch_fwd(const void* q, const void* k, const void* v, const AttnShape& sh,
                      const sepattn_index& idx, void* o, float* lse, hipStream_t stream);

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d);
// `ev` (nullable): kBwdLaunches + 1 events recorded before the first launch
// and after each launch, for per-kernel timing.
constexpr int kBwdLaunches = 3;
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, const AttnShape& sh, const sepattn_index& idx, void* dq,
                      void* dk, void* dv, void* ws, hipStream_t stream, hipEvent_t* ev);

hipError_t launch_cache_init(const sepcache& c, hipStream_t stream);
hipError_t launch_cache_prefill(const sepcache& c, const void* k, const void* v, const int32_t* tok, int P,
                                const sepattn_index& idx, hipStream_t stream);
hipError_t launch_cache_update(const sepcache& c, const void* k_new, const void* v_new,
                               const int32_t* tok_new, const SepSet& sep, hipStream_t stream);
size_t decode_workspace_bytes(const sepcache& c, int Hq);
// `ev` (nullable): 3 events, before the decode kernel, after it, after the merge.
hipError_t launch_decode(const sepcache& c, const void* q, int Hq, const float* rope_cos,
                         const float* rope_sin, float scale, void* o, void* ws, hipStream_t stream,
                         hipEvent_t* ev);
// Size of the library's fixed per-device scratch (the decode partials of
// sepcache_decode_noalloc).
constexpr size_t kNoAllocScratchBytes = SEPATTN_NOALLOC_SCRATCH_BYTES;
// launch_decode with the fixed scratch as its workspace (callers check the size)
hipError_t launch_decode_noalloc(const sepcache& c, const void* q, int Hq, const float* rope_cos,
                                 const float* rope_sin, float scale, void* o, hipStream_t stream);

}  // namespace sepattn
