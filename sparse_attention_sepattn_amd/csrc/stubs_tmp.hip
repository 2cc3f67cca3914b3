#include "internal.hpp"
namespace sepattn {
size_t bwd_workspace_bytes(int, int, int, int, int) { return 256; }
hipError_t launch_bwd(const void*, const void*, const void*, const void*, const float*, const void*, const AttnShape&, const sepattn_index&, void*, void*, void*, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_cache_init(const sepcache&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_cache_update(const sepcache&, const void*, const void*, const int32_t*, const SepSet&, hipStream_t) { return hipErrorNotSupported; }
size_t decode_workspace_bytes(const sepcache&, int) { return 256; }
hipError_t launch_decode(const sepcache&, const void*, int, const float*, const float*, float, void*, void*, hipStream_t) { return hipErrorNotSupported; }
}
