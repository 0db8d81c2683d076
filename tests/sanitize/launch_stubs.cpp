// Stand-ins for the GPU side of libcpattn, linked with the host sources
// (plan.cpp, api.cpp) into the sanitizer test driver: the HIP runtime
// entry points the host code calls and the kernel launchers. Nothing here
// touches a GPU; a launcher only counts the call, so a test can tell a
// validated call (it reaches the launcher) from a rejected one (it does
// not).
#include <hip/hip_runtime_api.h>

#include "internal.h"

extern "C" hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;  // compute units
  return hipSuccess;
}

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP runtime"; }

namespace cpa {

int g_launches = 0;

int launch_merge(const MergeArgs&, void*) { return ++g_launches, 0; }
int launch_decode_gqa(const DecodeGqaArgs&, void*) { return ++g_launches, 0; }
int launch_decode_mla(const DecodeMlaArgs&, void*) { return ++g_launches, 0; }
int launch_prefill_gqa(const PrefillGqaArgs&, const cpa_segment*, int, void*) { return ++g_launches, 0; }
int launch_prefill_mla(const PrefillMlaArgs&, const cpa_segment*, int, void*) { return ++g_launches, 0; }
int launch_cache_write_rr(const CacheWriteArgs&, void*) { return ++g_launches, 0; }
int launch_sparse_mla(const SparseMlaArgs&, void*) { return ++g_launches, 0; }
int launch_topk_local(const TopkLocalArgs&, void*) { return ++g_launches, 0; }
int launch_topk_merge(const TopkMergeArgs&, void*) { return ++g_launches, 0; }
int gqa_head_blocks(int G) { return (G + 15) / 16; }

int noalloc_scratch(void** ptr) {
  alignas(256) static unsigned char host_stand_in[256];  // never dereferenced: only launchers would
  *ptr = host_stand_in;
  return hipSuccess;
}

}  // namespace cpa
