// Library-owned scratch memory for the entry points that allocate nothing.
//
// The split-KV decode launch keeps the partial states of its internal split
// (split outputs and LSEs) in device memory beyond the caller's inputs and
// outputs. attn_decode_shard takes that memory as a workspace argument;
// attn_decode_shard_noalloc uses this file-scope array instead, so a caller
// that cannot allocate (code under stream capture, a tight serving loop, a
// harness that forbids hipMalloc) can still run the launch.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends. Host code never passes the array's name to a kernel (in host
// code it names a host-side stand-in): the device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and that
// address is what the launches receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace cpa {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace cpa
