// Writing entries into a rank's round-robin local cache ("How GPUs Share a
// Long Context During LLM Inference", 3.1: the code that reads and writes
// the cache translates a slot into a GPU, slot mod C, and a row, slot / C).
//
// Entry i (a row of src) belongs to request req[i] at slot slot[i]; this rank
// (rank of C) stores it as row n_repl + slot / C of that request's local
// cache when slot mod C == rank, and skips it otherwise. Entries with a
// negative slot or request, or a row past the local cache, are skipped (the
// caller sizes the cache with cp_plan_round_robin). HBM-bound byte copy with
// 16-byte (or 4-byte) lanes.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

// Each wavefront takes 64 consecutive entries: lane l reads entry l's slot and
// request (coalesced), a ballot finds the entries this rank owns, and the
// wavefront copies each owned row with all 64 lanes.
template <typename V>
__global__ __launch_bounds__(256) void cache_write_rr_kernel(cpa::CacheWriteArgs a) {
  const int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  const int lane = threadIdx.x & 63;
  if (base >= a.n) return;
  const int64_t i = base + lane;
  int64_t row = -1;
  int32_t req = -1;
  if (i < a.n) {
    const int64_t slot = a.slot[i];
    req = a.req[i];
    if (slot >= 0 && req >= 0 && req < a.B && slot % a.C == a.rank) {
      const int64_t r = a.n_repl + slot / a.C;
      if (r < a.Lmax) row = r;
    }
  }
  uint64_t owned = __ballot(row >= 0);
  const int nv = (int)(a.row_bytes / sizeof(V));
  while (owned) {
    const int e = __builtin_ctzll(owned);
    owned &= owned - 1;
    const int64_t r = __shfl(row, e);
    const int32_t q = __shfl(req, e);
    const V* s = reinterpret_cast<const V*>(a.src + (base + e) * a.src_row);
    V* d = reinterpret_cast<V*>(a.dst + q * a.dst_b + r * a.dst_row);
    for (int k = lane; k < nv; k += 64) d[k] = __builtin_nontemporal_load(s + k);
  }
}

}  // namespace

namespace cpa {

int launch_cache_write_rr(const CacheWriteArgs& a, void* stream) {
  if (a.n == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n + 255) / 256));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  if (a.vec16)
    hipLaunchKernelGGL(cache_write_rr_kernel<u32x4>, grid, dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(cache_write_rr_kernel<unsigned>, grid, dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace cpa
