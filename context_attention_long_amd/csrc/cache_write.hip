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
// wavefront copies their rows as (row, chunk) items spread over its lanes,
// four items per lane in flight (all loads, then all stores).
template <typename V>
__global__ __launch_bounds__(256) void cache_write_rr_kernel(cpa::CacheWriteArgs a) {
  __shared__ int own_lane[4][64];  // per wavefront: lane of the j-th owned entry
  const int wv = threadIdx.x >> 6;
  const int64_t base = ((int64_t)blockIdx.x * 4 + wv) * 64;
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
  const uint64_t owned = __ballot(row >= 0);
  const int n_own = __popcll(owned);
  if (n_own == 0) return;
  if (row >= 0)
    own_lane[wv][__builtin_amdgcn_mbcnt_hi((uint32_t)(owned >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)owned, 0u))] =
        lane;
  const int nv = (int)(a.row_bytes / sizeof(V));  // chunks per row
  const int total = n_own * nv;
  constexpr int U = 4;
  for (int t0 = 0; t0 < total; t0 += 64 * U) {
    V buf[U];
    int64_t doff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + 64 * u + lane;
      const int tt = t < total ? t : total - 1;  // past the end: repeat the last item, store nothing
      const int j = tt / nv, k = tt - j * nv;
      const int e = own_lane[wv][j];
      const int64_t r = __shfl(row, e);
      const int32_t q = __shfl(req, e);
      buf[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(a.src + (base + e) * a.src_row) + k);
      doff[u] = t < total ? q * a.dst_b + r * a.dst_row + (int64_t)k * (int64_t)sizeof(V) : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (doff[u] >= 0) *reinterpret_cast<V*>(a.dst + doff[u]) = buf[u];
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
