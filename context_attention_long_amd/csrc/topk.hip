// Exact top-k selection for sparse attention with a split index.
//
// What it computes: "DeepSeek-V4 Attention Inference Systems" notes, 5.2 --
// each rank keeps its best k entries as (score, global id) pairs, the at
// most P x k candidates are merged into the exact global top k (exact
// because the union of the local lists contains it), and the selected ids
// go to their owners; "How GPUs Share a Long Context During LLM Inference",
// 4.1 -- with the index split, a rank alone cannot tell which of its entries
// survive. Order: higher score first, equal scores (-0 = +0) by lower global
// id, NaN below every number; every rank uses the same rule, which is what
// makes the union contain the global top k.
//
// One workgroup per query row. The order is a 64-bit key per candidate:
// an order-preserving map of the score in the high word, the complement of
// the id in the low word, so larger key = better and keys are distinct.
// A most-significant-digit radix select (8 bits per pass, one LDS
// histogram per wavefront) finds the k-th key, stopping as soon as a digit
// bin holds exactly the entries still needed; then a stable compaction
// writes the selection in candidate order. Up to 16384 candidates per row
// keep their score keys in LDS (64 KB, candidate j at word j) for all
// passes; longer rows are re-read from memory (L2) on every pass.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

constexpr int kThreads = 1024;            // 16 wavefronts: the passes are latency-bound
constexpr int kWaves = kThreads / 64;
constexpr int kE = 16;                     // chunks of 1024 candidates per compaction round
constexpr int kLdsCands = kE * kThreads;   // 16384 candidates with keys in LDS

// Score key: larger = better; 0 is reserved for "no candidate" (an unused
// register slot or a list entry past its count), NaN maps to 1.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 1u;                                   // NaN: below every number
  const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);  // -0 counts as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelectLds {
  uint32_t hist[256];
  uint64_t mask[kE][kWaves];  // selection ballot per (chunk, wave)
  uint32_t off[kE][kWaves];   // output offset of each (chunk, wave)
  uint32_t lcnt[64];          // selected per source list (merge)
  int32_t cnt_in[64];         // entries of each source list (merge)
  uint32_t wsum[kWaves];
  uint32_t bcast[4];
};

// The digit search of one radix pass over the per-wave histograms: the digit
// d holding the need-th largest key, the count of entries in bins above d and
// in bin d. `phantom` visited slots with key 0 (no candidate) sit in bin 0
// and are taken out. Every thread returns the result.
__device__ __forceinline__ void pick_digit(SelectLds& sl, uint32_t need, uint32_t phantom, uint32_t& d,
                                           uint32_t& above, uint32_t& bin) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __syncthreads();
  if (w == 0) {
    uint32_t b[4], s = 0;  // lane l: bins 255-4l .. 252-4l (descending digit order)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bi = 255 - 4 * lane - i;
      b[i] = sl.hist[bi] - (bi == 0 ? phantom : 0u);
      s += b[i];
    }
    uint32_t incl = s;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    uint32_t ab = incl - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ab < need && need <= ab + b[i]) {
        sl.bcast[0] = 255u - 4u * lane - i;
        sl.bcast[1] = ab;
        sl.bcast[2] = b[i];
      }
      ab += b[i];
    }
  }
  __syncthreads();
  d = sl.bcast[0], above = sl.bcast[1], bin = sl.bcast[2];
  __syncthreads();
}

// Histogram add of one digit per lane (lanes with in = false skip): one LDS
// atomic into the workgroup's histogram. (Counting a thread's first two
// distinct digits in registers first was measured slower.)
__device__ __forceinline__ void hist_add(uint32_t* hist, bool in, uint32_t digit) {
  if (in) atomicAdd(&hist[digit], 1u);
}

__device__ __forceinline__ void clear_hist(SelectLds& sl) {
  if (threadIdx.x < 256) sl.hist[threadIdx.x] = 0;
}

// Threshold of a selection: candidate with key K = (score key << 32) | ~id is
// selected iff it exists and (K >> shift) >= prefix; shift = 64: all that
// exist; shift < 0: none.
struct Thresh {
  uint64_t prefix;
  int shift;
};

__device__ __forceinline__ bool above_hi(uint32_t sk, const Thresh& t) {
  return (sk >> (t.shift - 32)) >= (uint32_t)t.prefix;  // for 32 <= shift < 64
}

// Radix select. each(f) visits slots, every lane of a wavefront the same
// number of times: f(slot, any, sk) with any = false for a visit past the
// end, else the score key (0: no candidate; `phantom` such slots are
// visited); low(slot) gives the low key
// word (~id), asked for only when equal scores reach the threshold. A slot
// without candidate has key 0, below every candidate, so it can only sit in
// the bins of the all-zero prefix, from which pick_digit removes it.
template <typename Each, typename Low>
__device__ __forceinline__ Thresh radix_select(uint32_t total, uint32_t phantom, int k, Each&& each, Low&& low,
                                               SelectLds& sl) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  Thresh t{0, 64};
  if (total <= (uint32_t)k) return t;
  if (k <= 0) return Thresh{0, -1};
  // leading score-key bits shared by every candidate: the first digit starts
  // below them (the merge's candidates all lie in the upper tail, where the
  // top digit would put almost everything into one or two bins)
  uint32_t kand = ~0u, kor = 0u;
  each([&](int, bool any, uint32_t sk) {
    if (any && sk != 0) kand &= sk, kor |= sk;
  });
  for (int o = 32; o > 0; o >>= 1) {
    kand &= (uint32_t)__shfl_xor((int)kand, o);
    kor |= (uint32_t)__shfl_xor((int)kor, o);
  }
  if (lane == 0) sl.mask[0][w] = ((uint64_t)kand << 32) | kor;
  __syncthreads();
  kand = ~0u, kor = 0u;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) kand &= (uint32_t)(sl.mask[0][i] >> 32), kor |= (uint32_t)sl.mask[0][i];
  __syncthreads();
  const int cb = (kand ^ kor) ? __clz(kand ^ kor) : 32;  // common leading bits
  int prev = 64 - cb;                                     // key bits below the common ones
  t.prefix = (uint64_t)kand >> (32 - cb);
  uint32_t need = (uint32_t)k;
  while (prev > 0) {
    const int sh = prev > 32 ? max(prev - 8, 32) : prev - 8;
    const uint32_t dmask = (1u << (prev - sh)) - 1u;
    clear_hist(sl);
    __syncthreads();
    if (sh >= 32) {
      const int s32 = sh - 32;
      const uint64_t pre = t.prefix;
      each([&](int, bool any, uint32_t sk) {
        hist_add(sl.hist, any && ((uint64_t)sk >> (prev - 32)) == pre, (sk >> s32) & dmask);
      });
    } else {
      const uint32_t hi = (uint32_t)(t.prefix >> (32 - prev));  // the full score key
      each([&](int slot, bool any, uint32_t sk) {
        bool in = any && sk == hi && hi != 0;  // a slot without candidate has key 0
        uint64_t key = 0;
        if (in) {
          key = ((uint64_t)sk << 32) | low(slot);
          in = (key >> prev) == t.prefix;
        }
        hist_add(sl.hist, in, (uint32_t)(key >> sh) & dmask);
      });
    }
    uint32_t d, above, bin;
    pick_digit(sl, need, t.prefix == 0 ? phantom : 0u, d, above, bin);
    need -= above;
    t.prefix = (t.prefix << (prev - sh)) | d;
    t.shift = sh;
    prev = sh;
    if (bin == need) return t;  // every entry of this bin is selected
  }
  return t;
}

template <typename Low>
__device__ __forceinline__ bool is_sel(uint32_t sk, int slot, const Thresh& t, Low&& low) {
  if (sk == 0 || t.shift < 0) return false;
  if (t.shift >= 64) return true;
  if (t.shift >= 32) return above_hi(sk, t);
  const uint64_t key = ((uint64_t)sk << 32) | low(slot);
  return (key >> t.shift) >= t.prefix;
}

// Stable compaction in candidate order (chunk e holds candidates 256 e +
// thread, e < nchunk <= kE): sel(e) says whether this thread's candidate of
// chunk e is selected; emit(e, pos) writes it at output position pos.
// Returns the number selected.
template <typename Sel, typename Emit>
__device__ __forceinline__ uint32_t compact(int nchunk, Sel&& sel, Emit&& emit, SelectLds& sl) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  auto chunks = [&](auto&& f) {
#pragma unroll 4
    for (int e = 0; e < nchunk; ++e) f(e);
  };
  chunks([&](int e) {
    const uint64_t m = __ballot(sel(e));
    if (lane == 0) sl.mask[e][w] = m;
  });
  __syncthreads();
  // exclusive offsets of the (chunk, wave) cells in candidate order, by
  // wave 0: lane l scans cells 4l .. 4l+3 (kE x kWaves = 256 cells)
  static_assert(kE * kWaves == 256, "one wavefront scans the cells");
  if (w == 0) {
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cell = 4 * lane + i;
      c[i] = cell / kWaves < nchunk ? (uint32_t)__popcll(sl.mask[cell / kWaves][cell % kWaves]) : 0u;
      sum += c[i];
    }
    uint32_t incl = sum;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    uint32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cell = 4 * lane + i;
      sl.off[cell / kWaves][cell % kWaves] = run;
      run += c[i];
    }
    if (lane == 63) sl.wsum[0] = incl;
  }
  __syncthreads();
  chunks([&](int e) {
    const uint64_t m = sl.mask[e][w];
    if ((m >> lane) & 1ull) emit(e, sl.off[e][w] + (uint32_t)__popcll(m & ((1ull << lane) - 1ull)));
  });
  const uint32_t total = sl.wsum[0];
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------- local

// kLds: the row's score keys fit LDS (L <= 16384); otherwise they are
// re-read from memory every pass.
template <bool kLds>
__global__ __launch_bounds__(kThreads) void topk_local_kernel(cpa::TopkLocalArgs a) {
  __shared__ SelectLds sl;
  __shared__ uint32_t skl[kLds ? kLdsCands : 1];  // the row's score bits
  const int n = blockIdx.x, tid = threadIdx.x;
  int nv = a.n_valid ? a.n_valid[n] : a.L;
  nv = nv < 0 ? 0 : (nv > a.L ? a.L : nv);
  const float* sc = a.scores + (int64_t)n * a.s_n;
  auto id_of = [&](int j) { return (int32_t)(a.id_base + (int64_t)j * a.id_stride); };
  auto low = [&](int j) { return (uint64_t)(~(uint32_t)id_of(j)); };
  if constexpr (kLds) {
    // batches of 16 loads in flight, keys into LDS
    for (int j0 = 0; j0 < nv; j0 += 16 * kThreads) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = sc[min(j0 + tid + kThreads * u, nv - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + tid + kThreads * u;
        if (j < nv) skl[j] = __float_as_uint(v[u]);
      }
    }
  }
  auto score_at = [&](int j) {
    if constexpr (kLds) return __uint_as_float(skl[j]);
    else return sc[j];
  };
  auto key_at = [&](int j) { return score_key(score_at(j)); };
  // every lane runs the same trip count; the keys of four chunks are read
  // together (unconditionally, clamped) so their LDS latencies overlap
  auto each = [&](auto&& f) {
    for (int j0 = 0; j0 < nv; j0 += 4 * kThreads) {
      uint32_t kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kk[u] = key_at(min(j0 + tid + u * kThreads, nv - 1));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + tid + u * kThreads;
        f(j, j < nv, kk[u]);
      }
    }
  };
  __syncthreads();
  const Thresh t = radix_select((uint32_t)nv, 0u, a.k, each, low, sl);

  float* os = a.out_score + (int64_t)n * a.k;
  int32_t* oi = a.out_id + (int64_t)n * a.k;
  int32_t* orow = a.out_row + (int64_t)n * a.k;
  uint32_t run = 0;
  const int nchunk = (nv + kThreads - 1) / kThreads;
  for (int c0 = 0; c0 < nchunk; c0 += kE) {
    const int nc = min(kE, nchunk - c0);
    const uint32_t base = run;
    run += compact(
        nc,
        [&](int e) {
          const int j = tid + kThreads * (c0 + e);
          const int jc = min(j, nv - 1);  // clamped: the key read and id stay in range
          return (j < nv) & is_sel(key_at(jc), jc, t, low);
        },
        [&](int e, uint32_t pos) {
          const int j = tid + kThreads * (c0 + e);
          pos += base;
          if (pos < (uint32_t)a.k) {
            os[pos] = score_at(j);
            oi[pos] = id_of(j);
            orow[pos] = j;
          }
        },
        sl);
  }
  const int c = run < (uint32_t)a.k ? (int)run : a.k;
  for (int p = c + tid; p < a.k; p += kThreads) {
    os[p] = -INFINITY;
    oi[p] = -1;
    orow[p] = -1;
  }
  if (tid == 0) a.out_count[n] = c;
}

// ---------------------------------------------------------------- merge

template <bool kLds>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(cpa::TopkMergeArgs a) {
  __shared__ SelectLds sl;
  __shared__ uint32_t skl[kLds ? kLdsCands : 1];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int M = a.P * a.k_in;
  const int64_t plane = (int64_t)a.N * a.k_in;  // one rank's [N, k_in] block
  if (tid < 64) {
    int c = 0;
    if (tid < a.P) {
      c = a.cand_count ? a.cand_count[(int64_t)tid * a.N + n] : a.k_in;
      c = c < 0 ? 0 : (c > a.k_in ? a.k_in : c);
    }
    sl.cnt_in[tid] = c;
    sl.lcnt[tid] = 0;
    uint32_t t = (uint32_t)c;  // total over the lists (wave 0)
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
    if (tid == 0) sl.wsum[0] = t;
  }
  __syncthreads();
  const uint32_t total = sl.wsum[0];
  // candidate j is entry s = j mod k_in of list p = j / k_in. With the keys
  // in LDS (j < 2^24) the quotient comes from a float reciprocal and one
  // correction step (an integer division costs dozens of instructions).
  const float rk = a.k_in > 0 ? 1.0f / (float)a.k_in : 0.f;
  auto list_of = [&](int j) {
    if constexpr (kLds) {
      int q = (int)((float)j * rk);
      const int r = j - q * a.k_in;
      q += r < 0 ? -1 : (r >= a.k_in ? 1 : 0);
      return q;
    } else {
      return j / a.k_in;
    }
  };
  auto elem = [&](int j) { const int p = list_of(j); return p * plane + (int64_t)n * a.k_in + (j - p * a.k_in); };
  auto exists = [&](int j) { const int p = list_of(j); return j - p * a.k_in < sl.cnt_in[p]; };
  auto low = [&](int j) { return (uint64_t)(~(uint32_t)a.cand_id[elem(j)]); };
  if constexpr (kLds) {
    for (int j0 = 0; j0 < M; j0 += 16 * kThreads) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = a.cand_score[elem(min(j0 + tid + kThreads * u, M - 1))];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + tid + kThreads * u;
        if (j < M) skl[j] = exists(j) ? score_key(v[u]) : 0u;
      }
    }
  }
  auto key_at = [&](int j) {
    if constexpr (kLds) return skl[j];
    else return exists(j) ? score_key(a.cand_score[elem(j)]) : 0u;
  };
  auto each = [&](auto&& f) {
    for (int j0 = 0; j0 < M; j0 += 4 * kThreads) {
      uint32_t kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kk[u] = key_at(min(j0 + tid + u * kThreads, M - 1));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + tid + u * kThreads;
        f(j, j < M, kk[u]);
      }
    }
  };
  __syncthreads();
  const Thresh t = radix_select(total, (uint32_t)M - total, a.k, each, low, sl);

  auto sel_of = [&](int j) {
    const int jc = min(j, M - 1);  // clamped: the key read and id stay in range
    return (j < M) & is_sel(key_at(jc), jc, t, low);
  };
  // per-list counts: the owners' offsets in the rank-major output. A
  // wavefront's 64 consecutive candidates span at most two lists when
  // k_in >= 64: two ballots and two atomics instead of one per candidate.
  const int lane = tid & 63;
#pragma unroll 4
  for (int j0 = 0; j0 < M; j0 += kThreads) {
    const int j = j0 + tid;
    const bool sl_j = sel_of(j);
    if (a.k_in >= 64) {
      const int jw = j0 + (tid & ~63);  // the wavefront's first candidate
      const int plo = list_of(jw);
      const bool lo = list_of(j) == plo;
      const uint32_t clo = (uint32_t)__popcll(__ballot(sl_j && lo));
      const uint32_t chi = (uint32_t)__popcll(__ballot(sl_j && !lo));
      if (lane == 0 && clo) atomicAdd(&sl.lcnt[plo], clo);
      if (lane == 0 && chi) atomicAdd(&sl.lcnt[plo + 1], chi);
    } else if (sl_j) {
      atomicAdd(&sl.lcnt[list_of(j)], 1u);
    }
  }
  __syncthreads();
  int32_t* oid = a.out_id + (int64_t)n * a.k;
  uint32_t run = 0;
  const int nchunk = (M + kThreads - 1) / kThreads;
  for (int c0 = 0; c0 < nchunk; c0 += kE) {
    const int nc = min(kE, nchunk - c0);
    const uint32_t base0 = run;
    run += compact(
        nc, [&](int e) { return sel_of(tid + kThreads * (c0 + e)); },
        [&](int e, uint32_t pos) {
          const int j = tid + kThreads * (c0 + e);
          pos += base0;
          if (pos < (uint32_t)a.k) {
            const int p = list_of(j);
            uint32_t base = 0;
            for (int q = 0; q < p; ++q) base += sl.lcnt[q];
            const int64_t el = elem(j);
            oid[pos] = a.cand_id[el];
            a.owner_row[((int64_t)p * a.N + n) * a.k + (pos - base)] = a.cand_row[el];
          }
        },
        sl);
  }
  // counts (capped at k over the rank-major order) and padding
  uint32_t base = 0;
  for (int p = 0; p < a.P; ++p) {
    const uint32_t c = sl.lcnt[p];
    const uint32_t kept = base >= (uint32_t)a.k ? 0u : (base + c <= (uint32_t)a.k ? c : (uint32_t)a.k - base);
    int32_t* orow = a.owner_row + ((int64_t)p * a.N + n) * a.k;
    for (int q = (int)kept + tid; q < a.k; q += kThreads) orow[q] = -1;
    if (tid == 0) a.owner_count[(int64_t)p * a.N + n] = (int32_t)kept;
    base += c;
  }
  const int c = run < (uint32_t)a.k ? (int)run : a.k;
  for (int q = c + tid; q < a.k; q += kThreads) oid[q] = -1;
}

}  // namespace

namespace cpa {

int launch_topk_local(const TopkLocalArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.L <= kLdsCands)
    hipLaunchKernelGGL(topk_local_kernel<true>, dim3((unsigned)a.N), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(topk_local_kernel<false>, dim3((unsigned)a.N), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

int launch_topk_merge(const TopkMergeArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if ((int64_t)a.P * a.k_in <= kLdsCands)
    hipLaunchKernelGGL(topk_merge_kernel<true>, dim3((unsigned)a.N), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(topk_merge_kernel<false>, dim3((unsigned)a.N), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace cpa
