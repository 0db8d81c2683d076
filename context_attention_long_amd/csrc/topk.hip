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
// A most-significant-digit radix select (8 bits per pass, an LDS
// histogram in 16 copies) finds the k-th key, starting below the leading
// bits every candidate shares and stopping as soon as a digit bin holds
// exactly the entries still needed. The selection is then every key at or
// above one 64-bit threshold; a stable compaction takes it in candidate
// order. Up to 16384 candidates per row keep their score keys in LDS (64 KB,
// candidate j at word j, key 0 in the other words) for all passes; the
// compaction then lists the selected candidates in the same words, and their
// scores, ids and rows are read in one batch. Longer rows are re-read from
// memory (L2) on every pass and written out chunk by chunk.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"

namespace {

constexpr int kThreads = 1024;            // 16 wavefronts per row
constexpr int kWaves = kThreads / 64;
constexpr int kE = 16;                     // chunks of 1024 candidates per compaction round
constexpr int kLdsCands = kE * kThreads;   // 16384 candidates with keys in LDS
constexpr int kVisit = 4 * kThreads;       // slots per step of a sweep: 4 per thread, read together

// Score key: larger = better; 0 is reserved for "no candidate" (an unused
// register slot or a list entry past its count), NaN maps to 1.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 1u;                                   // NaN: below every number
  const uint32_t u = __float_as_uint(s == 0.f ? 0.f : s);  // -0 counts as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The digit histogram is kept in 16 copies, lane l adding into copy l mod
// 16: a float score's leading digits (sign and exponent bits) put most
// entries into a few bins, and LDS atomics of one wavefront on one address
// serialise. A copy's row is 260 words, so copy c's bin d sits in bank
// (4 c + d) mod 64: the copies of one bin never share a bank.
constexpr int kCopies = 16;
constexpr int kCopyWords = 260;

struct alignas(16) SelectLds {
  uint32_t hist[kCopies][kCopyWords];
  uint64_t mask[kE][kWaves];  // selection ballot per (chunk, wave)
  uint32_t off[kE][kWaves];   // output offset of each (chunk, wave)
  uint32_t lcnt[64];          // selected per source list (merge of long lists)
  uint32_t lbase[65];         // first output position of each source list (merge)
  int32_t cnt_in[64];         // entries of each source list (merge)
  uint4 item[64];             // merge load items (see merge_items)
  uint32_t wsum[kWaves];
  uint32_t bcast[4];
};

// Inclusive scans over the 64 lanes of a wavefront with DPP moves (no LDS
// round trips): shifts by 1, 2, 4, 8 within rows of 16 lanes, then the last
// lane of row 0 (2) carried into row 1 (3), then lane 31 into rows 2 and 3.
// Lanes without a source take `id`, the operation's identity.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t id, Op&& op) {
  int x = (int)v;
  const int e = (int)id;
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(e, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(e, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(e, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(e, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(e, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = (int)op((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(e, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)x;
}

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  return wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// The digit search of one radix pass over the histogram's copies: the digit
// d holding the need-th largest key, the count of entries in bins above d and
// in bin d. `phantom` visited slots with key 0 (no candidate) sit in bin 0
// and are taken out. Every thread returns the result.
__device__ __forceinline__ void pick_digit(SelectLds& sl, uint32_t need, uint32_t phantom, uint32_t& d,
                                           uint32_t& above, uint32_t& bin) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __syncthreads();
  if (w == 0) {
    uint32_t b[4] = {0u, 0u, 0u, 0u}, s = 0;  // lane l: bins 255-4l .. 252-4l (descending digit order)
#pragma unroll
    for (int cp = 0; cp < kCopies; ++cp) {
      const uint4 h = *reinterpret_cast<const uint4*>(&sl.hist[cp][252 - 4 * lane]);
      b[0] += h.w, b[1] += h.z, b[2] += h.y, b[3] += h.x;
    }
    if (lane == 63) b[3] -= phantom;  // bin 0
#pragma unroll
    for (int i = 0; i < 4; ++i) s += b[i];
    const uint32_t incl = wave_incl_sum(s);
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
  // (no barrier after the read: bcast is written again only after the next
  // pass's two barriers, and the histogram reads are done)
  d = sl.bcast[0], above = sl.bcast[1], bin = sl.bcast[2];
}

// Histogram add of one digit per lane (lanes with in = false skip): one LDS
// atomic into the lane's copy. (Counting a thread's first two distinct
// digits in registers first, and adding the lanes of a shared digit with one
// atomic, were measured slower.)
__device__ __forceinline__ void hist_add(SelectLds& sl, bool in, uint32_t digit) {
  if (in) atomicAdd(&sl.hist[threadIdx.x & (kCopies - 1)][digit], 1u);
}

__device__ __forceinline__ void clear_hist(SelectLds& sl) {
  // 1024 threads x 4 words: copy t / 64, bins 4 (t mod 64) .. + 3
  static_assert(kCopies * 256 == 4 * kThreads, "one 16-byte store per thread clears the copies");
  *reinterpret_cast<uint4*>(&sl.hist[threadIdx.x >> 6][4 * (threadIdx.x & 63)]) = uint4{0u, 0u, 0u, 0u};
}

// Selection of a radix select: a candidate with score key sk and low key
// word lo is selected iff sk != 0 and (sk, lo) >= (hi, lo_t) in
// lexicographic order. {0, 0} selects every candidate; hi = ~0u selects none
// (no score key reaches it: +inf maps to 0xff800000).
struct Thresh {
  uint32_t hi, lo;
};

// kTie: the threshold's low word is not 0, so candidates whose score key
// equals the threshold's compare their low word (low(slot), read only for
// them); without it the test is branch-free.
template <bool kTie, typename Low>
__device__ __forceinline__ bool is_sel(uint32_t sk, int slot, const Thresh& t, Low&& low) {
  const bool gt = sk > t.hi, eq = (sk == t.hi) & (sk != 0u);
  if constexpr (kTie) return gt || (eq && low(slot) >= t.lo);
  else return gt | eq;
}

// Leading score-key bits shared by every candidate, from each thread's AND
// and OR over its own keys (key 0 left out). Every thread returns the count
// cb and the AND (whose top cb bits are the shared ones).
__device__ __forceinline__ int common_bits(uint32_t& kand, uint32_t kor, SelectLds& sl) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  kand = wave_scan(kand, ~0u, [](uint32_t a, uint32_t b) { return a & b; });  // lane 63: the wavefront's
  kor = wave_scan(kor, 0u, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane == 63) sl.mask[0][w] = ((uint64_t)kand << 32) | kor;
  __syncthreads();  // (the next write of mask[0] follows several barriers)
  kand = ~0u, kor = 0u;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) kand &= (uint32_t)(sl.mask[0][i] >> 32), kor |= (uint32_t)sl.mask[0][i];
  return (kand ^ kor) ? __clz(kand ^ kor) : 32;
}

// Radix select of the k largest keys among `total` candidates. each(f)
// visits slots, every lane of a wavefront the same number of times: f(slot,
// any, sk) with any = false for a visit past the end, else the score key
// (0: no candidate; `phantom` such slots are visited); low(slot) gives the
// low key word (~id), asked for only when equal scores reach the threshold.
// kand / kor: this thread's AND and OR over the score keys (key 0 left out).
// A slot without candidate has key 0, below every candidate, so it can only
// sit in the bins of the all-zero prefix, from which pick_digit removes it.
// kTop: the histogram already holds the top 8 bits of every candidate's key
// (counted while the keys were loaded; empty slots not counted).
template <bool kTop = false, typename Each, typename Low>
__device__ __forceinline__ Thresh radix_select(uint32_t total, uint32_t phantom, int k, uint32_t kand, uint32_t kor,
                                               Each&& each, Low&& low, SelectLds& sl) {
  if (total <= (uint32_t)k) return Thresh{0u, 0u};
  if (k <= 0) return Thresh{~0u, ~0u};
  // the digits start below the shared leading bits (the merge's candidates
  // all lie in the upper tail, where the top digit would put almost
  // everything into one or two bins)
  const int cb = common_bits(kand, kor, sl);  // (its barrier also publishes a kTop histogram)
  int prev = 64 - cb;  // key bits below the known prefix
  uint64_t prefix = (uint64_t)kand >> (32 - cb);
  int shift = prev;
  uint32_t need = (uint32_t)k;
  if constexpr (kTop) {
    uint32_t d, above, bin;
    pick_digit(sl, need, 0u, d, above, bin);
    need -= above;
    if (bin == need) {
      const uint64_t thr = (uint64_t)d << 56;
      return Thresh{(uint32_t)(thr >> 32), 0u};
    }
    if (cb <= 8) prefix = d, prev = 56;  // else the shared bits (d among them) go further
  }
  while (prev > 0) {
    const int sh = prev > 32 ? max(prev - 8, 32) : prev - 8;
    const uint32_t dmask = (1u << (prev - sh)) - 1u;
    clear_hist(sl);
    __syncthreads();
    if (sh >= 32) {
      // a digit of the score key among the keys whose bits above prev - 32
      // are the prefix
      const int s32 = sh - 32, p32 = prev - 32;
      const uint32_t hmask = p32 >= 32 ? 0u : ~0u << p32;
      const uint32_t hval = p32 >= 32 ? 0u : (uint32_t)prefix << p32;
      each([&](int, bool any, uint32_t sk) { hist_add(sl, any && (sk & hmask) == hval, (sk >> s32) & dmask); });
    } else {
      // equal score keys at the threshold: a digit of the low word among the
      // keys with that score key whose low bits above prev are the prefix's
      const uint32_t hi = (uint32_t)(prefix >> (32 - prev));
      const uint32_t lmask = prev >= 32 ? 0u : ~0u << prev;
      const uint32_t lval = prev >= 32 ? 0u : (uint32_t)prefix << prev;
      each([&](int slot, bool any, uint32_t sk) {
        uint32_t lo = 0u;
        bool in = false;
        if (any && sk == hi && hi != 0u) {  // a slot without candidate has key 0
          lo = low(slot);
          in = (lo & lmask) == lval;
        }
        hist_add(sl, in, (lo >> sh) & dmask);
      });
    }
    uint32_t d, above, bin;
    pick_digit(sl, need, prefix == 0 ? phantom : 0u, d, above, bin);
    need -= above;
    prefix = (prefix << (prev - sh)) | d;
    shift = sh;
    prev = sh;
    if (bin == need) break;  // every entry of this bin is selected
  }
  const uint64_t thr = prefix << shift;  // prefix holds 64 - shift bits
  return Thresh{(uint32_t)(thr >> 32), (uint32_t)thr};
}

// Stable compaction in candidate order (chunk e holds candidates 1024 e +
// thread, e < nchunk <= kE): sel(e) says whether this thread's candidate of
// chunk e is selected; emit(e, pos) writes it at output position pos.
// kAll: all kE chunks, unrolled so their reads overlap (sel must then be
// safe for every chunk). Returns the number selected.
template <bool kAll = false, typename Sel, typename Emit>
__device__ __forceinline__ uint32_t compact(int nchunk, Sel&& sel, Emit&& emit, SelectLds& sl) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t mine = 0;  // kAll: bit e = this thread's candidate of chunk e is selected
  if constexpr (kAll) nchunk = kE;
  auto chunks = [&](auto&& f) {
    if constexpr (kAll) {
#pragma unroll
      for (int e = 0; e < kE; ++e) f(e);
    } else {
#pragma unroll 4
      for (int e = 0; e < nchunk; ++e) f(e);
    }
  };
  if constexpr (kAll) {
    // every chunk's test first (their LDS reads overlap), then lane e keeps
    // chunk e's ballot and the lanes store them at once
    bool s[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) s[e] = sel(e);
#pragma unroll
    for (int e = 0; e < kE; ++e) mine |= (uint32_t)s[e] << e;
    int mlo = 0, mhi = 0;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const uint64_t m = __ballot(s[e]);
      mlo = lane == e ? (int)(uint32_t)m : mlo;
      mhi = lane == e ? (int)(uint32_t)(m >> 32) : mhi;
    }
    if (lane < kE) sl.mask[lane][w] = ((uint64_t)(uint32_t)mhi << 32) | (uint32_t)mlo;
  } else {
    chunks([&](int e) {
      const uint64_t m = __ballot(sel(e));
      if (lane == 0) sl.mask[e][w] = m;
    });
  }
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
    const uint32_t incl = wave_incl_sum(sum);
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
  if constexpr (kAll) {
    // each lane visits only its selected chunks (a small share of the 16)
    for (uint32_t bits = mine; bits; bits &= bits - 1u) {
      const int e = __builtin_ctz(bits);
      const uint64_t m = sl.mask[e][w];
      emit(e, sl.off[e][w] + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)));
    }
  } else {
    chunks([&](int e) {
      const uint64_t m = sl.mask[e][w];
      if ((m >> lane) & 1ull) emit(e, sl.off[e][w] + (uint32_t)__popcll(m & ((1ull << lane) - 1ull)));
    });
  }
  const uint32_t total = sl.wsum[0];
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------- local

// Score keys of a row's first nv slots into LDS, key 0 in the other slots
// (all 16384 are written, so any slot may be read); returns this thread's AND
// and OR over its keys (key 0 left out). key(j, v) maps slot j's loaded
// score v and must be safe for any j < 16384 (v is junk for j >= nv).
template <typename Addr, typename Key>
__device__ __forceinline__ void keys_to_lds(uint32_t* skl, int nv, const float* base, Addr&& addr, Key&& key,
                                            uint32_t& kand, uint32_t& kor, SelectLds& sl) {
  const int tid = threadIdx.x;
  kand = ~0u, kor = 0u;
  float v[kE];  // one batch of 16 loads in flight
#pragma unroll
  for (int u = 0; u < kE; ++u) v[u] = nv > 0 ? base[addr(min(tid + kThreads * u, nv - 1))] : 0.f;
#pragma unroll
  for (int u = 0; u < kE; ++u) {
    const int j = tid + kThreads * u;
    const uint32_t kk = key(j, v[u]);
    const uint32_t kj = j < nv ? kk : 0u;
    skl[j] = kj;
    kor |= kj;
    kand &= kj ? kj : ~0u;
    hist_add(sl, kj != 0u, kj >> 24);  // the first radix digit
  }
}

// The merge loads its P lists as (list p, block i of 1024 entries) items,
// f = p nblk + i, at most 64 when the keys fit LDS. Lane f of wave 0 writes
// item f: {element offset of entry 1024 i (2 words), its LDS word p k_in +
// 1024 i, entries with a score (up to 1024) | entries inside the list << 16};
// items past P nblk are empty. c: lane p's list count.
__device__ __forceinline__ void merge_items(const cpa::TopkMergeArgs& a, int n, int c, SelectLds& sl) {
  const int f = threadIdx.x & 63;
  const int nblk = (a.k_in + kThreads - 1) / kThreads;
  const int p = nblk > 0 ? f / nblk : 0, i = f - p * nblk;
  const int cp = __shfl(c, p & 63);
  uint4 d = {0u, 0u, (uint32_t)kLdsCands, 0u};
  if (f < a.P * nblk) {
    const int64_t e = (int64_t)p * ((int64_t)a.N * a.k_in) + (int64_t)n * a.k_in + kThreads * i;
    const int has = min(max(cp - kThreads * i, 0), kThreads), in = min(a.k_in - kThreads * i, kThreads);
    d = uint4{(uint32_t)e, (uint32_t)(e >> 32), (uint32_t)(p * a.k_in + kThreads * i), (uint32_t)has | (uint32_t)in << 16};
  }
  sl.item[f] = d;
}

// The merge's score keys into LDS from the items: entry s of list p goes to
// word p k_in + s (key 0 past the list's count), words from P k_in on get
// key 0; skl holds 1024 more words, written but never read (entries past
// k_in in a list's last block, and empty items, write there).
__device__ __forceinline__ void merge_keys_to_lds(uint32_t* skl, const cpa::TopkMergeArgs& a, SelectLds& sl,
                                                  uint32_t& kand, uint32_t& kor) {
  const int tid = threadIdx.x;
  const int nitem = a.P * ((a.k_in + kThreads - 1) / kThreads);
  kand = ~0u, kor = 0u;
  for (int f0 = 0; f0 < nitem; f0 += kE) {  // nitem <= 64: items f0 .. f0 + 15 all exist
    float v[kE];
    int slot[kE];
    bool ok[kE];
#pragma unroll
    for (int u = 0; u < kE; ++u) {
      const uint4 d = sl.item[f0 + u];
      ok[u] = tid < (int)(d.w & 0xffffu);
      slot[u] = tid < (int)(d.w >> 16) ? (int)d.z + tid : kLdsCands + tid;
      const int64_t e = (int64_t)(((uint64_t)d.y << 32) | d.x) + tid;
      v[u] = a.cand_score[ok[u] ? e : 0];  // every lane loads (element 0 stands in)
    }
#pragma unroll
    for (int u = 0; u < kE; ++u) {
      const uint32_t kj = ok[u] ? score_key(v[u]) : 0u;
      skl[slot[u]] = kj;
      kor |= kj;
      kand &= kj ? kj : ~0u;
      hist_add(sl, kj != 0u, kj >> 24);  // the first radix digit
    }
  }
  for (int j = a.P * a.k_in + tid; j < kLdsCands; j += kThreads) skl[j] = 0u;
}

// Sweep over the LDS keys of slots [0, npad): the keys of four chunks are
// read together so their LDS latencies overlap.
template <typename F>
__device__ __forceinline__ void each_lds(const uint32_t* skl, int npad, F&& f) {
  const int tid = threadIdx.x;
  for (int j0 = 0; j0 < npad; j0 += kVisit) {
    uint32_t kk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kk[u] = skl[j0 + tid + u * kThreads];
#pragma unroll
    for (int u = 0; u < 4; ++u) f(j0 + tid + u * kThreads, true, kk[u]);
  }
}

// kLds: the row's score keys fit LDS (L <= 16384); otherwise they are
// re-read from memory every pass.
template <bool kLds>
__global__ __launch_bounds__(kThreads) void topk_local_kernel(cpa::TopkLocalArgs a) {
  __shared__ SelectLds sl;
  __shared__ uint32_t skl[kLds ? kLdsCands : 1];  // score keys, then the selected slots
  const int n = blockIdx.x, tid = threadIdx.x;
  int nv = a.n_valid ? a.n_valid[n] : a.L;
  nv = nv < 0 ? 0 : (nv > a.L ? a.L : nv);
  const float* sc = a.scores + (int64_t)n * a.s_n;
  auto id_of = [&](int j) { return (int32_t)(a.id_base + (int64_t)j * a.id_stride); };
  auto low = [&](int j) { return ~(uint32_t)id_of(j); };
  float* os = a.out_score + (int64_t)n * a.k;
  int32_t* oi = a.out_id + (int64_t)n * a.k;
  int32_t* orow = a.out_row + (int64_t)n * a.k;
  uint32_t run;
  if constexpr (kLds) {
    const int npad = (nv + kVisit - 1) / kVisit * kVisit;
    uint32_t kand, kor;
    clear_hist(sl);
    __syncthreads();
    keys_to_lds(
        skl, nv, sc, [](int j) { return j; }, [](int, float v) { return score_key(v); }, kand, kor, sl);
    __syncthreads();
    auto each = [&](auto&& f) { each_lds(skl, npad, f); };
    const Thresh t = radix_select<true>((uint32_t)nv, (uint32_t)(npad - nv), a.k, kand, kor, each, low, sl);
    // the selected slots in candidate order replace the keys (every key read
    // is done before the first write: compact synchronises in between)
    auto emit = [&](int e, uint32_t pos) {
      if (pos < (uint32_t)a.k) skl[pos] = (uint32_t)(tid + kThreads * e);
    };
    auto sel = [&](auto tie) {
      return [&, tie](int e) {
        const int j = tid + kThreads * e;
        return is_sel<decltype(tie)::value>(skl[j], j, t, low);
      };
    };
    run = t.lo ? compact<true>(0, sel(std::true_type{}), emit, sl) : compact<true>(0, sel(std::false_type{}), emit, sl);
    const int c = run < (uint32_t)a.k ? (int)run : a.k;
    // scores from the row itself (-0 and NaN bits kept), ids and rows
    for (int p0 = 0; p0 < c; p0 += 4 * kThreads) {
      int j[4];
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) j[u] = (int)skl[min(p0 + tid + u * kThreads, c - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = sc[j[u]];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + tid + u * kThreads;
        if (p < c) {
          os[p] = v[u];
          oi[p] = id_of(j[u]);
          orow[p] = j[u];
        }
      }
    }
  } else {
    auto key_at = [&](int j) { return score_key(sc[j]); };
    // every lane runs the same trip count; the keys of four chunks are read
    // together (unconditionally, clamped)
    auto each = [&](auto&& f) {
      for (int j0 = 0; j0 < nv; j0 += kVisit) {
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
    uint32_t kand = ~0u, kor = 0u;
    each([&](int, bool any, uint32_t sk) {
      if (any && sk != 0u) kand &= sk, kor |= sk;
    });
    const Thresh t = radix_select((uint32_t)nv, 0u, a.k, kand, kor, each, low, sl);
    run = 0;
    const int nchunk = (nv + kThreads - 1) / kThreads;
    for (int c0 = 0; c0 < nchunk; c0 += kE) {
      const int nc = min(kE, nchunk - c0);
      const uint32_t base = run;
      run += compact(
          nc,
          [&](int e) {
            const int j = tid + kThreads * (c0 + e);
            const int jc = min(j, nv - 1);  // clamped: the key read and id stay in range
            return (j < nv) && is_sel<true>(key_at(jc), jc, t, low);
          },
          [&](int e, uint32_t pos) {
            const int j = tid + kThreads * (c0 + e);
            pos += base;
            if (pos < (uint32_t)a.k) {
              os[pos] = sc[j];
              oi[pos] = id_of(j);
              orow[pos] = j;
            }
          },
          sl);
    }
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
  __shared__ uint32_t skl[kLds ? kLdsCands + kThreads : 1];  // score keys, then the selected candidates
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
    const uint32_t t = wave_incl_sum((uint32_t)c);  // lane 63: the total over the lists
    if (tid == 63) sl.wsum[0] = t;
    if constexpr (kLds) merge_items(a, n, c, sl);
  }
  if constexpr (kLds) clear_hist(sl);
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
  auto elem_in = [&](int j, int p) { return p * plane + (int64_t)n * a.k_in + (j - p * a.k_in); };
  auto elem = [&](int j) { return elem_in(j, list_of(j)); };
  auto exists = [&](int j) { const int p = list_of(j); return j - p * a.k_in < sl.cnt_in[p]; };
  auto low = [&](int j) { return ~(uint32_t)a.cand_id[elem(j)]; };
  int32_t* oid = a.out_id + (int64_t)n * a.k;
  if constexpr (kLds) {
    const int npad = (M + kVisit - 1) / kVisit * kVisit;
    uint32_t kand, kor;
    merge_keys_to_lds(skl, a, sl, kand, kor);
    __syncthreads();
    auto each = [&](auto&& f) { each_lds(skl, npad, f); };
    const Thresh t = radix_select<true>(total, (uint32_t)npad - total, a.k, kand, kor, each, low, sl);
    // the selected candidates in candidate order replace the keys
    auto emit = [&](int e, uint32_t pos) {
      if (pos < (uint32_t)a.k) skl[pos] = (uint32_t)(tid + kThreads * e);
    };
    auto sel = [&](auto tie) {
      return [&, tie](int e) {
        const int j = tid + kThreads * e;
        return is_sel<decltype(tie)::value>(skl[j], j, t, low);
      };
    };
    const uint32_t run =
        t.lo ? compact<true>(0, sel(std::true_type{}), emit, sl) : compact<true>(0, sel(std::false_type{}), emit, sl);
    const int c = run < (uint32_t)a.k ? (int)run : a.k;
    // where list p's run starts in the output: the selected candidates before
    // its first one, from the compaction's cell offsets and ballots
    if (tid < 64) {
      if (tid < a.P) {
        const int j0 = tid * a.k_in;  // < 16384
        const int e = j0 >> 10, cw = (j0 >> 6) & (kWaves - 1), cl = j0 & 63;
        const uint32_t before = sl.off[e][cw] + (uint32_t)__popcll(sl.mask[e][cw] & ((1ull << cl) - 1ull));
        sl.lbase[tid] = before < (uint32_t)c ? before : (uint32_t)c;
      }
      if (tid == 0) sl.lbase[a.P] = (uint32_t)c;
    }
    __syncthreads();
    // ids and owner rows of the selection, one batch of loads per 4096
    for (int p0 = 0; p0 < c; p0 += 4 * kThreads) {
      int q[4];
      int32_t id[4], row[4];
      int64_t el[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = (int)skl[min(p0 + tid + u * kThreads, c - 1)];
        q[u] = list_of(j);
        el[u] = elem_in(j, q[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) id[u] = a.cand_id[el[u]], row[u] = a.cand_row[el[u]];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + tid + u * kThreads;
        if (p < c) {
          oid[p] = id[u];
          a.owner_row[((int64_t)q[u] * a.N + n) * a.k + (p - (int)sl.lbase[q[u]])] = row[u];
        }
      }
    }
    for (int p = 0; p < a.P; ++p) {
      const int kept = (int)(sl.lbase[p + 1] - sl.lbase[p]);
      int32_t* orow = a.owner_row + ((int64_t)p * a.N + n) * a.k;
      for (int q = kept + tid; q < a.k; q += kThreads) orow[q] = -1;
      if (tid == 0) a.owner_count[(int64_t)p * a.N + n] = kept;
    }
    for (int q = c + tid; q < a.k; q += kThreads) oid[q] = -1;
  } else {
    auto key_at = [&](int j) { return exists(j) ? score_key(a.cand_score[elem(j)]) : 0u; };
    auto each = [&](auto&& f) {
      for (int j0 = 0; j0 < M; j0 += kVisit) {
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
    uint32_t kand = ~0u, kor = 0u;
    each([&](int, bool any, uint32_t sk) {
      if (any && sk != 0u) kand &= sk, kor |= sk;
    });
    const Thresh t = radix_select(total, (uint32_t)M - total, a.k, kand, kor, each, low, sl);
    auto sel_of = [&](int j) {
      const int jc = min(j, M - 1);  // clamped: the key read and id stay in range
      return (j < M) && is_sel<true>(key_at(jc), jc, t, low);
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
