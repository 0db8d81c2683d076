// Paged caches: a request's cache is read through a block table that maps
// fixed-size logical blocks to physical pages of a shared pool
// ("DeepSeek-V4 Attention Inference Systems", 1 and 9.1: the decode kernel
// consumes the paged cache directly). Token t of request b lives in pool row
// table[b][t >> shift] * 2^shift + (t & (2^shift - 1)); a table entry
// outside [0, n_pages) is read as page 0.
//
// A workgroup handles one split [t0, t1) of a request's range: before its
// loop it copies the ids of the pages the split touches into LDS (at most
// kPageCap; the host picks enough splits), so the loaders turn a token into
// a row with one LDS read.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace cpa {

// Rows of a contiguous cache: token t is row t.
struct LinearRows {
  static constexpr bool kLinear = true;
  __device__ __forceinline__ int64_t row(int64_t t) const { return t; }
  // tokens a..b are consecutive rows
  __device__ __forceinline__ bool consecutive(int64_t, int64_t) const { return true; }
};

// Rows of a paged cache, from the split's page ids in LDS.
struct PagedRows {
  static constexpr bool kLinear = false;
  const int* pages;  // LDS: ids of pages p0, p0 + 1, ...
  int64_t p0;
  int shift;
  __device__ __forceinline__ int64_t row(int64_t t) const {
    const int j = min((int)((t >> shift) - p0), kPageCap - 1);  // in bounds whatever the range
    return ((int64_t)pages[j] << shift) | (t & ((1 << shift) - 1));
  }
  // tokens a..b (a <= b) lie in one page, so their rows are consecutive
  __device__ __forceinline__ bool consecutive(int64_t a, int64_t b) const { return (a >> shift) == (b >> shift); }
};

// Copies the ids of the pages [t0, t1) touches (entries outside [0, n_pages)
// as 0) into pages[]; threads tid = 0..nthreads-1 of the workgroup share the
// work and the caller places a barrier after it.
__device__ __forceinline__ PagedRows load_pages(int* pages, const int32_t* table_row, int64_t t0, int64_t t1,
                                                int shift, int32_t n_pages, int tid, int nthreads) {
  const int64_t p0 = t0 >> shift;
  const int np = t1 > t0 ? (int)min((int64_t)kPageCap, ((t1 - 1) >> shift) - p0 + 1) : 0;
  for (int j = tid; j < np; j += nthreads) {
    const int32_t e = table_row[p0 + j];
    pages[j] = (uint32_t)e < (uint32_t)n_pages ? e : 0;
  }
  return PagedRows{pages, p0, shift};
}

}  // namespace cpa
