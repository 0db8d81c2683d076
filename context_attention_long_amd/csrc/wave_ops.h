// Cross-lane reductions shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace cpa {

// Maximum / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane
// groups that hold one column of a 16x16 MFMA result, e.g. one head), with
// the gfx950 row-swap permutes instead of LDS round trips.
// (compare-select rather than fmaxf: the swapped values are not known to be
// canonical floats, and fmaxf would canonicalise both operands first)
__device__ __forceinline__ float max4_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a0 = __uint_as_float(a[0]), a1 = __uint_as_float(a[1]);
  const float y = a0 > a1 ? a0 : a1;
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  const float b0 = __uint_as_float(b[0]), b1 = __uint_as_float(b[1]);
  return b0 > b1 ? b0 : b1;
}

__device__ __forceinline__ float sum4_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace cpa
