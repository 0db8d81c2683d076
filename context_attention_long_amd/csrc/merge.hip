// Exact LSE merge of S partial attention states.
//
// "How GPUs Share a Long Context During LLM Inference", 3.3: each shard
// reports its output and the log of its sum of exponentiated scores; the
// global LSE is the logsumexp of the shard LSEs and each shard's output is
// rescaled by exp(lse_c - lse) before the outputs are added. The
// "DeepSeek-V4 Attention Inference Systems" notes, section 5, state the same
// combine with max-shifted sums; it is exact up to the order of additions.
//
// Layout: one wavefront per (n, h) row; every lane reads the S LSE values
// (broadcast loads), then the wave streams the S output rows with 16-byte
// loads, four columns per lane per step. The merge is HBM-bound: S * Dv * 4
// bytes in and Dv * 4 (or 2) bytes out per row.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // keep NaN quiet
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void merge_kernel(cpa::MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.N * a.H) return;
  const int64_t n = row / a.H, h = row % a.H;
  const float* lse = a.lse + n * a.l_n + h * a.l_h;
  float m = -INFINITY;
  for (int s = 0; s < a.S; ++s) m = fmaxf(m, lse[s * a.l_s]);
  float lse_tot;
  float inv_tot = 0.f;
  if (m == -INFINITY) {
    lse_tot = -INFINITY;  // no state carries mass: O = 0
  } else {
    float tot = 0.f;
    for (int s = 0; s < a.S; ++s) tot += expf(lse[s * a.l_s] - m);
    lse_tot = m + logf(tot);
    inv_tot = 1.f / tot;
  }
  if (a.lse_out && lane == 0) a.lse_out[n * a.lo_n + h * a.lo_h] = lse_tot;
  const float* o = a.o + n * a.o_n + h * a.o_h;
  for (int d = lane * 4; d < a.Dv; d += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m != -INFINITY) {
      for (int s = 0; s < a.S; ++s) {
        const float w = expf(lse[s * a.l_s] - m) * inv_tot;  // exp(lse_s - lse)
        const float4 x = *reinterpret_cast<const float4*>(o + s * a.o_s + d);
        acc.x += w * x.x;
        acc.y += w * x.y;
        acc.z += w * x.z;
        acc.w += w * x.w;
      }
    }
    if (a.out_bf16) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + n * a.out_n + h * a.out_h + d;
      uint2 pk;
      pk.x = (uint32_t)bf16_rne(acc.x) | ((uint32_t)bf16_rne(acc.y) << 16);
      pk.y = (uint32_t)bf16_rne(acc.z) | ((uint32_t)bf16_rne(acc.w) << 16);
      *reinterpret_cast<uint2*>(out) = pk;
    } else {
      float* out = reinterpret_cast<float*>(a.out) + n * a.out_n + h * a.out_h + d;
      *reinterpret_cast<float4*>(out) = acc;
    }
  }
}

}  // namespace

namespace cpa {

int launch_merge(const MergeArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.N * a.H;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace cpa
