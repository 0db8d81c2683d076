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
// (broadcast loads), then the wave reads the S output rows with 16-byte
// loads, four columns per lane per piece: S * Dv * 4 bytes in and Dv * 4
// (or 2) bytes out per row.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // keep NaN quiet
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The kernel is bound by memory latency, not bandwidth: a row's wavefront
// moves S * Dv * 4 bytes, a few KB. So every load of a chunk of up to kCh
// states (their LSEs, and the two 4-column pieces a lane owns in a 512-column
// stretch) is issued before the first one is used: one round trip per chunk
// instead of one per state and piece. Additions keep the order s = 0, 1, ...
// kExact: S == CH (compile-time). Otherwise CH = kCh and the last chunk's
// missing states re-read state S - 1 and are skipped.
constexpr int kCh = 8;

template <int CH, bool kExact>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void merge_kernel(cpa::MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.N * a.H) return;
  const int S = kExact ? CH : a.S;
  const int64_t n = row / a.H, h = row % a.H;
  const float* lse = a.lse + n * a.l_n + h * a.l_h;
  auto state = [&](int s0, int j) { return kExact ? j : min(s0 + j, S - 1); };
  auto load_lse = [&](int s0, float (&v)[CH]) {
#pragma unroll
    for (int j = 0; j < CH; ++j) v[j] = lse[(int64_t)state(s0, j) * a.l_s];
  };
  float m = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float v[CH];
    load_lse(s0, v);
#pragma unroll
    for (int j = 0; j < CH; ++j) m = fmaxf(m, v[j]);  // a repeated state leaves the max unchanged
  }
  float lse_tot;
  float inv_tot = 0.f;
  if (m == -INFINITY) {
    lse_tot = -INFINITY;  // no state carries mass: O = 0
  } else {
    float tot = 0.f;
    for (int s0 = 0; s0 < S; s0 += CH) {
      float v[CH];
      load_lse(s0, v);
#pragma unroll
      for (int j = 0; j < CH; ++j)
        if (kExact || s0 + j < S) tot += expf(v[j] - m);
    }
    lse_tot = m + logf(tot);
    inv_tot = 1.f / tot;
  }
  if (a.lse_out && lane == 0) a.lse_out[n * a.lo_n + h * a.lo_h] = lse_tot;
  const float* o = a.o + n * a.o_n + h * a.o_h;
  auto store = [&](int d, const float4& acc) {
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
  };
  for (int d = lane * 4; d < a.Dv; d += 512) {
    // the lane's columns d and d + 256 (when inside the row)
    const bool two = d + 256 < a.Dv;
    const int d2 = two ? d + 256 : d;
    float4 acc0 = make_float4(0.f, 0.f, 0.f, 0.f), acc1 = acc0;
    if (m != -INFINITY) {
      for (int s0 = 0; s0 < S; s0 += CH) {
        float v[CH];
        float4 x0[CH], x1[CH];
        load_lse(s0, v);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const float* os = o + (int64_t)state(s0, j) * a.o_s;
          x0[j] = *reinterpret_cast<const float4*>(os + d);
          x1[j] = *reinterpret_cast<const float4*>(os + d2);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          if (!kExact && s0 + j >= S) continue;
          const float w = expf(v[j] - m) * inv_tot;  // exp(lse_s - lse)
          acc0.x += w * x0[j].x;
          acc0.y += w * x0[j].y;
          acc0.z += w * x0[j].z;
          acc0.w += w * x0[j].w;
          acc1.x += w * x1[j].x;
          acc1.y += w * x1[j].y;
          acc1.z += w * x1[j].z;
          acc1.w += w * x1[j].w;
        }
      }
    }
    store(d, acc0);
    if (two) store(d2, acc1);
  }
}

}  // namespace

namespace cpa {

int launch_merge(const MergeArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.N * a.H;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipStream_t st = (hipStream_t)stream;
  switch (a.S) {
    case 1: hipLaunchKernelGGL((merge_kernel<1, true>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((merge_kernel<2, true>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((merge_kernel<3, true>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((merge_kernel<4, true>), grid, dim3(256), 0, st, a); break;
    case 5: hipLaunchKernelGGL((merge_kernel<5, true>), grid, dim3(256), 0, st, a); break;
    case 6: hipLaunchKernelGGL((merge_kernel<6, true>), grid, dim3(256), 0, st, a); break;
    case 7: hipLaunchKernelGGL((merge_kernel<7, true>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((merge_kernel<8, true>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((merge_kernel<kCh, false>), grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace cpa
