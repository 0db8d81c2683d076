// Sparse (top-k index list) MLA attention over a latent cache.
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 2.4 -- a query of a sparse-attention model brings its own list of selected
// tokens; vLLM GLM-5.3 part 2, footnote 1 -- each query reads its 2,048
// selected latent rows for all heads (QK over 576 dims, PV over 512). The
// output is the partial O + LSE of the listed rows, so owner-local lists on
// several ranks combine with the LSE merge (DeepSeek-V4 notes, 5.2).
//
// One workgroup per (query, split): the split's share of the query's list
// runs through the wave-specialised MLA core (mla_ws.h, ws_pv_gather; for an
// FP8 cache with per-token scales the FP8-resident core, mla_fp8.h), which
// gathers the listed rows into LDS tiles with direct loads whose addresses
// come from the list itself (staged in LDS ahead of use). The splits of a
// query are merged by the LSE merge.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mla_core.h"
#include "mla_fp8.h"
#include "mla_ws.h"

namespace {

using namespace cpa::mla;

template <bool kFp8, cpa::Policy kP>
__global__ __launch_bounds__(kWsThreads, 1) void sparse_mla_kernel(cpa::SparseMlaArgs a) {
  constexpr int kTileLds = kFp8 ? f8::kGatherStages * f8::kTileBytes : kSmemBytes;
  __shared__ __attribute__((aligned(16))) char smem[kTileLds];
  __shared__ __attribute__((aligned(16))) char ssc[kFp8 ? f8::kGatherStages * f8::kScaleSlot : 16];
  __shared__ __attribute__((aligned(16))) char plds[2 * kH * kPRowBytes];
  __shared__ __attribute__((aligned(16))) char ring[kIdxRingBytes];
  __shared__ float alpha_s[2 * kH], lsum_s[kH];
  const Lds S{smem, plds, alpha_s, lsum_s};

  // (query, split) of this workgroup. Block indices are dealt round-robin
  // to the 8 XCDs (index mod 8); when the queries divide evenly over them,
  // the splits of query n all run on XCD n mod 8, so its bf16 query rows
  // come from HBM once and reach the other splits through that XCD's L2.
  int split, n;
  if (a.N % 8 == 0 && a.nsplit > 1) {
    const int x = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
    n = (j / a.nsplit) * 8 + x;
    split = j % a.nsplit;
  } else {
    split = (int)(blockIdx.x % a.nsplit);
    n = (int)(blockIdx.x / a.nsplit);
  }
  const int tid = threadIdx.x;
  const int w = (tid >> 6) & 3, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const bool qk_role = tid < 256;

  int b = a.req ? a.req[n] : n;
  int cnt = a.n_idx ? a.n_idx[n] : a.K;
  cnt = cnt < 0 ? 0 : (cnt > a.K ? a.K : cnt);
  if (b < 0 || b >= a.B || a.Lmax <= 0) cnt = 0, b = 0;  // no request or empty cache: nothing selected
  const int e0 = (int)((int64_t)cnt * split / a.nsplit);
  const int e1 = (int)((int64_t)cnt * (split + 1) / a.nsplit);
  // the tile "positions" are list entries [e0, e1)
  const Tiles T(0, e1 - e0, blockIdx.x * 2654435761u >> 7);
  const LdsBases L = lds_bases(w, g, c);

  // selection bits of tile i from the entry ring of PV wavefront w
  const char* wring = ring + w * (kIdxSlots * kIdxSlotBytes);
  auto mask = [&](int i) -> uint32_t {
    const int v = *reinterpret_cast<const int*>(wring + (i % kIdxSlots) * kIdxSlotBytes + 4 * (lane & 31));
    return (uint32_t)__ballot((uint32_t)v < (uint32_t)a.Lmax);
  };
  const int32_t* ilist = a.idx + (int64_t)n * a.i_n + e0;
  auto finish_lse = [&](const QkStat& st) {
    const float l = sum4_rows(st.l_run);
    if (g == 0) S.lsum[16 * w + c] = l;
    __syncthreads();
    if (g == 0)
      a.lse[(int64_t)split * a.l_s + (int64_t)n * a.l_n + (int64_t)(16 * w + c) * a.l_h] =
          l > 0.f ? (st.m_run + log2f(l)) * kLn2 : -INFINITY;
  };
  if (qk_role) {
    QkStat st{-INFINITY, 0.f};
    const uint16_t* qhead = a.q + (int64_t)n * a.q_n + (int64_t)(16 * w + c) * a.q_h;
    if constexpr (kFp8) {
      const f8::Lds S8{smem, ssc, plds, alpha_s, lsum_s, f8::kGatherStages - 1};
      f8::Query Q;
      f8::load_query(qhead, g, Q);
      f8::ws_qk<true>(T, w, g, c, f8::bases(w, g, c), Q, a.scale_log2, st, S8, mask);
    } else {
      bf16x8 qreg[kQSteps];
      load_q(qhead, g, qreg);
      ws_qk<true>(T, w, g, c, L, qreg, a.scale_log2, st, S, [&](int i) { return ws_tile(S, i); }, mask);
    }
    finish_lse(st);
  } else {
    f32x4 oacc[kMv][4];
#pragma unroll
    for (int m = 0; m < kMv; ++m)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) oacc[m][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp8) {
      const f8::Lds S8{smem, ssc, plds, alpha_s, lsum_s, f8::kGatherStages - 1};
      f8::ws_pv_gather<kP>(T, reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)b * a.c_b, a.c_t,
                           a.kv_scale + (int64_t)b * a.s_b, a.s_t, ilist, a.Lmax, tid - 256, w, g, c,
                           f8::bases(w, g, c), oacc, S8, ring);
    } else {
      ws_pv_gather<kP>(T, reinterpret_cast<const uint16_t*>(a.cache) + (int64_t)b * a.c_b, a.c_t, ilist, a.Lmax,
                       tid - 256, w, g, c, L, oacc, S, ring);
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = 16 * hb + c;
      const float lh = lsum_s[head];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      float* op = a.o + (int64_t)split * a.o_s + (int64_t)n * a.o_n + (int64_t)head * a.o_h + 128 * w + 4 * g;
#pragma unroll
      for (int m = 0; m < kMv; ++m) *reinterpret_cast<f32x4*>(op + 16 * m) = oacc[m][hb] * inv;
    }
  }
}

}  // namespace

namespace cpa {

int launch_sparse_mla(const SparseMlaArgs& a, void* stream) {
  const dim3 grid((unsigned)((int64_t)a.N * a.nsplit));
  hipStream_t st = (hipStream_t)stream;
  if (a.fp8) {
    if (a.reuse)
      hipLaunchKernelGGL((sparse_mla_kernel<true, Policy::kReuse>), grid, dim3(kWsThreads), 0, st, a);
    else
      hipLaunchKernelGGL((sparse_mla_kernel<true, Policy::kStream>), grid, dim3(kWsThreads), 0, st, a);
  } else if (a.reuse) {
    hipLaunchKernelGGL((sparse_mla_kernel<false, Policy::kReuse>), grid, dim3(kWsThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((sparse_mla_kernel<false, Policy::kStream>), grid, dim3(kWsThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace cpa
