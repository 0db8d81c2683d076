// Split-KV decode over a token-sharded MLA latent cache (bf16, or OCP FP8
// E4M3 with one fp32 scale per token).
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 3.2-3.4 -- a rank attends each request's single query over its own share
// of the cache and reports partial output + LSE; 1.3 and the vLLM DCP post,
// 5.3 -- one latent vector per token is read by all heads.
//
// One workgroup per (query row, split): the split's contiguous token range
// runs through the wave-specialised MLA core (mla_ws.h for a bf16 cache,
// mla_fp8.h for FP8), which reads every cache byte from HBM once per
// workgroup (nontemporal when one query row reads it: the shard is read once
// per launch). The workgroup writes its
// split's normalised output and LSE; the splits of a row are merged by the
// LSE merge.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mla_core.h"
#include "mla_ws.h"
#include "mla_fp8.h"

namespace {

using namespace cpa::mla;

// 8 wavefronts. bf16 cache: tiles arrive by direct loads (mla_ws.h). FP8
// cache: the raw codes stay FP8 in LDS and QK runs on the FP8 matrix cores
// (mla_fp8.h). kP: kStream (one query row per request: every cache byte is
// read once) or kReuse (several query rows read each tile through the
// shared L2).
// kPaged: the cache is a pool read through a block table (paged.h).
template <bool kFp8, cpa::Policy kP, bool kPaged>
__global__ __launch_bounds__(kWsThreads, 1) void decode_mla_ws_kernel(cpa::DecodeMlaArgs a) {
  constexpr int kTileLds = kFp8 ? f8::kStages * f8::kTileBytes : kSmemBytes;
  constexpr int kScaleLds = kFp8 ? f8::kStages * f8::kScaleSlot : 16;
  __shared__ __attribute__((aligned(16))) char smem[kTileLds];
  __shared__ __attribute__((aligned(16))) char ssc[kScaleLds];
  __shared__ __attribute__((aligned(16))) char plds[2 * kH * kPRowBytes];
  __shared__ float alpha_s[2 * kH], lsum_s[kH];
  __shared__ int pages_s[kPaged ? cpa::kPageCap : 1];

  // Work unit u = b * nsplit + split and query row k. Block indices are
  // dealt round-robin to the 8 XCDs (index mod 8). When the requests divide
  // evenly over the XCDs, every workgroup of request b runs on XCD b mod 8:
  // its query rows come from HBM once and reach the other splits through
  // that XCD's L2. Otherwise consecutive units go to consecutive XCDs. The Q
  // rows of one unit are 8 indices apart either way (one XCD, so they share
  // the unit's tiles in L2).
  int u, k;
  if (a.B % 8 == 0 && a.nsplit > 1) {
    const int x = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8), per = a.nsplit * a.Q;
    u = ((j / per) * 8 + x) * a.nsplit + (j % per) / a.Q;
    k = (j % per) % a.Q;
  } else {
    u = (int)(blockIdx.x / (8 * a.Q)) * 8 + (int)(blockIdx.x % 8);
    k = (int)(blockIdx.x / 8) % a.Q;
  }
  if (u >= a.B * a.nsplit) return;
  const int split = u % a.nsplit;
  const int b = u / a.nsplit;
  const int row = b * a.Q + k;
  const int tid = threadIdx.x;
  const int w = (tid >> 6) & 3, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const bool qk_role = tid < 256;

  int64_t beg = a.kv_begin[b], end = a.kv_end[row];
  beg = beg < 0 ? 0 : (beg > a.Lmax ? a.Lmax : beg);
  end = end < beg ? beg : (end > a.Lmax ? a.Lmax : end);
  const int64_t len = end - beg;
  const Tiles T(beg + len * split / a.nsplit, beg + len * (split + 1) / a.nsplit, (unsigned)u * 2654435761u >> 7);
  cpa::PagedRows pr{};
  if constexpr (kPaged) {
    pr = cpa::load_pages(pages_s, a.block_table + (int64_t)b * a.bt_b, T.t0, T.t1, a.page_shift, a.n_pages, tid,
                         kWsThreads);
    __syncthreads();
  }
  auto rows_of = [&]() {
    if constexpr (kPaged) return pr;
    else return cpa::LinearRows{};
  };

  if (qk_role) {
    const uint16_t* qhead = a.q + (int64_t)b * a.q_b + (int64_t)k * a.q_q + (int64_t)(16 * w + c) * a.q_h;
    QkStat st{-INFINITY, 0.f};
    if constexpr (kFp8) {
      const f8::Lds S{smem, ssc, plds, alpha_s, lsum_s, f8::kStages - 1};
      f8::Query Q;
      f8::load_query(qhead, g, Q);
      f8::ws_qk(T, w, g, c, f8::bases(w, g, c), Q, a.scale_log2, st, S);
    } else {
      const Lds S{smem, plds, alpha_s, lsum_s};
      bf16x8 qreg[kQSteps];
      load_q(qhead, g, qreg);
      ws_qk(T, w, g, c, lds_bases(w, g, c), qreg, a.scale_log2, st, S, [&](int i) { return ws_tile(S, i); },
            [](int) { return 0xffffffffu; });
    }
    const float l = sum4_rows(st.l_run);
    if (g == 0) lsum_s[16 * w + c] = l;
    __syncthreads();
    if (g == 0)
      a.lse[(int64_t)split * a.l_s + (int64_t)row * a.l_b + (int64_t)(16 * w + c) * a.l_h] =
          l > 0.f ? (st.m_run + log2f(l)) * kLn2 : -INFINITY;
  } else {
    f32x4 oacc[kMv][4];
#pragma unroll
    for (int m = 0; m < kMv; ++m)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) oacc[m][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp8) {
      const f8::Lds S{smem, ssc, plds, alpha_s, lsum_s, f8::kStages - 1};
      f8::ws_pv<kP>(T, reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)b * a.c_b, a.c_t,
                    a.kv_scale + (int64_t)b * a.s_b, a.s_t, tid - 256, w, g, c, f8::bases(w, g, c), oacc, S,
                    rows_of());
    } else {
      const Lds S{smem, plds, alpha_s, lsum_s};
      ws_pv<kP>(T, reinterpret_cast<const uint16_t*>(a.cache) + (int64_t)b * a.c_b, a.c_t, tid - 256, w, g, c,
                lds_bases(w, g, c), oacc, S, rows_of());
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = 16 * hb + c;
      const float lh = lsum_s[head];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      float* op = a.o + (int64_t)split * a.o_s + (int64_t)row * a.o_b + (int64_t)head * a.o_h + 128 * w + 4 * g;
#pragma unroll
      for (int m = 0; m < kMv; ++m) *reinterpret_cast<f32x4*>(op + 16 * m) = oacc[m][hb] * inv;
    }
  }
}

}  // namespace

namespace cpa {

int launch_decode_mla(const DecodeMlaArgs& a, void* stream) {
  const dim3 grid((unsigned)(((int64_t)a.B * a.nsplit + 7) / 8 * 8 * a.Q));
  constexpr auto kS = Policy::kStream, kR = Policy::kReuse;
  hipStream_t st = (hipStream_t)stream;
  if (a.block_table != nullptr) {  // one query row per request (the host checks)
    if (a.fp8)
      hipLaunchKernelGGL((decode_mla_ws_kernel<true, kS, true>), grid, dim3(kWsThreads), 0, st, a);
    else
      hipLaunchKernelGGL((decode_mla_ws_kernel<false, kS, true>), grid, dim3(kWsThreads), 0, st, a);
  } else if (a.fp8 && a.Q == 1)
    hipLaunchKernelGGL((decode_mla_ws_kernel<true, kS, false>), grid, dim3(kWsThreads), 0, st, a);
  else if (a.fp8)
    hipLaunchKernelGGL((decode_mla_ws_kernel<true, kR, false>), grid, dim3(kWsThreads), 0, st, a);
  else if (a.Q == 1)
    hipLaunchKernelGGL((decode_mla_ws_kernel<false, kS, false>), grid, dim3(kWsThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mla_ws_kernel<false, kR, false>), grid, dim3(kWsThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace cpa
