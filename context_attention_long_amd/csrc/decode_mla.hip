// Split-KV decode over a token-sharded MLA latent cache (bf16, or OCP FP8
// E4M3 with one fp32 scale per token).
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 3.2-3.4 -- a rank attends each request's single query over its own share
// of the cache and reports partial output + LSE; 1.3 and the vLLM DCP post,
// 5.3 -- one latent vector per token is read by all heads.
//
// One workgroup per (query row, split): the split's contiguous token range
// runs through the wave-specialised MLA core (mla_ws.h), which reads every
// cache byte from HBM once per workgroup (nontemporal when one query row
// reads it: the shard is read once per launch). The workgroup writes its
// split's normalised output and LSE; the splits of a row are merged by the
// LSE merge.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mla_core.h"
#include "mla_ws.h"

namespace {

using namespace cpa::mla;

// 8 wavefronts: bf16 tiles arrive by direct loads, FP8 tiles are converted
// into LDS by the PV wavefronts. kP: kStream (one query row per request:
// every cache byte is read once) or kReuse (several query rows read each
// tile through the shared L2).
template <bool kFp8, cpa::Policy kP>
__global__ __launch_bounds__(kWsThreads, 1) void decode_mla_ws_kernel(cpa::DecodeMlaArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ __attribute__((aligned(16))) char plds[2 * kH * kPRowBytes];
  __shared__ float alpha_s[2 * kH], lsum_s[kH];
  const Lds S{smem, plds, alpha_s, lsum_s};

  const int u = (int)(blockIdx.x / (8 * a.Q)) * 8 + (int)(blockIdx.x % 8);
  const int k = (int)(blockIdx.x / 8) % a.Q;
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
  const LdsBases L = lds_bases(w, g, c);

  if (qk_role) {
    bf16x8 qreg[kQSteps];
    load_q(a.q + (int64_t)b * a.q_b + (int64_t)k * a.q_q + (int64_t)(16 * w + c) * a.q_h, g, qreg);
    QkStat st{-INFINITY, 0.f};
    if constexpr (kFp8) {
      const float* sbase = a.kv_scale + (int64_t)b * a.s_b;
      const uint32_t st32 = (uint32_t)a.s_t;  // the host bounds the scale stride
      auto scales = [&](int i, TokScale& ts) {  // the 8 tokens whose scores this lane holds
        const int64_t tok0 = T.t0 + (int64_t)T.phys(i) * kBN;
        const int lim = (int)min((int64_t)(kBN - 1), T.t1 - 1 - tok0);
        const float* sb = sbase + tok0 * a.s_t;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t r = (uint32_t)min(16 * (j >> 2) + 4 * g + (j & 3), lim);
          if constexpr (kP == cpa::Policy::kStream) ts.v[j] = __builtin_nontemporal_load(sb + r * st32);
          else ts.v[j] = sb[r * st32];
        }
      };
      // this role's share of the FP8 conversion, 4 units per thread: step i
      // (before the barrier that publishes tile i+1) converts tile i+1 into
      // stage (i+1) % 3 from set (i+1) & 1 and refills that set with tile
      // i+3; the PV role converts its units of the same tile in the same
      // interval.
      Fp8Units<4, kP> U;
      U.base = reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)b * a.c_b, U.c_t = a.c_t, U.t = tid;
      if (T.ntiles > 0) U.template prologue<1>(T, S);
      auto convert_ahead = [&](int i, auto parity) {
        constexpr int P = decltype(parity)::value;
        char* dst = S.tiles + ((i + 1) % 3) * kTileBytes;
        const int refill_t = min(i + 3, T.ntiles - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          U.convert(j, P ^ 1, dst);
          U.load(T, refill_t, j, P ^ 1);
        }
      };
      ws_qk<true>(T, w, g, c, L, qreg, a.scale_log2, st, S, [&](int i) { return S.tiles + (i % 3) * kTileBytes; },
                  scales, [](int) { return 0xffffffffu; }, convert_ahead);
    } else {
      ws_qk<false>(T, w, g, c, L, qreg, a.scale_log2, st, S, [&](int i) { return ws_tile(S, i); },
                   [](int, TokScale&) {}, [](int) { return 0xffffffffu; });
    }
    const float l = sum4_rows(st.l_run);
    if (g == 0) S.lsum[16 * w + c] = l;
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
    if constexpr (kFp8)
      ws_pv_fp8<kP>(T, reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)b * a.c_b, a.c_t, tid - 256, w, g, c, L,
                    oacc, S);
    else
      ws_pv<kP>(T, reinterpret_cast<const uint16_t*>(a.cache) + (int64_t)b * a.c_b, a.c_t, tid - 256, w, g, c, L,
                oacc, S);
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
  if (a.fp8 && a.Q == 1)
    hipLaunchKernelGGL((decode_mla_ws_kernel<true, kS>), grid, dim3(kWsThreads), 0, st, a);
  else if (a.fp8)
    hipLaunchKernelGGL((decode_mla_ws_kernel<true, kR>), grid, dim3(kWsThreads), 0, st, a);
  else if (a.Q == 1)
    hipLaunchKernelGGL((decode_mla_ws_kernel<false, kS>), grid, dim3(kWsThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mla_ws_kernel<false, kR>), grid, dim3(kWsThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace cpa
