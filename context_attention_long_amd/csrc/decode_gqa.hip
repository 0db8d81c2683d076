// Split-KV decode for GQA caches (f32 or bf16), one query per request.
//
// "How GPUs Share a Long Context During LLM Inference", 3.2-3.4: a rank runs
// attention of each request's single new query over its own share of the
// cache and reports the partial output with its LSE; vLLM "Decode Context
// Parallelism", 4.1 and 5.4: the GQA kv heads are broadcast to their query
// heads. Query head h reads kv head h / (Hq / Hkv).
//
// One workgroup per (query row, kv head, split): the G query heads of the
// group share every K/V tile staged in LDS. A request has Q >= 1 query rows
// (speculative / MTP decode), each with its own end of range. Scores, the running max / sum
// and the output accumulators are fp32; the running statistics are kept in
// the log2 domain (scores pre-multiplied by scale * log2 e) and converted
// back to a natural-log LSE at the end. A split covers an even share of the
// request's [begin, end) range, so any range length is processed in full.
//
// This kernel is the general GQA path (small workloads, f32 parity cases);
// the MLA latent cache has its own MFMA kernel.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;  // tokens per LDS tile

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <bool kBf16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (kBf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <bool kQBf16, bool kKvBf16>
__global__ __launch_bounds__(kThreads) void decode_gqa_kernel(cpa::DecodeGqaArgs a) {
  extern __shared__ float smem[];
  const int D = a.D, G = a.Hq / a.Hkv, Dp = a.D + 1;  // padded LDS row
  float* qs = smem;                  // [G][D]
  float* ks = qs + G * D;            // [kTile][Dp]
  float* vs = ks + kTile * Dp;       // [kTile][Dp]
  float* ps = vs + kTile * Dp;       // [G][kTile]
  float* alpha_s = ps + G * kTile;   // [G]
  float* m_s = alpha_s + G;          // [G]
  float* l_s = m_s + G;              // [G]

  const int split = blockIdx.x % a.nsplit;
  const int kvh = (blockIdx.x / a.nsplit) % a.Hkv;
  const int row = blockIdx.x / (a.nsplit * a.Hkv);  // output row: query row k of request b
  const int b = row / a.Q, k = row % a.Q;
  const int tid = threadIdx.x;

  int64_t beg = a.kv_begin[b], end = a.kv_end[row];
  beg = beg < 0 ? 0 : (beg > a.Lmax ? a.Lmax : beg);
  end = end < beg ? beg : (end > a.Lmax ? a.Lmax : end);
  const int64_t len = end - beg;
  const int64_t t0 = beg + len * split / a.nsplit;
  const int64_t t1 = beg + len * (split + 1) / a.nsplit;

  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    qs[i] = load_elem<kQBf16>(a.q, b * a.q_b + k * a.q_q + (int64_t)(kvh * G + g) * a.q_h + d);
  }
  for (int g = tid; g < G; g += kThreads) {
    m_s[g] = -INFINITY;
    l_s[g] = 0.f;
  }
  // output accumulators: element e = tid + kThreads * i of the [G][D] block
  constexpr int kMaxAcc = 32;  // G * D <= 8192
  float acc[kMaxAcc];
#pragma unroll
  for (int i = 0; i < kMaxAcc; ++i) acc[i] = 0.f;
  const int n_acc = (G * D + kThreads - 1) / kThreads;

  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  for (int64_t tt = t0; tt < t1; tt += kTile) {
    const int nvalid = (int)((t1 - tt) < kTile ? (t1 - tt) : kTile);
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < kTile * D; i += kThreads) {
      const int t = i / D, d = i % D;
      float kx = 0.f, vx = 0.f;
      if (t < nvalid) {
        const int64_t tok = tt + t;
        kx = load_elem<kKvBf16>(kb, ((int64_t)b * a.k_b + tok * a.k_t + (int64_t)kvh * a.k_h + d));
        vx = load_elem<kKvBf16>(vb, ((int64_t)b * a.v_b + tok * a.v_t + (int64_t)kvh * a.v_h + d));
      }
      ks[t * Dp + d] = kx;
      vs[t * Dp + d] = vx;
    }
    __syncthreads();
    for (int p = tid; p < G * kTile; p += kThreads) {
      const int g = p / kTile, t = p % kTile;
      float s = -INFINITY;
      if (t < nvalid) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot += qs[g * D + d] * ks[t * Dp + d];
        s = dot * a.scale_log2;
      }
      ps[g * kTile + t] = s;
    }
    __syncthreads();
    for (int g = tid; g < G; g += kThreads) {
      float mt = -INFINITY;
      for (int t = 0; t < nvalid; ++t) mt = fmaxf(mt, ps[g * kTile + t]);
      const float m_old = m_s[g];
      const float m_new = fmaxf(m_old, mt);
      const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
      float sum = 0.f;
      for (int t = 0; t < kTile; ++t) {
        const float p = (t < nvalid) ? exp2f(ps[g * kTile + t] - m_new) : 0.f;
        ps[g * kTile + t] = p;
        sum += p;
      }
      l_s[g] = l_s[g] * alpha + sum;
      m_s[g] = m_new;
      alpha_s[g] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxAcc; ++i) {
      const int e = tid + kThreads * i;
      if (i < n_acc && e < G * D) {
        const int g = e / D, d = e % D;
        float x = acc[i] * alpha_s[g];
        for (int t = 0; t < nvalid; ++t) x += ps[g * kTile + t] * vs[t * Dp + d];
        acc[i] = x;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMaxAcc; ++i) {
    const int e = tid + kThreads * i;
    if (i < n_acc && e < G * D) {
      const int g = e / D, d = e % D;
      const float l = l_s[g];
      const int h = kvh * G + g;
      a.o[split * a.o_s + (int64_t)row * a.o_b + (int64_t)h * a.o_h + d] = l > 0.f ? acc[i] / l : 0.f;
    }
  }
  for (int g = tid; g < G; g += kThreads) {
    const float l = l_s[g];
    const int h = kvh * G + g;
    // natural-log LSE from the log2-domain statistics
    a.lse[split * a.l_s + (int64_t)row * a.l_b + (int64_t)h * a.l_h] =
        l > 0.f ? (m_s[g] + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

namespace cpa {

int launch_decode_gqa(const DecodeGqaArgs& a, void* stream) {
  const int G = a.Hq / a.Hkv;
  const size_t smem = sizeof(float) * ((size_t)G * a.D + 2 * (size_t)kTile * (a.D + 1) +
                                       (size_t)G * kTile + 3 * (size_t)G);
  const dim3 grid((unsigned)((int64_t)a.B * a.Q * a.Hkv * a.nsplit));
  hipStream_t st = (hipStream_t)stream;
  auto go = [&](auto kernel) {
    if (smem > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return (int)e;
    }
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), smem, st, a);
    return (int)hipGetLastError();
  };
  if (a.q_bf16 && a.kv_dtype == CPA_BF16) return go(decode_gqa_kernel<true, true>);
  if (a.q_bf16) return go(decode_gqa_kernel<true, false>);
  if (a.kv_dtype == CPA_BF16) return go(decode_gqa_kernel<false, true>);
  return go(decode_gqa_kernel<false, false>);
}

}  // namespace cpa
