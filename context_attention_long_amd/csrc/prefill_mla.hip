// Causal prefill-shard attention over an MLA latent cache: 64 query heads
// share one 576-dim latent per token; QK runs over all 576 dims and PV over
// the first 512 (vLLM GLM-5.3 post, footnote 1; "How GPUs Share a Long
// Context During LLM Inference", 1.3). A query at position p (cached prefix
// included) reads keys 0..p of its request (same article, 1.1, 2.3).
//
// One workgroup per local query row: its 64 heads over the contiguous key
// range [0, p] run through the shared MLA core (mla_core.h), the same tile
// pipeline as split-KV decode, with the default cache policy (neighbouring
// rows read the same latent tiles at about the same time, mostly from L2).
// Rows are launched most expensive first. The causal mask is the end of the
// range: only the last tile holds keys past p, and those are masked.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "internal.h"
#include "mla_core.h"
#include "mla_ws.h"

namespace {

using namespace cpa::mla;

constexpr int kMaxSeg = 64;

struct Seg {
  int32_t q_row0, q_len, pos0, pos_stride;
  int64_t kv_row0;
  int32_t tile_begin, n_tiles;
};

struct Args {
  const uint16_t* q;     // [n_local, 64, 576]
  const uint16_t* lat;   // [T_kv, 1, 576]
  void* out;             // [n_local, 64, 512]
  float* lse;            // [n_local, 64]
  int64_t q_n, q_h, k_t, o_n, o_h, l_n, l_h;
  int32_t n_seg, out_bf16;
  float scale_log2;
  Seg seg[kMaxSeg];
};

// One workgroup per query row on the wave-specialised core (mla_ws.h): 4
// QK + 4 PV wavefronts.
__global__ __launch_bounds__(kWsThreads, 1) void prefill_mla_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __shared__ __attribute__((aligned(16))) char plds[2 * kH * kPRowBytes];
  __shared__ float alpha_s[2 * kH], lsum_s[kH];
  const Lds S{smem, plds, alpha_s, lsum_s};

  const int tid = threadIdx.x;
  const int w = (tid >> 6) & 3, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const bool qk_role = tid < 256;

  // ---- the query row of this workgroup (most expensive first) ----
  const int wi = blockIdx.x;
  int sj = 0;
  for (int j = 1; j < a.n_seg; ++j)
    if (wi >= a.seg[j].tile_begin) sj = j;
  const Seg Sg = a.seg[sj];
  const int qi = Sg.q_len - 1 - (wi - Sg.tile_begin);
  const int64_t q_row = (int64_t)Sg.q_row0 + qi;
  const int pos = Sg.pos0 + qi * Sg.pos_stride;
  const Tiles T(0, (int64_t)pos + 1, 0u);
  const LdsBases L = lds_bases(w, g, c);

  if (qk_role) {
    bf16x8 qreg[kQSteps];
    load_q(a.q + q_row * a.q_n + (int64_t)(16 * w + c) * a.q_h, g, qreg);
    QkStat st{-INFINITY, 0.f};
    ws_qk(T, w, g, c, L, qreg, a.scale_log2, st, S, [&](int i) { return ws_tile(S, i); },
          [](int) { return 0xffffffffu; });
    const float l = sum4_rows(st.l_run);
    if (g == 0) S.lsum[16 * w + c] = l;
    __syncthreads();
    if (g == 0) a.lse[q_row * a.l_n + (int64_t)(16 * w + c) * a.l_h] = (st.m_run + log2f(l)) * kLn2;
  } else {
    f32x4 oacc[kMv][4];
#pragma unroll
    for (int m = 0; m < kMv; ++m)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) oacc[m][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws_pv<cpa::Policy::kReuse>(T, a.lat + Sg.kv_row0 * a.k_t, a.k_t, tid - 256, w, g, c, L, oacc, S);
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = 16 * hb + c;
      const float inv = 1.f / lsum_s[head];  // key 0 is always in range: the sum is >= 1
      const int64_t o0 = q_row * a.o_n + (int64_t)head * a.o_h + 128 * w + 4 * g;
#pragma unroll
      for (int m = 0; m < kMv; ++m) {
        const f32x4 o = oacc[m][hb] * inv;
        if (a.out_bf16)
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o0 + 16 * m) =
              make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
        else
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o0 + 16 * m) = o;
      }
    }
  }
}

}  // namespace

namespace cpa {

int launch_prefill_mla(const PrefillMlaArgs& in, const cpa_segment* seg, int n_seg, void* stream) {
  std::vector<int> order;
  for (int i = 0; i < n_seg; ++i)
    if (seg[i].q_len > 0) order.push_back(i);
  auto last_pos = [&](int i) { return (int64_t)seg[i].pos0 + (int64_t)(seg[i].q_len - 1) * seg[i].pos_stride; };
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return last_pos(x) > last_pos(y); });
  for (size_t base = 0; base < order.size(); base += kMaxSeg) {
    Args a{};
    a.q = in.q;
    a.lat = in.lat;
    a.out = in.out;
    a.lse = in.lse;
    a.q_n = in.q_n, a.q_h = in.q_h, a.k_t = in.k_t;
    a.o_n = in.o_n, a.o_h = in.o_h, a.l_n = in.l_n, a.l_h = in.l_h;
    a.out_bf16 = in.out_bf16;
    a.scale_log2 = in.scale_log2;
    int ns = 0, rows = 0;
    for (size_t j = base; j < order.size() && ns < kMaxSeg; ++j, ++ns) {
      const cpa_segment& s = seg[order[j]];
      Seg& d = a.seg[ns];
      d.q_row0 = s.q_row0;
      d.q_len = s.q_len;
      d.pos0 = s.pos0;
      d.pos_stride = s.pos_stride;
      d.kv_row0 = s.kv_row0;
      d.tile_begin = rows;
      d.n_tiles = s.q_len;
      rows += s.q_len;
    }
    a.n_seg = ns;
    if (rows == 0) continue;
    hipLaunchKernelGGL(prefill_mla_kernel, dim3((unsigned)rows), dim3(kWsThreads), 0, (hipStream_t)stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cpa
