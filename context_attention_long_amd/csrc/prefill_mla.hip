// Causal prefill-shard attention over an MLA latent cache: 64 query heads
// share one 576-dim latent per token; QK runs over all 576 dims and PV over
// the first 512 (vLLM GLM-5.3 post, footnote 1; "How GPUs Share a Long
// Context During LLM Inference", 1.3). A query at position p (cached prefix
// included) reads keys 0..p of its request (same article, 1.1, 2.3).
//
// Work decomposition (gfx950): one workgroup per local query row and its 64
// heads; rows of the attention problem are the heads. A 64-key latent tile
// (72 KB) is staged in LDS by direct global->LDS loads, double buffered.
// The four wavefronts split the work two ways:
//  * QK: wave w computes S^T for key half (w & 1) x head half (w >> 1) with
//    v_mfma_f32_32x32x16_bf16 (36 k-steps over 576 dims; Q^T for its 32
//    heads stays in registers). Row maxima of the two key halves meet in
//    LDS; each wave then writes its probabilities P (bf16) to LDS, already in
//    the order the PV operand wants, and the per-head rescale factor.
//  * PV: wave w accumulates O^T for dims [128w, 128w+128) of all 64 heads,
//    A = V^T read from the same latent tile with ds_read_b64_tr_b16, B = P^T
//    from LDS; its accumulator is rescaled lane-locally (lane = head).
// Only the tile holding the query's own position is masked.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "internal.h"
#include "lds_dma.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kH = 64;
constexpr int kDk = 576, kDv = 512;
constexpr int kBN = 64;                          // keys per tile
constexpr int kThreads = 256;
constexpr int kRowChunks = kDk / 8;              // 72 chunks of 16 B per latent row
constexpr int kRowBytes = kDk * 2;               // 1152
constexpr int kTileBytes = kBN * kRowBytes;      // 73728
constexpr int kLdPerThread = kBN * kRowChunks / kThreads;  // 18
constexpr int kPRowBytes = 144;                  // P row: 8 chunks + 1 pad chunk
constexpr int kMaxSeg = 64;
constexpr float kLn2 = 0.69314718055994531f;

static_assert(kBN * kRowChunks % kThreads == 0, "tile must split evenly over the threads");

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

// Physical 16-byte chunk of logical chunk c in latent row r: the low 3 chunk
// bits XOR f(r), f = row bits (b2, b3, b1), a function of r mod 16 so that
// rows 16 apart share offsets (immediate addressing). On gfx950's LDS
// (64 banks x 4 B, 1152-byte rows alternate bank halves) this keeps the
// 16-byte QK reads (32 rows x 2 chunks) and the 8-byte transposing V reads
// (4 rows x 2 chunk halves per 16 lanes) at the full read rate; the rates of
// these patterns were measured.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r & 2) << 1) | ((r & 4) >> 2) | ((r & 8) >> 2)); }

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) char*)(p));
}

// Operand vectors are assembled only from whole registers (packed pairs,
// whole-vector casts): element-wise bf16 vector construction is lowered
// incorrectly by this toolchain's gfx950 code generator.
__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
}

__global__ __launch_bounds__(kThreads, 1) void prefill_mla_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char tiles[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) char plds[kH * kPRowBytes];
  __shared__ float red_max[2][kH];
  __shared__ float alpha_s[kH];
  __shared__ float lsum[2][kH];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const int kh = wave & 1, rh = wave >> 1;  // QK role
  const int dq = wave;                      // PV role: dims [128 dq, +128)

  // ---- the query row of this workgroup (most expensive first) ----
  const int wi = blockIdx.x;
  int sj = 0;
  for (int j = 1; j < a.n_seg; ++j)
    if (wi >= a.seg[j].tile_begin) sj = j;
  const Seg S = a.seg[sj];
  const int qi = S.q_len - 1 - (wi - S.tile_begin);
  const int64_t q_row = (int64_t)S.q_row0 + qi;
  const int pos = S.pos0 + qi * S.pos_stride;
  const int n_tiles = pos / kBN + 1;

  // ---- Q^T operand (QK role): head 32 rh + col, dims 16 s + 8 g .. +8 ----
  const int qk_head = 32 * rh + col;
  bf16x8 qreg[kDk / 16];
  {
    const uint16_t* qp = a.q + q_row * a.q_n + (int64_t)qk_head * a.q_h + 8 * g;
#pragma unroll
    for (int s = 0; s < kDk / 16; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  // ---- loader: wave w's k-th load fills LDS chunks [64 w + 256 k, +64) ----
  const uint16_t* lbase = a.lat + S.kv_row0 * a.k_t;
  auto load = [&](int kt, int st) {
    const int kb = kt * kBN;
#pragma unroll
    for (int k = 0; k < kLdPerThread; ++k) {
      const int P = tid + kThreads * k;
      const int rr = P / kRowChunks, pc = P % kRowChunks;
      const int kp = min(kb + rr, pos);  // past the query: re-read its own row (masked)
      const uint16_t* src = lbase + (int64_t)kp * a.k_t + swz(rr, pc) * 8;
      char* dst = tiles[st] + (64 * wave + kThreads * k) * 16;
      cpa::lds_dma16(src, cpa::lds_addr(dst));
    }
  };

  // ---- per-lane LDS offsets ----
  // QK A operand: key row 32 kh + col, logical chunk 2 s + g = 8 (s >> 2) + (2 (s & 3) + g)
  int qk_off[4];
  {
    const int rr = 32 * kh + col;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qk_off[s4] = rr * kRowBytes + swz(rr, 2 * s4 + g) * 16;
  }
  // PV A operand (transposing read): 16-lane group lq, lane ls: key row
  // 16 ks + 4 (lq >> 1) + (ls >> 2) (+ 8), dims 128 dq + 32 mtv + 16 (lq & 1) + 4 (ls & 3)
  const int lq = lane >> 4, ls = lane & 15;
  int pv_off[2][2];  // [run][mtv & 1]; k-step ks adds 16 rows, (mtv >> 1) adds 64 dims = 128 B
#pragma unroll
  for (int run = 0; run < 2; ++run)
#pragma unroll
    for (int m1 = 0; m1 < 2; ++m1) {
      const int rr = 4 * (lq >> 1) + (ls >> 2) + 8 * run;
      const int cidx = 128 * dq + 32 * m1 + 16 * (lq & 1) + 4 * (ls & 3);
      pv_off[run][m1] = rr * kRowBytes + swz(rr, cidx >> 3) * 16 + (cidx & 7) * 2;
    }

  f32x16 oacc[4][2];  // [mtv][head block nt]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    oacc[i][0] = f32x16{};
    oacc[i][1] = f32x16{};
  }
  float m_run = -INFINITY;  // QK role: running max of head qk_head (log2 domain)
  float l_part = 0.f;       // QK role: this lane's share of the head's sum

  load(0, 0);
  for (int kt = 0; kt < n_tiles; ++kt) {
    cpa::wait_vmcnt<0>();  // this thread's part of tile kt landed
    __syncthreads();  // tile kt in LDS; PV of tile kt-1 finished everywhere
    const int st = kt & 1;
    if (kt + 1 < n_tiles) load(kt + 1, st ^ 1);
    const char* T = tiles[st];
    const int kb = kt * kBN;

    // ---- QK: S^T [32 keys of half kh][32 heads of half rh] ----
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < kDk / 16; ++s) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(T + qk_off[s & 3] + 128 * (s >> 2));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], sacc, 0, 0, 0);
    }
    if (kb + kBN - 1 > pos) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + 32 * kh + 8 * (i >> 2) + 4 * g + (i & 3);
        sacc[i] = key <= pos ? sacc[i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (g == 0) red_max[kh][qk_head] = mx;
    __syncthreads();
    // reference max in the scaled log2 domain, moved lazily (only when the
    // tile's max exceeds it by more than 2^8; O and l share it, so the result
    // is unchanged); p = 2^(s * c - m): one FMA + v_exp_f32. Key 0 is in tile
    // 0, so the reference is finite from then on.
    const float mt = fmaxf(red_max[0][qk_head], red_max[1][qk_head]) * a.scale_log2;
    float alpha = 1.f;
    if (mt > m_run + 8.f) {
      alpha = __builtin_amdgcn_exp2f(m_run - mt);
      m_run = mt;
    }
    const float m_new = m_run;
    float psum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[i], a.scale_log2, -m_new));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[i + 1], a.scale_log2, -m_new));
      psum += p0 + p1;
      pk[i >> 1] = pack_bf16(p0, p1);
    }
    l_part = l_part * alpha + psum;
    // P^T for k-steps ks = 2 kh + a: the lane's values i = 8a .. 8a+7 (head, group g)
    char* prow = plds + qk_head * kPRowBytes;
    *reinterpret_cast<uint4*>(prow + ((2 * kh + 0) * 2 + g) * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    *reinterpret_cast<uint4*>(prow + ((2 * kh + 1) * 2 + g) * 16) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    if (kh == 0 && g == 0) alpha_s[qk_head] = alpha;
    __syncthreads();

    // ---- PV: O^T [dims of quarter dq][64 heads] ----
    const float al0 = alpha_s[col], al1 = alpha_s[32 + col];
    if (__any(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        oacc[i][0] *= al0;
        oacc[i][1] *= al1;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 pb0 = *reinterpret_cast<const bf16x8*>(plds + col * kPRowBytes + (2 * ks + g) * 16);
      const bf16x8 pb1 = *reinterpret_cast<const bf16x8*>(plds + (32 + col) * kPRowBytes + (2 * ks + g) * 16);
#pragma unroll
      for (int mtv = 0; mtv < 4; ++mtv) {
        const i16x4 v0 = lds_read_tr(T + pv_off[0][mtv & 1] + 16 * ks * kRowBytes + 128 * (mtv >> 1));
        const i16x4 v1 = lds_read_tr(T + pv_off[1][mtv & 1] + 16 * ks * kRowBytes + 128 * (mtv >> 1));
        const bf16x8 va = join_tr(v0, v1);
        oacc[mtv][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb0, oacc[mtv][0], 0, 0, 0);
        oacc[mtv][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb1, oacc[mtv][1], 0, 0, 0);
      }
    }
  }

  // ---- finish: total sum per head, normalise, store ----
  const float lp = l_part + __shfl_xor(l_part, 32);
  if (g == 0) lsum[kh][qk_head] = lp;
  __syncthreads();
  if (kh == 0 && g == 0) {
    const float l = lsum[0][qk_head] + lsum[1][qk_head];
    a.lse[q_row * a.l_n + (int64_t)qk_head * a.l_h] = (m_run + log2f(l)) * kLn2;
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int head = 32 * nt + col;
    const float inv = 1.f / (lsum[0][head] + lsum[1][head]);
#pragma unroll
    for (int mtv = 0; mtv < 4; ++mtv)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dv = 128 * dq + 32 * mtv + 8 * i4 + 4 * g;
        const f32x16& o = oacc[mtv][nt];
        if (a.out_bf16) {
          uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + q_row * a.o_n + (int64_t)head * a.o_h + dv;
          *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16(o[4 * i4] * inv, o[4 * i4 + 1] * inv),
                                                     pack_bf16(o[4 * i4 + 2] * inv, o[4 * i4 + 3] * inv));
        } else {
          float* op = reinterpret_cast<float*>(a.out) + q_row * a.o_n + (int64_t)head * a.o_h + dv;
          *reinterpret_cast<float4*>(op) =
              make_float4(o[4 * i4] * inv, o[4 * i4 + 1] * inv, o[4 * i4 + 2] * inv, o[4 * i4 + 3] * inv);
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
    hipLaunchKernelGGL(prefill_mla_kernel, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cpa
