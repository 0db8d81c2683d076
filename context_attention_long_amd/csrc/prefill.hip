// Causal attention of one rank's local queries against their true causal
// history: the prefill shard of context parallelism.
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 2.1 (each rank attends its own queries against the full, gathered K/V),
// 2.3 (zigzag: a run of consecutive queries per block, reads end where the
// block ends; a cached prefix is read by both blocks), 2.4 (interleave: the
// rank's queries are C positions apart, each with its own causal extent);
// SGLang "Prefill context parallelism" docs, zigzag / interleave metadata.
// A query at position p reads keys 0..p of its request, diagonal included
// (1.1). GQA: query head h reads kv head h / (Hq / Hkv).
//
// Work decomposition (gfx950): one workgroup of 4 wavefronts covers 128
// (query, head) rows that share one kv head -- 128/G consecutive local rows
// of one segment times the G query heads of the group -- so every K/V tile
// staged in LDS feeds all 128 rows. Each wavefront owns 32 rows.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read
//    from the row-major K tile, B = Q^T held in registers; every lane then
//    holds 32 key scores of a single row, so the row max / sum need one
//    cross-lane step (lanes l and l^32).
//  * O^T += V^T P^T: B = P^T is the score registers converted to bf16 (the
//    16 keys of a k-step are ordered to match the score layout), A = V^T is
//    read from the row-major V tile with ds_read_b64_tr_b16.
//  * The causal mask is evaluated only on tiles that straddle a row's
//    position; tiles past a wavefront's last row are skipped.
//  * Segments (at most kMaxSeg per launch) travel in the kernel arguments;
//    the host orders them by decreasing cost and each segment's tiles run
//    from the most expensive (last rows) down, so the longest work units are
//    dispatched first. The kv head is the fastest-varying block index, so
//    with 8 kv heads each XCD (blockIdx % 8) keeps one head's K/V in its L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <vector>

#include "internal.h"
#include "lds_dma.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;              // head dim (QK and PV)
constexpr int kBN = 64;              // keys per tile
constexpr int kRows = 128;           // (query, head) rows per workgroup
constexpr int kThreads = 256;
constexpr int kRowBytes = kD * 2;    // 256 B = 16 chunks of 16 B
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KB (K or V)
constexpr int kLdPerThread = 2 * kTileBytes / 16 / kThreads;  // 8 chunks (K and V)
constexpr int kMaxSeg = 64;
constexpr float kLn2 = 0.69314718055994531f;

struct Seg {
  int32_t q_row0, q_len, pos0, pos_stride;
  int64_t kv_row0;
  int32_t tile_begin, n_tiles;  // this segment's range of work indices
};

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  float* lse;
  int64_t q_n, q_h, k_t, k_h, v_t, v_h, o_n, o_h, l_n, l_h;
  int32_t Hkv, G, QT, n_seg, out_bf16;
  float scale_log2;
  Seg seg[kMaxSeg];
};

// Physical chunk of logical 16-byte chunk c in tile row r (256-byte rows,
// XOR over the row's 16 chunks). f is linear in the row's low 4 bits; it
// keeps both operand reads at the full gfx950 LDS rate (64 banks x 4 B):
// the 16-byte K reads (32 rows x 2 chunks) and the 8-byte transposing V
// reads (4 rows x 2 chunk halves per 16 lanes). The rates of these exact
// patterns were measured; a plain bit permutation of the row index left the
// V reads at half rate.
__device__ __forceinline__ int swz(int r, int c) {
  const int f = ((r & 1) ? 14 : 0) ^ ((r & 2) ? 9 : 0) ^ ((r & 4) ? 8 : 0) ^ ((r & 8) ? 2 : 0);
  return c ^ f;
}

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) char*)(p));
}

// Operand vectors are assembled only from whole registers: packed pairs and
// whole-vector bit casts. (Building a bf16 vector one element at a time is
// lowered incorrectly by the gfx950 code generator of this toolchain: it
// duplicates or misaligns elements.)
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 (round to nearest even) of a pair, as one 32-bit word: a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]),
                                                 pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])));
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(kThreads, 2) void prefill_gqa_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][kTileBytes];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const int kvh = blockIdx.x % a.Hkv;
  const int wi = blockIdx.x / a.Hkv;

  // ---- which segment and tile this workgroup owns ----
  int sj = 0;
  for (int j = 1; j < a.n_seg; ++j)
    if (wi >= a.seg[j].tile_begin) sj = j;
  const Seg S = a.seg[sj];
  const int tile = S.n_tiles - 1 - (wi - S.tile_begin);  // most expensive first
  const int q_first = tile * a.QT;                       // first local row (segment-relative)
  const int q_count = min(a.QT, S.q_len - q_first);

  // ---- this lane's row: (query qi, head hi) of the workgroup's 128 rows ----
  const int r = wave * 32 + col;
  const int hi = r / a.QT, qi = r % a.QT;
  const bool row_valid = qi < q_count;
  const int qi_c = row_valid ? qi : q_count - 1;  // padded rows recompute the last valid row
  const int64_t q_row = (int64_t)S.q_row0 + q_first + qi_c;
  const int head = kvh * a.G + hi;
  const int pos = S.pos0 + (q_first + qi_c) * S.pos_stride;

  // positions covered by the workgroup and by this wavefront
  const int wg_last_pos = S.pos0 + (q_first + q_count - 1) * S.pos_stride;
  int w_first, w_last;
  {
    // rows of wave w: r in [32w, 32w+32): queries (r % QT) clamped to q_count
    const int r0 = wave * 32, r1 = wave * 32 + 31;
    int qlo, qhi;
    if (a.QT >= 32) {
      qlo = min(r0 % a.QT, q_count - 1);
      qhi = min(r1 % a.QT, q_count - 1);
    } else {  // the wave spans several heads and so every query of the tile
      qlo = 0;
      qhi = q_count - 1;
    }
    w_first = S.pos0 + (q_first + qlo) * S.pos_stride;
    w_last = S.pos0 + (q_first + qhi) * S.pos_stride;
  }
  const int n_tiles = wg_last_pos / kBN + 1;

  // ---- Q^T operand: row r, dims 16s + 8g .. +8 ----
  // (made opaque once loaded, so the wait for these loads happens here:
  // deferred into the tile loop, the compiler's vmcnt count -- blind to the
  // tile loads issued from inline assembly -- would also wait for those)
  bf16x8 qreg[kD / 16];
  {
    const uint16_t* qp = a.q + q_row * a.q_n + (int64_t)head * a.q_h + 8 * g;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) asm volatile("" : "+v"(qreg[s]));
  }

  // ---- K/V tile loader: direct global -> LDS, 16 bytes per lane ----
  // Wave w's k-th load writes LDS chunks [64w + 256k, +64) of the stage's
  // [K 1024 | V 1024] chunks; each lane fetches the logical chunk that the
  // swizzle puts at its position. Keys past the workgroup's last position
  // re-read that last row (finite data; their scores are masked).
  const uint16_t* kbase = a.k + S.kv_row0 * a.k_t + (int64_t)kvh * a.k_h;
  const uint16_t* vbase = a.v + S.kv_row0 * a.v_t + (int64_t)kvh * a.v_h;
  const int64_t k_t = a.k_t, v_t = a.v_t;
  // loop-invariant byte offsets of this thread's 8 chunks inside a tile
  uint32_t toff[kLdPerThread];
#pragma unroll
  for (int k = 0; k < kLdPerThread; ++k) {
    const int P = tid + kThreads * k;  // chunk P of [K 1024 | V 1024]: K for k < 4
    const int rr = (P >> 4) & (kBN - 1);
    toff[k] = (uint32_t)((rr * (k < kLdPerThread / 2 ? k_t : v_t) + swz(rr, P & 15) * 8) * 2);
  }
  auto load = [&](int kt, int st) {
    const int kb = kt * kBN;
    char* dst0 = &lds[st][0][0] + 64 * wave * 16;
    if (kb + kBN - 1 <= wg_last_pos) {
      // full tile: uniform bases, per-lane offsets fixed
      const uint16_t* kt_base = kbase + (int64_t)kb * k_t;
      const uint16_t* vt_base = vbase + (int64_t)kb * v_t;
#pragma unroll
      for (int k = 0; k < kLdPerThread; ++k)
        cpa::lds_dma16_sbase(k < kLdPerThread / 2 ? kt_base : vt_base, toff[k],
                             cpa::lds_addr(dst0 + kThreads * k * 16));
    } else {
      // last tile: keys past the workgroup's last position re-read that row
#pragma unroll
      for (int k = 0; k < kLdPerThread; ++k) {
        const int P = tid + kThreads * k;
        const int rr = (P >> 4) & (kBN - 1);
        const int64_t kp = min(kb + rr, wg_last_pos);
        const uint16_t* src = (k < kLdPerThread / 2 ? kbase + kp * k_t : vbase + kp * v_t) + swz(rr, P & 15) * 8;
        cpa::lds_dma16(src, cpa::lds_addr(dst0 + kThreads * k * 16));
      }
    }
  };

  // ---- per-lane LDS offsets (tile-relative) ----
  // QK A operand: key row 32mt + col, chunk 2s + g  -> base per (mt, s&7 pattern)
  int qk_off[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int rr = 32 * mt + col;
#pragma unroll
    for (int s = 0; s < 8; ++s) qk_off[mt][s] = rr * kRowBytes + swz(rr, 2 * s + g) * 16;
  }
  // PV A operand (transposing read): 16-lane group q = lane/16; rows
  // 16ks + 4(q/2) + (lane%16)/4 (+8), columns 32mtv + 16(q%2) + 4(lane%4)
  const int lq = lane >> 4, ls = lane & 15;
  int pv_off[2][4];  // [key run][mtv] for k-step 0; k-step ks adds 16 rows
#pragma unroll
  for (int run = 0; run < 2; ++run)
#pragma unroll
    for (int mtv = 0; mtv < 4; ++mtv) {
      const int rr = 4 * (lq >> 1) + (ls >> 2) + 8 * run;
      const int cidx = 32 * mtv + 16 * (lq & 1) + 4 * (ls & 3);  // element column
      pv_off[run][mtv] = rr * kRowBytes + swz(rr, cidx >> 3) * 16 + (cidx & 7) * 2;
    }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // one tile; ST (the LDS stage) is a compile-time constant so every operand
  // read is a per-lane base plus an immediate offset
  auto compute = [&](int kt, auto stage) {
    constexpr int ST = decltype(stage)::value;
    const int kb = kt * kBN;
    if (kb > w_last) return;  // every row of this wave is past: skip (wave-uniform)
    const char* Kt = &lds[ST][0][0];
    const char* Vt = &lds[ST][1][0];

    // ---- S^T = K Q^T ----
    // (the two key blocks alternate, and each K operand is read two k-steps
    // ahead, so an LDS read has four MFMAs to land)
    constexpr int kAhead = 2;
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    bf16x8 ka[kD / 16][2];
#pragma unroll
    for (int s = 0; s < kAhead; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) ka[s][mt] = *reinterpret_cast<const bf16x8*>(Kt + qk_off[mt][s]);
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) {
      if (s + kAhead < kD / 16) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          ka[s + kAhead][mt] = *reinterpret_cast<const bf16x8*>(Kt + qk_off[mt][s + kAhead]);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s][mt], qreg[s], sacc[mt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- mask (only tiles that reach past the wave's first row), max ----
    // The running max is kept in the scaled log2 domain; the max is taken over
    // raw scores (the scale is positive) and p = 2^(s * c - m) is one FMA and
    // one v_exp_f32 (results below 2^-126 flush to 0, which only drops terms
    // smaller than the fp32 sum can hold).
    if (kb + kBN - 1 > w_first) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
          sacc[mt][i] = key <= pos ? sacc[mt][i] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescale: the reference max m_run moves only when the tile's max
    // exceeds it by more than 2^8 (then p <= 256 until the next move; O and l
    // share the reference, so the result is unchanged). Key 0 is in the first
    // tile of every row, so m_run is finite from then on.
    const float mt = mx * a.scale_log2;
    if (__any(mt > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
    }
    const float m_new = m_run;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[ks >> 1][8 * (ks & 1) + j], a.scale_log2, -m_new));
        psum += p;
        pf[j] = p;
      }
      pb[ks] = pack8(pf);
    }
    l_run += psum;
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mtv = 0; mtv < 4; ++mtv) {
        const i16x4 v0 = lds_read_tr(Vt + pv_off[0][mtv] + 16 * ks * kRowBytes);
        const i16x4 v1 = lds_read_tr(Vt + pv_off[1][mtv] + 16 * ks * kRowBytes);
        const bf16x8 va = join_tr(v0, v1);
        oacc[mtv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], oacc[mtv], 0, 0, 0);
      }
    }
  };

  load(0, 0);
  for (int kt = 0; kt < n_tiles; kt += 2) {
    cpa::wait_vmcnt<0>();  // this thread's part of tile kt landed
    __syncthreads();       // tile kt complete in LDS; every wave is done with stage 1
    if (kt + 1 < n_tiles) load(kt + 1, 1);
    compute(kt, std::integral_constant<int, 0>{});
    if (kt + 1 >= n_tiles) break;
    cpa::wait_vmcnt<0>();
    __syncthreads();       // tile kt + 1 complete; every wave is done with stage 0
    if (kt + 2 < n_tiles) load(kt + 2, 0);
    compute(kt + 1, std::integral_constant<int, 1>{});
  }

  // ---- finish ----
  float l = l_run + __shfl_xor(l_run, 32);
  if (!row_valid) return;
  const float inv = 1.f / l;
  if (a.out_bf16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + q_row * a.o_n + (int64_t)head * a.o_h;
#pragma unroll
    for (int mtv = 0; mtv < 4; ++mtv)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dv = 32 * mtv + 8 * i4 + 4 * g;
        uint2 pk;
        pk.x = (uint32_t)bf16_rne(oacc[mtv][4 * i4 + 0] * inv) | ((uint32_t)bf16_rne(oacc[mtv][4 * i4 + 1] * inv) << 16);
        pk.y = (uint32_t)bf16_rne(oacc[mtv][4 * i4 + 2] * inv) | ((uint32_t)bf16_rne(oacc[mtv][4 * i4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + dv) = pk;
      }
  } else {
    float* op = reinterpret_cast<float*>(a.out) + q_row * a.o_n + (int64_t)head * a.o_h;
#pragma unroll
    for (int mtv = 0; mtv < 4; ++mtv)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dv = 32 * mtv + 8 * i4 + 4 * g;
        float4 v;
        v.x = oacc[mtv][4 * i4 + 0] * inv;
        v.y = oacc[mtv][4 * i4 + 1] * inv;
        v.z = oacc[mtv][4 * i4 + 2] * inv;
        v.w = oacc[mtv][4 * i4 + 3] * inv;
        *reinterpret_cast<float4*>(op + dv) = v;
      }
  }
  if (g == 0) a.lse[q_row * a.l_n + (int64_t)head * a.l_h] = (m_run + log2f(l)) * kLn2;
}

}  // namespace

namespace cpa {

// Validated GQA launch (d = 128): segments are already checked by the caller.
int launch_prefill_gqa(const PrefillGqaArgs& in, const cpa_segment* seg, int n_seg, void* stream) {
  // cost of a segment = keys read by its last row
  std::vector<int> order;
  for (int i = 0; i < n_seg; ++i)
    if (seg[i].q_len > 0) order.push_back(i);
  auto last_pos = [&](int i) { return (int64_t)seg[i].pos0 + (int64_t)(seg[i].q_len - 1) * seg[i].pos_stride; };
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return last_pos(x) > last_pos(y); });
  const int QT = kRows / in.G;
  for (size_t base = 0; base < order.size(); base += kMaxSeg) {
    Args a{};
    a.q = in.q;
    a.k = in.k;
    a.v = in.v;
    a.out = in.out;
    a.lse = in.lse;
    a.q_n = in.q_n, a.q_h = in.q_h, a.k_t = in.k_t, a.k_h = in.k_h, a.v_t = in.v_t, a.v_h = in.v_h;
    a.o_n = in.o_n, a.o_h = in.o_h, a.l_n = in.l_n, a.l_h = in.l_h;
    a.Hkv = in.Hkv;
    a.G = in.G;
    a.QT = QT;
    a.out_bf16 = in.out_bf16;
    a.scale_log2 = in.scale_log2;
    int ns = 0, tiles = 0;
    for (size_t j = base; j < order.size() && ns < kMaxSeg; ++j, ++ns) {
      const cpa_segment& s = seg[order[j]];
      Seg& d = a.seg[ns];
      d.q_row0 = s.q_row0;
      d.q_len = s.q_len;
      d.pos0 = s.pos0;
      d.pos_stride = s.pos_stride;
      d.kv_row0 = s.kv_row0;
      d.tile_begin = tiles;
      d.n_tiles = (s.q_len + QT - 1) / QT;
      tiles += d.n_tiles;
    }
    a.n_seg = ns;
    const int64_t blocks = (int64_t)tiles * in.Hkv;
    if (blocks == 0) continue;
    hipLaunchKernelGGL(prefill_gqa_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cpa
