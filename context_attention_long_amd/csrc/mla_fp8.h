// FP8 latent cache variant of the wave-specialised MLA core (mla_ws.h).
//
// What it computes: the same online-softmax state as the bf16 core --
// attention of one query's 64 heads over a range of an MLA latent cache,
// QK over the 576 latent dims, PV over the first 512 ("How GPUs Share a Long
// Context During LLM Inference", 1.3; vLLM GLM-5.3 post, footnote 1) -- for
// an OCP E4M3 cache with one fp32 scale per token: entry_t = e4m3_t * scale_t.
// The scale multiplies the score and the probability (s_t = scale_t q.e_t,
// and p_t scale_t multiplies e_t in PV), so the codes enter both products
// unscaled and exactly.
//
// Design (gfx950): both products run on the FP8 matrix cores and the cache
// codes are never converted.
//  * The tile stays FP8 in LDS: direct global -> LDS loads of the raw rows
//    (32 tokens = 18 KB per stage, 8 stages), issued by three of the PV
//    wavefronts. A step consumes 64 tokens (two stages). Its 64 token scales
//    arrive with one direct 4-byte-per-lane load (lane l: token l of the
//    step), issued six steps ahead by the fourth PV wavefront, which issues
//    nothing else: those small loads return late, and loads of one
//    wavefront complete in order, so behind them the row loads of the same
//    wavefront held the cache stream to 3.7 TB/s.
//  * QK: v_mfma_scale_f32_16x16x128_f8f6f4, A = 16 tokens x 128 dims of K
//    straight from LDS, B = the query in E4M3. A bf16 query value is split
//    exactly into two E4M3 values, q 2^e = hi + lo (e: a per-head power of
//    two that puts the head's largest |q| in [128, 256); hi holds 4
//    significant bits and the remainder the next 4, all of a bf16 value for
//    every element within 2^-10 of the head's maximum), so QK = hi.K + lo.K
//    in two FP8 MFMAs: the time of one bf16 MFMA, the bf16 product to fp32
//    rounding. The 64 rope dims are a fifth k-step that holds them twice,
//    against their hi codes in one half and their lo codes in the other,
//    so it takes one MFMA instead of two. 2^-e is folded into the softmax
//    scale.
//  * PV: v_mfma_scale_f32_32x32x64_f8f6f4, A = V^T (32 dims x 64 tokens)
//    from ds_read_b64_tr_b8 (lane c of each 16-lane group receives byte c
//    of the 8 rows its group addresses: one dim, 8 tokens per read), B = the
//    PV weights w_t = p_t scale_t. The weights of a step are scaled by a
//    per-head power of two that puts their maximum in [128, 256) and split
//    into hi + lo E4M3 values (relative error <= 2^-9, as a bf16 weight);
//    the MFMA's E8M0 scale on B undoes the power of two exactly.
//  * A step has two phases, each ended by a barrier. Phase A: the QK
//    wavefronts store the weights of step i-1 (with each head's rescale
//    factor and power of two) into one LDS buffer and run the QK MFMAs of
//    step i, alone on the matrix units, while the PV wavefronts issue the
//    loads of later stages. Phase B: the QK wavefronts turn the scores of
//    step i into weights (VALU work) while the PV wavefronts run the PV
//    MFMAs of step i-1 from the buffer. So the softmax overlaps matrix work
//    instead of following it, and the buffer is written only after every
//    PV wavefront has read it.
//  * A stage is stored unit-major in blocks of 16 rows: the 16 rows of one
//    16-byte unit are 256 contiguous bytes (the two 8-row halves of odd
//    units swapped). Each 16-lane group of a QK operand read then reads 256
//    contiguous bytes and each transposing V read 2 x 128 bytes in opposite
//    bank halves -- conflict-free, where a row-major layout of the 576-byte
//    rows cost two cycles per 16-byte read whatever the XOR swizzle (LDS
//    bank-conflict counter). The direct loads fill the stage 1 KB at a
//    time, each lane fetching the row unit its slot holds. The weight rows
//    are XOR-swizzled in 16-byte chunks.
#pragma once

#include <hip/hip_runtime.h>

#include "mla_core.h"
#include "mla_ws.h"

namespace cpa {
namespace mla {
namespace f8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowBytes = kDk;                   // 576 one-byte codes per token
constexpr int kRowUnits = kRowBytes / 16;        // 36 units of 16 bytes
constexpr int kTileUnits = kBN * kRowUnits;      // 1152 per 32-token stage
constexpr int kTileBytes = kTileUnits * 16;      // 18432
constexpr int kStages = 8;
constexpr int kScaleSlot = 256;                  // 64 token scales of a step (one 4-byte load per lane)
constexpr int kScaleSlots = 8;                   // steps of scales in LDS
constexpr int kScaleAhead = 6;                   // steps between a scale load and its use
constexpr int kUnitLoads = 6;                    // row loads per stage and thread of PV wavefronts 0-2
constexpr int kLoaders = 3 * 64;                 // threads that load rows
constexpr int kStepTok = 2 * kBN;                // 64 tokens per step
constexpr int kQSteps8 = 4;                      // QK k-steps of 128 dims over dims 0..511
constexpr int kWBytes = 2 * kH * kStepTok;       // hi and lo weight codes of a step: 8 KB
constexpr int kPvM = 4;                          // PV m-tiles of 32 dims per wavefront (128 dims)

static_assert(kTileUnits == kUnitLoads * kLoaders, "unit split over the loading threads");
static_assert(kScaleAhead < kScaleSlots, "a scale slot is reloaded only after its step");
static_assert(kRowUnits % 4 == 0, "swizzle groups of four units");

struct Lds {
  char* tiles;   // kStages x kTileBytes
  char* scales;  // kScaleSlots x kScaleSlot: f32 token scales of a step (token 32 kg + r at 32 kg + r)
  char* w;       // kWBytes: [hi, lo][64 heads][64 tokens] weight codes of one step
  float* alpha;  // [64] rescale factor of each head for the step
  int* wexp;     // [64] E8M0 code undoing each head's weight scaling
  float* lsum;   // [64]
};

// 16-byte slot of unit u (0..35) of stage row r (0..31), and its inverse.
__device__ __forceinline__ int slot(int r, int u) {
  return (r >> 4) * (16 * kRowUnits) + 16 * u + ((((r >> 3) ^ u) & 1) << 3) + (r & 7);
}
__device__ __forceinline__ void slot_ru(int p, int& r, int& u) {
  const int q = p % (16 * kRowUnits), i = q & 15;
  u = q >> 4;
  r = 16 * (p / (16 * kRowUnits)) + ((((i >> 3) ^ u) & 1) << 3) + (i & 7);
}

// Byte offset of the 16-token chunk `chunk` of head `h`'s weight row (hl 0 =
// hi codes, 1 = lo codes).
__device__ __forceinline__ int w_off(int hl, int h, int chunk) {
  return hl * (kH * kStepTok) + h * kStepTok + 16 * (chunk ^ ((h >> 2) & 3));
}

__device__ __forceinline__ char* stage(const Lds& S, int t) { return S.tiles + (t & (kStages - 1)) * kTileBytes; }
__device__ __forceinline__ char* scale_slot(const Lds& S, int step) {
  return S.scales + (step & (kScaleSlots - 1)) * kScaleSlot;
}

struct Bases {
  int qk[2][2];    // [row block rb][half h]: row 16 rb + c, unit 2g + h (k-step s adds 2048 s)
  int rope[2][2];  // [rb][h]: row 16 rb + c, unit 32 + 2 (g & 1) + h
  int pv[4];       // [read rd]: row 8 rd + c / 2 of the lane's stage, unit 8w + u1 (m-tile m adds 512 m)
};

// PV lane layout (32x32x64): lane (dim d = l % 32, kg = l / 32) holds the
// 32 tokens 32 kg .. 32 kg + 31 of the step, i.e. all rows of stage kg of
// the step; its 16-lane group reads unit 8w + 2m + ((l >> 4) & 1) of 8 rows
// per read.
__device__ __forceinline__ Bases bases(int w, int lane) {
  Bases L;
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 16 * rb + c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      L.qk[rb][h] = 16 * slot(r, 2 * g + h);
      L.rope[rb][h] = 16 * slot(r, 32 + 2 * (g & 1) + h);
    }
  }
  const int u1 = (lane >> 4) & 1, kg = lane >> 5;
#pragma unroll
  for (int rd = 0; rd < 4; ++rd)
    L.pv[rd] = kg * kTileBytes + 16 * slot(8 * rd + (c >> 1), 8 * w + u1) + 8 * (c & 1);
  return L;
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(__attribute__((address_space(3))) char*)(p));
}

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Split of x (|x| < 448) into two E4M3 codes per value, 4 values per 32-bit
// word: hi = RNE(x), lo = RNE(x - hi); hi + lo = x to a relative 2^-9, and
// exactly for a bf16 value of magnitude >= 2^-2.
__device__ __forceinline__ void split4(const float (&x)[4], int& hw, int& lw) {
  hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hw, true);
  const auto h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, false);
  const auto h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, true);
  lw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - h01[0], x[1] - h01[1], 0, false);
  lw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - h23[0], x[3] - h23[1], lw, true);
}

// The power of two 2^k that puts m = max |x| (> 0) in [128, 256).
__device__ __forceinline__ int pow2_for(float m) {
  int e = (m > 0.f && m <= 3.0e38f) ? 8 - __builtin_amdgcn_frexp_expf(m) : 0;
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

// The QK role's query operands for head 16w + c (lane group g):
//   hi[s], lo[s]: E4M3 codes of q 2^e for dims 128 s + 32 g + j (byte j);
//   rope:         rope dims 512 + 32 (g & 1) + j: their hi codes in lanes
//                 g < 2 and their lo codes in lanes g >= 2, so one MFMA over
//                 128 dims adds hi.K + lo.K of the 64 rope dims (the A
//                 operand repeats the rope dims in its upper half);
// the caller multiplies the score by 2^-e (inv_scale).
struct Query {
  i32x8 hi[kQSteps8], lo[kQSteps8], rope;
  float inv_scale;
};

__device__ __forceinline__ void load_query(const uint16_t* qhead, int g, Query& Q) {
  typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
  u16x8 raw[kQSteps8 + 1][4];
  const int gr = g & 1;  // rope: lanes g and g + 2 read the same dims
#pragma unroll
  for (int s = 0; s < kQSteps8; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) raw[s][v] = *reinterpret_cast<const u16x8*>(qhead + 128 * s + 32 * g + 8 * v);
#pragma unroll
  for (int v = 0; v < 4; ++v) raw[kQSteps8][v] = *reinterpret_cast<const u16x8*>(qhead + 512 + 32 * gr + 8 * v);
  float mx = 0.f;
#pragma unroll
  for (int s = 0; s <= kQSteps8; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(bf16f(raw[s][v][j])));
  mx = max4_rows(mx);
  const int e = pow2_for(mx);
  Q.inv_scale = __builtin_ldexpf(1.0f, -e);
#pragma unroll
  for (int s = 0; s <= kQSteps8; ++s) {
    i32x8 h8, l8;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float x[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = __builtin_ldexpf(bf16f(raw[s][d >> 1][4 * (d & 1) + t]), e);
      int hw, lw;
      split4(x, hw, lw);
      h8[d] = hw;
      l8[d] = lw;
    }
    if (s < kQSteps8) {
      Q.hi[s] = h8;
      Q.lo[s] = l8;
    } else {
      Q.rope = g < 2 ? h8 : l8;
    }
  }
  // opaque from here on, so the loads are waited for here and never repeated
#pragma unroll
  for (int s = 0; s < kQSteps8; ++s) asm volatile("" : "+v"(Q.hi[s]), "+v"(Q.lo[s]));
  asm volatile("" : "+v"(Q.rope));
}

__device__ __forceinline__ f32x4 mfma16(const i32x8& a, const i32x8& b, const f32x4& c) {
  // E4M3 A and B (format 0), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(i32x4 a, i32x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// S^T of the step's four 16-token blocks (mb: rows 16 (mb & 1) .. + 15 of
// stage 2i + (mb >> 1)) for the wave's 16 heads, scaled by 2^e. Per k-step
// the four blocks' hi MFMAs run first, then their lo MFMAs: an FP8 MFMA
// that accumulates onto the result of the one just before it waits for
// that result (chains of dependent MFMAs ran at half rate), so the two
// MFMAs of one accumulator are four apart. The next k-step's A operands
// are read during the current one. In the rope k-step lanes g >= 2 read
// the row's rope dims again, against the lo codes of the query (Query), so
// that k-step takes one MFMA per block.
template <typename StageFn>
__device__ __forceinline__ void qk_step(StageFn&& stage_of, const Bases& L, const Query& Q, f32x4 (&sacc)[4]) {
  auto load_a = [&](int mb, int s) -> i32x8 {
    const char* tile = stage_of(mb >> 1);
    const int rb = mb & 1;
    const int o0 = s < kQSteps8 ? L.qk[rb][0] + 2048 * s : L.rope[rb][0];
    const int o1 = s < kQSteps8 ? L.qk[rb][1] + 2048 * s : L.rope[rb][1];
    return join(*reinterpret_cast<const i32x4*>(tile + o0), *reinterpret_cast<const i32x4*>(tile + o1));
  };
  i32x8 a[2][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) a[0][mb] = load_a(mb, 0);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s <= kQSteps8; ++s) {
    const int cur = s & 1;
    if (s < kQSteps8) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) a[cur ^ 1][mb] = load_a(mb, s + 1);
    }
    if (s < kQSteps8) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sacc[mb] = mfma16(a[cur][mb], Q.hi[s], sacc[mb]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sacc[mb] = mfma16(a[cur][mb], Q.lo[s], sacc[mb]);
    } else {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sacc[mb] = mfma16(a[cur][mb], Q.rope, sacc[mb]);
    }
  }
}

// Per step, the QK lane's share of the weights: tokens 16 mb + 4g + k of the
// step (mb = 0..3, k = 0..3), 4 per 32-bit word.
struct StepW {
  int hi[4], lo[4];
  float alpha;
  int wexp;
};

// QK role over the tiles 0 .. 2 ns - 1 of the sequence (a tile past the
// range is fully masked). Barriers: 2 + 2 ns, the PV role's sequence.
__device__ __forceinline__ void ws_qk(const Tiles& T, int w, int g, int c, const Bases& L, const Query& Q,
                                      float scale_log2, QkStat& st, const Lds& S) {
  if (T.ntiles <= 0) return;
  const int ns = (T.ntiles + 1) / 2;
  const float sl2 = scale_log2 * Q.inv_scale;
  const int head = 16 * w + c;
  auto nvalid = [&](int t) { return t < T.ntiles ? T.nvalid(t) : 0; };
  auto scores = [&](int i, f32x4 (&sacc)[4], float (&ts)[4][4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 sv = *reinterpret_cast<const f32x4*>(scale_slot(S, i) + 128 * (mb >> 1) + 64 * (mb & 1) + 16 * g);
#pragma unroll
      for (int k = 0; k < 4; ++k) ts[mb][k] = sv[k];
    }
    qk_step([&](int kg) -> const char* { return stage(S, 2 * i + kg); }, L, Q, sacc);
  };
  auto softmax = [&](int i, const f32x4 (&sacc)[4], const float (&ts)[4][4], StepW& out) {
    float x[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int k = 0; k < 4; ++k) x[mb][k] = sacc[mb][k] * ts[mb][k];
    const int nv0 = nvalid(2 * i), nv1 = nvalid(2 * i + 1);
    if (nv0 < kBN || nv1 < kBN) {  // wave-uniform: a ragged or padding tile
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tok = 16 * (mb & 1) + 4 * g + k;
          x[mb][k] = tok < ((mb >> 1) ? nv1 : nv0) ? x[mb][k] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int k = 0; k < 4; ++k) mx = fmaxf(mx, x[mb][k]);
    // reference max (log2 domain): moves only when a score passes it by 2^8
    const float mxs = max4_rows(mx) * sl2;
    const bool move = mxs > st.m_run + 8.f;
    const float m_new = move ? mxs : st.m_run;
    out.alpha = move ? __builtin_amdgcn_exp2f(st.m_run - m_new) : 1.f;  // 0 on the first step
    st.m_run = m_new;
    float psum = 0.f, wm = 0.f;
    float wv[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p = __builtin_amdgcn_exp2f(fmaf(x[mb][k], sl2, -m_new));
        psum += p;
        wv[mb][k] = p * ts[mb][k];
        wm = fmaxf(wm, wv[mb][k]);
      }
    st.l_run = st.l_run * out.alpha + psum;
    // weights scaled by 2^k2 so the head's largest lies in [128, 256)
    const int k2 = pow2_for(max4_rows(wm));
    const float sc = __builtin_ldexpf(1.0f, k2);
    out.wexp = 127 - k2;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = wv[mb][k] * sc;
      split4(y, out.hi[mb], out.lo[mb]);
    }
  };
  auto publish = [&](const StepW& o) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      *reinterpret_cast<int*>(S.w + w_off(0, head, mb) + 4 * g) = o.hi[mb];
      *reinterpret_cast<int*>(S.w + w_off(1, head, mb) + 4 * g) = o.lo[mb];
    }
    if (g == 0) {
      S.alpha[head] = o.alpha;
      S.wexp[head] = o.wexp;
    }
  };
  __syncthreads();  // Y_0: stages 0 and 1 ready
  StepW o;
  for (int i = 0; i < ns; ++i) {
    // phase A: weights of step i-1 out, QK MFMAs of step i
    if (i > 0) publish(o);
    f32x4 sacc[4];
    float ts[4][4];
    scores(i, sacc, ts);
    __syncthreads();  // Z_i: weights of step i-1 visible
    // phase B: softmax of step i (the PV wavefronts accumulate step i-1)
    softmax(i, sacc, ts, o);
    __syncthreads();  // Y_{i+1}: the PV wavefronts are done with the buffer; stages 2i+2, 2i+3 ready
  }
  publish(o);
  __syncthreads();  // W: weights of the last step visible
}

// PV role over the FP8 rows at `base` (token 0; c_t bytes per token) and the
// token scales at `sbase` (s_t floats per token); tp = thread index in the
// role (0..255). Per stage, thread tp < 192 of wavefronts 0-2 loads units
// tp + 192 k (k < 6); wavefront 3 loads the scales of step i + 6 during
// step i. A tile past the range re-reads the last real tile (its tokens
// are masked); entries past a ragged tile re-read its last token.
template <Policy kPol>
__device__ __forceinline__ void ws_pv(const Tiles& T, const uint8_t* base, int64_t c_t, const float* sbase,
                                      int64_t s_t, int tp, int w, const Bases& L, f32x16 (&oacc)[kPvM][2],
                                      const Lds& S) {
  if (T.ntiles <= 0) return;
  const int lane = tp & 63;
  const int ns = (T.ntiles + 1) / 2;
  const bool rows = w < 3;  // wave-uniform: row loader or scale loader
  uint32_t toff[kUnitLoads];  // source byte offsets of this thread's units in a full tile
#pragma unroll
  for (int k = 0; k < kUnitLoads; ++k) {
    int r, u;
    slot_ru((rows ? tp : 0) + kLoaders * k, r, u);  // the slot this thread's load k fills
    toff[k] = (uint32_t)r * (uint32_t)c_t + 16u * (uint32_t)u;
  }
  const uint64_t sb = uniform_ptr(base);
  auto dst = [&](int t, int k) -> uint32_t {  // LDS byte address of this wave's load k of stage t
    return __builtin_amdgcn_readfirstlane(lds_addr(stage(S, t) + 16 * (kLoaders * k + 64 * w)));
  };
  auto first_tok = [&](int t, int& lim) -> int64_t {  // a padding tile re-reads the last real one
    const int tt = t < T.ntiles ? t : T.ntiles - 1;
    const int64_t tok0 = T.t0 + (int64_t)T.phys(tt) * kBN;
    lim = (int)min((int64_t)(kBN - 1), T.t1 - 1 - tok0);
    return tok0;
  };
  auto issue = [&](int t) {  // rows of stage t (wavefronts 0-2)
    int lim;
    const int64_t tok0 = first_tok(t, lim);
    if (lim == kBN - 1) {
      const uint64_t tb = sb + (uint64_t)(tok0 * c_t);
#pragma unroll
      for (int k = 0; k < kUnitLoads; ++k) lds_dma16_s<kPol>(tb, toff[k], dst(t, k));
    } else {
#pragma unroll
      for (int k = 0; k < kUnitLoads; ++k) {
        int r, u;
        slot_ru(tp + kLoaders * k, r, u);
        lds_dma16<kPol>(base + (tok0 + min(r, lim)) * c_t + 16 * u, dst(t, k));
      }
    }
  };
  auto issue_step = [&](int s) {  // rows of step s (wavefronts 0-2)
    issue(2 * s);
    issue(2 * s + 1);
  };
  auto issue_scales = [&](int s) {  // scales of step s (wavefront 3)
    int lim;
    const int64_t tok0 = first_tok(2 * s + (lane >> 5), lim);
    lds_dma4<kPol>(sbase + (tok0 + min(lane & 31, lim)) * s_t,
                   __builtin_amdgcn_readfirstlane(lds_addr(scale_slot(S, s))));
  };
  // wavefront 3: all but the scale loads of `ahead` later steps landed
  auto wait_scales = [&](int ahead) {
    switch (ahead) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<1>(); break;
      case 2: wait_vmcnt<2>(); break;
      case 3: wait_vmcnt<3>(); break;
      case 4: wait_vmcnt<4>(); break;
      default: wait_vmcnt<5>(); break;
    }
  };
  // prologue: rows of steps 0 and 1, scales of steps 0 .. kScaleAhead - 1;
  // the phase A of step i issues the rows of step i+2 (into the stages of
  // step i-2, whose products are done) and the scales of step i + kScaleAhead
  if (rows) {
    issue_step(0);
    if (ns > 1) issue_step(1);
    if (ns > 1) wait_vmcnt<2 * kUnitLoads>();  // step 0 landed
    else wait_vmcnt<0>();
  } else {
    for (int s = 0; s < kScaleAhead && s < ns; ++s) issue_scales(s);
    wait_scales(min(kScaleAhead, ns) - 1);  // step 0's scales landed
  }
  __syncthreads();  // Y_0

  // O += V^T W of step j (stages 2j, 2j+1; lanes kg = 1 read the second)
  auto pv = [&](int j) {
    const char* tiles = S.tiles + (2 * j & (kStages - 1)) * kTileBytes;
    const int kg = lane >> 5;
    float al[2];
    int we[2];
    i32x8 wb[2][2];
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      const int h = 32 * n2 + (lane & 31);
      al[n2] = S.alpha[h];
      we[n2] = S.wexp[h];
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        wb[n2][hl] = join(*reinterpret_cast<const i32x4*>(S.w + w_off(hl, h, 2 * kg)),
                          *reinterpret_cast<const i32x4*>(S.w + w_off(hl, h, 2 * kg + 1)));
    }
    if (__any(al[0] != 1.f || al[1] != 1.f)) {
#pragma unroll
      for (int m = 0; m < kPvM; ++m)
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) oacc[m][n2] *= al[n2];
    }
    // V^T operands of the four m-tiles, then the hi MFMAs of all eight
    // accumulators and their lo MFMAs (an accumulator's two MFMAs are eight
    // apart)
    i32x8 va[kPvM];
#pragma unroll
    for (int m = 0; m < kPvM; ++m) {
      i32x2 r[4];
#pragma unroll
      for (int rd = 0; rd < 4; ++rd) r[rd] = lds_read_tr8(tiles + L.pv[rd] + 512 * m);
      va[m] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
      for (int m = 0; m < kPvM; ++m)
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2)
          oacc[m][n2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[m], wb[n2][hl], oacc[m][n2], 0, 0, 0, 127, 0,
                                                                         we[n2]);
  };

  for (int i = 0; i < ns; ++i) {
    // phase A (the QK wavefronts score step i): loads of later steps
    if (rows) {
      if (i + 2 < ns) issue_step(i + 2);
    } else if (i + kScaleAhead < ns) {
      issue_scales(i + kScaleAhead);
    }
    __syncthreads();  // Z_i: weights of step i-1 visible
    // phase B: products of step i-1
    if (i > 0) pv(i - 1);
    // step i+1 landed: rows of step i+2, scales of steps i+2 .. i+kScaleAhead may be in flight
    if (rows) {
      if (i + 2 < ns) wait_vmcnt<2 * kUnitLoads>();
      else wait_vmcnt<0>();
    } else {
      wait_scales(max(0, min(ns - 1, i + kScaleAhead) - (i + 1)));
    }
    __syncthreads();  // Y_{i+1}
  }
  __syncthreads();  // W: weights of the last step visible
  pv(ns - 1);
}

}  // namespace f8
}  // namespace mla
}  // namespace cpa
