// FP8 latent cache variant of the wave-specialised MLA core (mla_ws.h).
//
// What it computes: the same online-softmax state as the bf16 core --
// attention of one query's 64 heads over a range of an MLA latent cache,
// QK over the 576 latent dims, PV over the first 512 ("How GPUs Share a Long
// Context During LLM Inference", 1.3; vLLM GLM-5.3 post, footnote 1) -- for
// an OCP E4M3 cache with one fp32 scale per token: entry_t = e4m3_t * scale_t.
// The scale multiplies the score and the probability (s_t = scale_t q.e_t,
// and p_t scale_t multiplies e_t in PV), so the e4m3 codes enter the products
// unscaled and exactly.
//
// Design (gfx950), per 32-token tile:
//  * the tile stays FP8 in LDS: direct global -> LDS loads of the raw rows
//    (18 KB per tile, half the bytes of a bf16 tile), 8 stages in flight, the
//    32 token scales loaded the same way into a slot beside the stage;
//  * QK on the FP8 matrix cores: v_mfma_scale_f32_16x16x128_f8f6f4 takes
//    the K tile straight from LDS (A = 16 tokens x 128 dims) and the query
//    as FP8 (B). A bf16 query value q is split exactly into two E4M3 values,
//    q 2^e = hi + lo (e: a per-head power of two that puts the head's
//    largest |q| in [128, 256); hi has 4 significant bits, the remainder
//    the next 4, which is exactly what a bf16 value has beyond hi for every
//    element within 2^-10 of the head's maximum), so QK = hi.K + lo.K costs
//    two FP8 MFMAs -- the time of one bf16 MFMA -- and matches the bf16
//    product to fp32 rounding. The 64 rope dims run as two bf16 16x16x32
//    MFMAs on codes converted in registers. The factor 2^-e is folded into
//    the softmax scale;
//  * PV stays bf16 (P is a bf16 probability, as in the bf16 core): the V^T
//    operand comes from ds_read_b64_tr_b8 -- lane c of each 16-lane group
//    receives byte c of the 8 rows its group addresses, i.e. one value
//    dimension for 8 tokens -- and four v_cvt_scalef32_pk_bf16_fp8 turn the
//    8 codes into the bf16 operand. No bf16 copy of the tile is written.
//  * rows are XOR-swizzled in 16-byte units inside aligned groups of four;
//    the swizzle (bits r2 ^ r3 and r3 ^ r4 of the row) keeps the three read
//    patterns (QK 16-byte reads, rope 8-byte reads, transposing V reads)
//    free of LDS bank conflicts.
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

constexpr int kRowBytes = kDk;                   // 576 one-byte codes per token
constexpr int kRowUnits = kRowBytes / 16;        // 36 units of 16 bytes
constexpr int kTileUnits = kBN * kRowUnits;      // 1152
constexpr int kTileBytes = kTileUnits * 16;      // 18432
constexpr int kStages = 8;                       // tiles in LDS (loads run up to 7 tiles ahead)
constexpr int kScaleSlot = 256;                  // one 4-byte load per lane of a wavefront
constexpr int kLoads = 5;                        // loads per PV thread and tile (4-5 units + scales)
constexpr int kQSteps8 = 4;                      // FP8 k-steps of 128 dims (dims 0..511)
constexpr int kRopeSteps = 2;                    // bf16 k-steps of 32 dims (dims 512..575)
constexpr int kSmemBytes = kStages * (kTileBytes + kScaleSlot);

static_assert(kTileUnits == 4 * kThreads + kThreads / 2, "unit split over the PV threads");
static_assert(kRowUnits % 4 == 0, "swizzle groups of four units");

struct Lds {
  char* tiles;   // stages x kTileBytes
  char* scales;  // stages x kScaleSlot (f32 token scales of the tile, 32 used)
  char* p;       // [2][64 heads][64 B] bf16 probabilities
  float* alpha;  // [2][64]
  float* lsum;   // [64]
  int stage_mask;  // stages - 1 (a power of two: kStages for ranges, fewer for index lists)
};

// Swizzle of row r: the physical unit of logical unit u is u ^ swz(r). Rows
// are 144 words long, so row r starts at bank 16 (r & 3). The LDS (64 banks
// of 4 bytes) serves a 16-byte read in four passes of 16 lanes: lanes of one
// half-wave whose quad index ((lane >> 2) & 7) has even, or odd, parity
// (measured: two active lanes, different words of one bank, conflict iff
// they share a pass); an 8-byte read (plain or transposing) in two passes
// of 32 consecutive lanes. With bit 0 = r2 ^ r3 and bit 1 = r3 ^ r4 every
// pass of the K reads (rows 16 mt + c, units 2g + h), the rope reads (16
// rows, one unit) and the transposing value reads (rows 4g + (0..3) and
// 16 + 4g + (0..3), one unit) touches each bank once.
__device__ __forceinline__ int swz(int r) { return (((r >> 2) ^ (r >> 3)) & 1) | ((((r >> 3) ^ (r >> 4)) & 1) << 1); }

__device__ __forceinline__ int unit_off(int r, int u) { return r * kRowBytes + 16 * (u ^ swz(r)); }

// Token of element j of a lane in lane group g, in the order the QK output
// registers hold the scores (the k order of the PV product).
__device__ __forceinline__ int score_token(int g, int j) { return 16 * (j >> 2) + 4 * g + (j & 3); }

struct Bases {
  int qk[2][2];    // [token block mt][half h]: row 16 mt + c, unit 2g + h (k-step s adds 128 s)
  int rope[2][2];  // [mt][k-step]: row 16 mt + c, dims 512 + 32 s + 8 g
  int pv[4];       // [m & 3]: row score_token(g, c / 2), dims of m-tile m, byte 8 (c & 1); m >> 2 adds 64
};

__device__ __forceinline__ Bases bases(int w, int g, int c) {
  Bases L;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = 16 * mt + c;
#pragma unroll
    for (int h = 0; h < 2; ++h) L.qk[mt][h] = unit_off(r, 2 * g + h);
#pragma unroll
    for (int s = 0; s < kRopeSteps; ++s) L.rope[mt][s] = unit_off(r, 32 + 2 * s + (g >> 1)) + 8 * (g & 1);
  }
  const int r = score_token(g, c >> 1);
#pragma unroll
  for (int b = 0; b < 4; ++b) L.pv[b] = unit_off(r, 8 * w + b) + 8 * (c & 1);
  return L;
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(__attribute__((address_space(3))) char*)(p));
}

// 8 E4M3 codes (byte j = element j) -> 8 bf16 values, exactly.
__device__ __forceinline__ bf16x8 codes_to_bf16(i32x2 r) {
  const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, false));
  const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[0], 1.0f, true));
  const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, false));
  const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[1], 1.0f, true));
  return __builtin_bit_cast(bf16x8, make_uint4(o0, o1, o2, o3));
}

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// The QK role's query operands for head 16w + c (lane group g):
//   hi[s], lo[s]: FP8 codes of q 2^e for dims 128 s + 32 g + j, byte j;
//   rope[s]: bf16 of q 2^e for dims 512 + 32 s + 8 g + j;
// e puts the head's largest |q| (over all 576 dims) in [128, 256), so no
// code saturates; the caller multiplies the score by 2^-e (*inv_scale).
struct Query {
  i32x8 hi[kQSteps8], lo[kQSteps8];
  bf16x8 rope[kRopeSteps];
  float inv_scale;
};

__device__ __forceinline__ void load_query(const uint16_t* qhead, int g, Query& Q) {
  typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
  u16x8 raw[kQSteps8][4];
  u16x8 rr[kRopeSteps];
#pragma unroll
  for (int s = 0; s < kQSteps8; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) raw[s][v] = *reinterpret_cast<const u16x8*>(qhead + 128 * s + 32 * g + 8 * v);
#pragma unroll
  for (int s = 0; s < kRopeSteps; ++s) rr[s] = *reinterpret_cast<const u16x8*>(qhead + 512 + 32 * s + 8 * g);
  float mx = 0.f;
#pragma unroll
  for (int s = 0; s < kQSteps8; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(bf16f(raw[s][v][j])));
#pragma unroll
  for (int s = 0; s < kRopeSteps; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(bf16f(rr[s][j])));
  mx = max4_rows(mx);
  // mx = f 2^E with f in [0.5, 1): scaled by 2^(8 - E) the maximum lies in [128, 256)
  int e = (mx > 0.f && mx <= 3.0e38f) ? 8 - __builtin_amdgcn_frexp_expf(mx) : 0;
  e = e < -100 ? -100 : (e > 100 ? 100 : e);  // keeps 2^-e a normal float
  Q.inv_scale = __builtin_ldexpf(1.0f, -e);
#pragma unroll
  for (int s = 0; s < kQSteps8; ++s) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int v = d >> 1, j0 = 4 * (d & 1);
      float x[4], r[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = __builtin_ldexpf(bf16f(raw[s][v][j0 + t]), e);
      int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hw, true);
      r[0] = x[0] - __builtin_amdgcn_cvt_scalef32_f32_fp8(hw, 1.0f, 0);
      r[1] = x[1] - __builtin_amdgcn_cvt_scalef32_f32_fp8(hw, 1.0f, 1);
      r[2] = x[2] - __builtin_amdgcn_cvt_scalef32_f32_fp8(hw, 1.0f, 2);
      r[3] = x[3] - __builtin_amdgcn_cvt_scalef32_f32_fp8(hw, 1.0f, 3);
      int lw = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
      lw = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lw, true);
      Q.hi[s][d] = hw;
      Q.lo[s][d] = lw;
    }
  }
#pragma unroll
  for (int s = 0; s < kRopeSteps; ++s) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_ldexpf(bf16f(rr[s][j]), e);
    Q.rope[s] = pack8(x);  // exact: a power-of-two multiple of a bf16 value
  }
  // opaque from here on, so the loads are waited for here and never repeated
#pragma unroll
  for (int s = 0; s < kQSteps8; ++s) asm volatile("" : "+v"(Q.hi[s]), "+v"(Q.lo[s]));
#pragma unroll
  for (int s = 0; s < kRopeSteps; ++s) asm volatile("" : "+v"(Q.rope[s]));
}

__device__ __forceinline__ f32x4 mfma_f8(const i32x8& a, const i32x8& b, const f32x4& c) {
  // E4M3 A and B (format 0), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// S^T (2 blocks of 16 tokens x the wave's 16 heads) of one tile, scaled by 2^e.
__device__ __forceinline__ void qk_tile(const char* tile, const Bases& L, const Query& Q, f32x4 (&sacc)[2]) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    i32x8 ka[kQSteps8];
    i32x2 kr[kRopeSteps];
#pragma unroll
    for (int s = 0; s < kQSteps8; ++s) {
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(tile + L.qk[mt][0] + 128 * s);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(tile + L.qk[mt][1] + 128 * s);
      ka[s] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int s = 0; s < kRopeSteps; ++s) kr[s] = *reinterpret_cast<const i32x2*>(tile + L.rope[mt][s]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kQSteps8; ++s) {
      acc = mfma_f8(ka[s], Q.hi[s], acc);
      acc = mfma_f8(ka[s], Q.lo[s], acc);
    }
#pragma unroll
    for (int s = 0; s < kRopeSteps; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(kr[s]), Q.rope[s], acc, 0, 0, 0);
    sacc[mt] = acc;
  }
}

__device__ __forceinline__ char* stage(const Lds& S, int i) { return S.tiles + (i & S.stage_mask) * kTileBytes; }
__device__ __forceinline__ char* scale_slot(const Lds& S, int i) {
  return S.scales + (i & S.stage_mask) * kScaleSlot;
}

// QK role. Barriers: 1 (tile 0) + (ntiles - 1) (loop) + 1 (after the loop),
// the same sequence as the PV role's. kMask: mask(i) gives the selection
// bits of tile i (index lists).
template <bool kMask = false, typename MaskFn = uint32_t (*)(int)>
__device__ __forceinline__ void ws_qk(const Tiles& T, int w, int g, int c, const Bases& L, const Query& Q,
                                      float scale_log2, QkStat& st, const Lds& S, MaskFn&& mask = nullptr) {
  if (T.ntiles <= 0) return;
  const float sl2 = scale_log2 * Q.inv_scale;
  auto step = [&](int i, auto parity) {
    constexpr int P = decltype(parity)::value;
    f32x4 sacc[2];
    qk_tile(stage(S, i), L, Q, sacc);
    TokScale ts;
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(scale_slot(S, i) + 16 * g);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(scale_slot(S, i) + 64 + 16 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) ts.v[j] = s0[j], ts.v[4 + j] = s1[j];
    Soft sm;
    if constexpr (kMask) soft_scores<true, true>(sm, sacc, T.nvalid(i), g, sl2, ts, mask(i));
    else soft_scores<true>(sm, sacc, T.nvalid(i), g, sl2, ts);
    soft_ref(sm, st, sl2);
    soft_exp<true, 0, kMask>(sm, st, ts, sl2);
    soft_exp<true, 4, kMask>(sm, st, ts, sl2);
    soft_store(sm, st, S.p + kH * kPRowBytes * P, S.alpha + kH * P, w, g, c);
  };
  __syncthreads();  // tile 0 ready
  step(0, std::integral_constant<int, 0>{});
  int i = 0;
  for (; i + 2 < T.ntiles; i += 2) {
    __syncthreads();  // P_i and tile i+1 visible
    step(i + 1, std::integral_constant<int, 1>{});
    __syncthreads();
    step(i + 2, std::integral_constant<int, 0>{});
  }
  if (i + 1 < T.ntiles) {
    __syncthreads();
    step(i + 1, std::integral_constant<int, 1>{});
  }
  __syncthreads();  // P of the last tile visible
}

template <int N>
__device__ __forceinline__ void wait_tiles(int ahead) {
  // at most `ahead` later tiles of N loads each may still be in flight
  switch (ahead) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<N>(); break;
    case 2: wait_vmcnt<2 * N>(); break;
    case 3: wait_vmcnt<3 * N>(); break;
    case 4: wait_vmcnt<4 * N>(); break;
    case 5: wait_vmcnt<5 * N>(); break;
    default: wait_vmcnt<6 * N>(); break;
  }
}

// PV role over the FP8 rows at `base` (token 0; c_t bytes per token) and the
// token scales at `sbase` (s_t floats per token). tp = thread index in the
// role (0..255). Every PV thread issues exactly kLoads loads per tile: units
// tp + 256 k (k < 4); then waves 0 and 1 load units 1024 + tp and waves 2
// and 3 the tile's scales (both the same 64 values, one 4-byte load per
// lane; entries past the tile re-read its last token).
// rows.row(t) is the cache row (and scale entry) of token t: the token
// itself, or its row in a paged pool (every load then takes its own address).
template <Policy kPol, typename Rows = LinearRows>
__device__ __forceinline__ void ws_pv(const Tiles& T, const uint8_t* base, int64_t c_t, const float* sbase,
                                      int64_t s_t, int tp, int w, int g, int c, const Bases& L,
                                      f32x4 (&oacc)[kMv][4], const Lds& S, const Rows& rows = Rows{}) {
  if (T.ntiles <= 0) return;
  // the PV wavefronts win instruction arbitration on their SIMD: measured
  // 2-3 % shorter launches than equal priorities (the QK wavefronts first,
  // for their MFMAs or the whole step, was slower)
  __builtin_amdgcn_s_setprio(3);
  const int lane = tp & 63;
  const bool unit5 = w < 2;  // wave-uniform
  uint32_t toff[kLoads];     // source byte offsets of this thread's units in a full tile
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int U = k < 4 ? tp + kThreads * k : 4 * kThreads + tp;  // k = 4 only where unit5
    const int r = U / kRowUnits, pu = U % kRowUnits;
    toff[k] = (uint32_t)r * (uint32_t)c_t + 16u * (uint32_t)(pu ^ swz(r));
  }
  const uint64_t sb = uniform_ptr(base);
  auto dst = [&](int i, int k) -> uint32_t {  // LDS byte address of this wave's load k of tile i
    return __builtin_amdgcn_readfirstlane(lds_addr(stage(S, i) + 16 * (kThreads * k + 64 * w)));
  };
  auto scale_load = [&](int i) {
    const int64_t tok0 = T.t0 + (int64_t)T.phys(i) * kBN;
    const int lim = (int)min((int64_t)(kBN - 1), T.t1 - 1 - tok0);
    lds_dma4<kPol>(sbase + rows.row(tok0 + min(lane, lim)) * s_t,
                   __builtin_amdgcn_readfirstlane(lds_addr(scale_slot(S, i))));
  };
  // all loads of tile i at once (prologue; the ragged last tile)
  auto issue = [&](int i) {
    const int64_t tok0 = T.t0 + (int64_t)T.phys(i) * kBN;
    if (tok0 + kBN <= T.t1 && rows.consecutive(tok0, tok0 + kBN - 1)) {  // one base, per-thread offsets
      const uint64_t tb = Rows::kLinear ? sb + (uint64_t)(tok0 * c_t) : uniform_ptr(base + rows.row(tok0) * c_t);
#pragma unroll
      for (int k = 0; k < 4; ++k) lds_dma16_s<kPol>(tb, toff[k], dst(i, k));
      if (unit5) lds_dma16_s<kPol>(tb, toff[4], dst(i, 4));
    } else {
      const int lim = (int)min((int64_t)(kBN - 1), T.t1 - 1 - tok0);
#pragma unroll
      for (int k = 0; k < kLoads; ++k) {
        if (k == 4 && !unit5) break;
        const int U = k < 4 ? tp + kThreads * k : 4 * kThreads + tp;
        const int r = U / kRowUnits, pu = U % kRowUnits;
        lds_dma16<kPol>(base + rows.row(tok0 + min(r, lim)) * c_t + 16 * (pu ^ swz(r)), dst(i, k));
      }
    }
    if (!unit5) scale_load(i);
  };
  const int n = T.ntiles;
  for (int i = 0; i < kStages - 1 && i < n; ++i) issue(i);
  wait_tiles<kLoads>(min(kStages - 2, n - 1));  // tile 0 landed
  __syncthreads();

  constexpr int kAheadV = 4;
  auto pv = [&](int i, auto&& hook) {
    const char* cur = stage(S, i);
    const float* acur = S.alpha + kH * (i & 1);
    const char* pcur = S.p + kH * kPRowBytes * (i & 1);
    float al[4];
    bf16x8 pb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      al[hb] = acur[16 * hb + c];
      pb[hb] = *reinterpret_cast<const bf16x8*>(pcur + p_off(16 * hb + c, g));
    }
    i32x2 vr[kMv];
    auto load_v = [&](int m) { vr[m] = lds_read_tr8(cur + L.pv[m & 3] + 64 * (m >> 2)); };
#pragma unroll
    for (int m = 0; m < kAheadV; ++m) load_v(m);
    if (__any(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
      for (int m = 0; m < kMv; ++m)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) oacc[m][hb] *= al[hb];
    }
#pragma unroll
    for (int m = 0; m < kMv; ++m) {
      if (m + kAheadV < kMv) load_v(m + kAheadV);
      hook(m);
      const bf16x8 va = codes_to_bf16(vr[m]);
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        oacc[m][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hb], oacc[m][hb], 0, 0, 0);
    }
  };

  for (int i = 0; i + 1 < n; ++i) {
    // tile i+1 landed: after it at most the tiles up to i + kStages - 2 are in flight
    wait_tiles<kLoads>(min(kStages - 3, n - 2 - i));
    __syncthreads();  // P_i and tile i+1 visible; every wave is done with tile i-1
    // tile i + kStages - 1 goes into the stage tile i-1 used: a full tile's
    // loads are spread over the first m-steps, a ragged one issued at once
    const int nt = i + kStages - 1;
    const int64_t nxt0 = T.t0 + (int64_t)T.phys(nt < n ? nt : 0) * kBN;
    const bool spread = (nt < n) && (nxt0 + kBN <= T.t1) && rows.consecutive(nxt0, nxt0 + kBN - 1);
    if (nt < n && !spread) issue(nt);
    const uint64_t ntb =
        Rows::kLinear ? sb + (uint64_t)(nxt0 * c_t) : uniform_ptr(base + (spread ? rows.row(nxt0) : 0) * c_t);
    pv(i, [&](int m) {
      if (spread) {
        if (m < 4) lds_dma16_s<kPol>(ntb, toff[m], dst(nt, m));
        if (m == 4) {
          if (unit5) lds_dma16_s<kPol>(ntb, toff[4], dst(nt, 4));
          else scale_load(nt);
        }
      }
    });
  }
  __syncthreads();  // P of the last tile visible
  pv(n - 1, [](int) {});
}

// Stages of the index-list role (4: tiles i .. i+3 in LDS).
constexpr int kGatherStages = 4;

// PV role over the FP8 rows an index list names (sparse attention): tile t
// holds list entries [32 t, 32 t + 32) of the range. Each PV wavefront
// copies the 32 entries of a tile into its own LDS ring slot with one
// 4-byte-per-lane direct load, five tiles ahead; the row loads of tile t
// (three tiles ahead, the same units and swizzle as ws_pv) and the token
// scales take their row numbers from the ring. An entry outside [0, nrows)
// reads row 0 (its score is masked by the QK role). Loads per PV thread and
// tile: one entry copy and kLoads rows / scales, in that order.
template <Policy kPol>
__device__ __forceinline__ void ws_pv_gather(const Tiles& T, const uint8_t* base, int64_t c_t, const float* sbase,
                                             int64_t s_t, const int32_t* ilist, int nrows, int tp, int w, int g,
                                             int c, const Bases& L, f32x4 (&oacc)[kMv][4], const Lds& S,
                                             char* ring) {
  if (T.ntiles <= 0) return;
  // the PV wavefronts win instruction arbitration on their SIMD: measured
  // 2-3 % shorter launches than equal priorities (the QK wavefronts first,
  // for their MFMAs or the whole step, was slower)
  __builtin_amdgcn_s_setprio(3);
  const int lane = tp & 63;
  const int n = T.ntiles;
  const bool unit5 = w < 2;  // wave-uniform: waves 0, 1 load a fifth unit, waves 2, 3 the scales
  uint32_t rinfo[kLoads];    // tile row (high half) and swizzled byte offset in the row of this thread's units
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int U = k < 4 ? tp + kThreads * k : 4 * kThreads + tp;  // k = 4 only where unit5
    const int r = U / kRowUnits, pu = U % kRowUnits;
    rinfo[k] = ((uint32_t)r << 16) | (uint32_t)(16 * (pu ^ swz(r)));
  }
  const char* wring = ring + w * (kIdxSlots * kIdxSlotBytes);
  const uint32_t wring_lds = __builtin_amdgcn_readfirstlane(lds_addr(wring));
  const uint64_t ibase = uniform_ptr(ilist), cbase = uniform_ptr(base), sb = uniform_ptr(sbase);
  const uint32_t rowbytes = (uint32_t)c_t;  // the host bounds nrows * c_t below 2^32
  const uint32_t sstride = (uint32_t)(s_t * 4);
  auto slot = [&](int t) { return (t % kIdxSlots) * kIdxSlotBytes; };
  auto issue_idx = [&](int t) {
    const int tc = t < n ? t : n - 1;  // past the end: re-read the last tile's entries
    const int e = min(kBN * T.phys(tc) + (lane & 31), T.ntok - 1);
    lds_dma4_s<Policy::kReuse>(ibase, (uint32_t)e * 4u, wring_lds + (uint32_t)slot(t));
  };
  auto row_of = [&](int t, int row) -> uint32_t {
    const int v = *reinterpret_cast<const int*>(wring + slot(t) + 4 * row);
    return (uint32_t)v < (uint32_t)nrows ? (uint32_t)v : 0u;
  };
  auto dst = [&](int t, int k) -> uint32_t {  // LDS byte address of this wave's load k of tile t
    return __builtin_amdgcn_readfirstlane(lds_addr(stage(S, t) + 16 * (kThreads * k + 64 * w)));
  };
  // source offsets of tile t's loads (rows, or the scales of waves 2 and 3)
  auto offsets = [&](int t, uint32_t (&voff)[kLoads]) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k)
      voff[k] = (k == 4 && !unit5) ? row_of(t, lane & 31) * sstride
                                   : row_of(t, (int)(rinfo[k] >> 16)) * rowbytes + (rinfo[k] & 0xffffu);
  };
  auto load = [&](int t, int k, const uint32_t (&voff)[kLoads]) {
    if (k < 4 || unit5) lds_dma16_s<kPol>(cbase, voff[k], dst(t, k));
    else lds_dma4_s<kPol>(sb, voff[k], __builtin_amdgcn_readfirstlane(lds_addr(scale_slot(S, t))));
  };
  auto issue_tile = [&](int t) {
    uint32_t voff[kLoads];
    offsets(t, voff);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) load(t, k, voff);
  };
  // ---- prologue: entries of tiles 0..4, rows of tiles 0..2 ----
  issue_idx(0);
  issue_idx(1);
  issue_idx(2);
  wait_vmcnt<2>();  // entries of tile 0
  issue_tile(0);
  issue_idx(3);
  if (n > 1) {
    wait_vmcnt<kLoads + 2>();  // entries of tile 1 (then: 2, rows 0, 3)
    issue_tile(1);
  }
  issue_idx(4);
  if (n > 2) {
    wait_vmcnt<2 * kLoads + 2>();  // entries of tile 2 (then: rows 0, 3, rows 1, 4)
    issue_tile(2);
  }
  // rows of tile 0 landed (after them: entries 3, rows 1, entries 4, rows 2)
  if (n > 2) wait_vmcnt<2 * kLoads + 2>();
  else if (n == 2) wait_vmcnt<kLoads + 2>();
  else wait_vmcnt<2>();
  __syncthreads();

  constexpr int kAheadV = 4;
  auto pv = [&](int i, auto&& hook) {
    const char* cur = stage(S, i);
    const float* acur = S.alpha + kH * (i & 1);
    const char* pcur = S.p + kH * kPRowBytes * (i & 1);
    float al[4];
    bf16x8 pb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      al[hb] = acur[16 * hb + c];
      pb[hb] = *reinterpret_cast<const bf16x8*>(pcur + p_off(16 * hb + c, g));
    }
    i32x2 vr[kMv];
    auto load_v = [&](int m) { vr[m] = lds_read_tr8(cur + L.pv[m & 3] + 64 * (m >> 2)); };
#pragma unroll
    for (int m = 0; m < kAheadV; ++m) load_v(m);
    if (__any(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
      for (int m = 0; m < kMv; ++m)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) oacc[m][hb] *= al[hb];
    }
#pragma unroll
    for (int m = 0; m < kMv; ++m) {
      if (m + kAheadV < kMv) load_v(m + kAheadV);
      hook(m);
      const bf16x8 va = codes_to_bf16(vr[m]);
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        oacc[m][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hb], oacc[m][hb], 0, 0, 0);
    }
  };
  for (int i = 0; i + 1 < n; ++i) {
    // rows of tile i+1 landed: after them only the entries of tile i+4 and the rows of tile i+2
    if (i + 2 < n) wait_vmcnt<kLoads + 1>();
    else wait_vmcnt<1>();
    __syncthreads();  // P_i and tile i+1 visible; every wave is done with tile i-1 and P_{i-1}
    issue_idx(i + 5);
    const bool more = i + 3 < n;
    uint32_t voff[kLoads];
    if (more) offsets(i + 3, voff);
    pv(i, [&](int m) {
      if (more && m < kLoads) load(i + 3, m, voff);
    });
  }
  __syncthreads();  // P of the last tile visible
  pv(n - 1, [](int) {});
  wait_vmcnt<0>();  // entry loads issued past the last tile have landed
}

}  // namespace f8
}  // namespace mla
}  // namespace cpa
