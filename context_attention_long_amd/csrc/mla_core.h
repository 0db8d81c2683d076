// Building blocks of the MLA attention core: attention of one query's 64
// heads over a range of an MLA latent cache in 32-token LDS tiles. The
// pipeline that runs them (roles, stages, barriers) is in mla_ws.h.
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 1.3 and 3.2-3.4 -- all heads of a query read one latent vector per token;
// vLLM GLM-5.3 post, footnote 1 -- QK runs over the 576 latent dims and PV
// over 512 (the value of a token is the first 512 dims of its latent). FP8
// entries are e4m3 * scale_t. The result is the unnormalised running state
// (O, running max, running sum) of the online softmax over the range.
//
// Design (gfx950):
//  * QK (qk_tile): wave w computes S^T = K Q^T for heads 16w..16w+15 with
//    v_mfma_f32_16x16x32_bf16 (A = 16 tokens x 32 dims from the LDS tile,
//    B = Q^T held in registers for the whole range); each lane ends with 8
//    scores of one head, the head's row max takes two row-swap permutes;
//  * the softmax pieces (soft_*) turn the scores into bf16 probabilities P,
//    stored to LDS (one 16-byte store per lane) with each head's rescale
//    factor;
//  * PV: A = V^T read from the same latent tile with ds_read_b64_tr_b16
//    (each read feeds 4 MFMAs, one per head block), B = P^T from LDS; the
//    32 tokens of a k-step are taken in the order the score registers hold
//    them, so P needs no shuffle;
//  * the softmax reference max only moves when a score exceeds it by more
//    than 2^8 (p <= 256 meanwhile; O and the sum share the reference, so the
//    result is the same); rescaling O is then a rare branch;
//  * LDS rows are 72 chunks of 16 bytes, XOR-swizzled inside aligned groups
//    of 8 chunks (see swz) so both operand reads run at the full LDS rate.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "lds_dma.h"
#include "paged.h"
#include "wave_ops.h"

namespace cpa {
namespace mla {

using cpa::max4_rows;
using cpa::sum4_rows;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kH = 64;          // query heads sharing the latent
constexpr int kDk = 576;        // QK dims (latent)
constexpr int kDv = 512;        // PV dims (leading part of the latent)
constexpr int kBN = 32;         // tokens per LDS tile
constexpr int kThreads = 256;   // threads of one role (4 wavefronts)
constexpr int kRowChunks = kDk / 8;               // 72 chunks of 16 B per bf16 row
constexpr int kTileChunks = kBN * kRowChunks;     // 2304
constexpr int kTileBytes = kTileChunks * 16;      // 36864
constexpr int kLdChunks = kTileChunks / kThreads; // 9 chunks per thread (bf16)
constexpr int kStages = 4;
constexpr int kSmemBytes = kStages * kTileBytes;  // 144 KB
constexpr int kFp8RowChunks = kDk / 16;           // 36 source chunks per fp8 row
constexpr int kRawBytes = kBN * kDk;              // 18 KB: one 32-token FP8 tile
constexpr int kRawWaveLoads = kRawBytes / 1024;   // 18 wave-wide 16-byte loads per tile
constexpr int kPRowBytes = 64;                    // one head's 32 bf16 probabilities
constexpr int kQSteps = kDk / 32;                 // 18 QK k-steps
constexpr int kMv = kDv / 4 / 16;                 // 8 PV m-tiles per wave (128 dims)
constexpr float kLn2 = 0.69314718055994531f;

static_assert(kTileChunks % kThreads == 0, "tile must split evenly over the threads");
static_assert(kRawWaveLoads * 1024 == kRawBytes && kDk % 16 == 0, "raw FP8 tile layout");

// LDS the kernels declare and hand to the core.
struct Lds {
  char* tiles;     // kSmemBytes: bf16 stages, or FP8 raw stages + 2 bf16 tiles
  char* p;         // [2 buffers][64 heads][64 B] probabilities of a tile
  float* alpha;    // [2 buffers][64] rescale factor of each head for a tile
  float* lsum;     // [64] final softmax sum of each head
};

// Physical 16-byte chunk of logical chunk `c` in LDS row `r` (XOR inside the
// aligned group of 8 chunks). gfx950 LDS has 64 four-byte banks (256 B per
// clock); a row is 1152 B, so rows alternate between the two 128-byte bank
// halves and the XOR must separate the rows one read pass touches. With
// f(r) = bits (b0, b2, b1) of r both operand reads run at the full LDS rate:
// the 16-byte K reads (16 rows x 4 chunks) and the 8-byte transposing V
// reads (4 rows x 2 chunks per 16 lanes); the previous f(r) = (r ^ r>>3) & 7
// halved the K read rate (measured with a microbenchmark of these patterns).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 1) | ((r & 2) << 1) | ((r & 4) >> 1)); }

// Byte offset of head h's 16-byte P chunk g (k-elements 8g..8g+7) in the P
// buffer; the chunk XOR keeps both the stores and the operand loads free of
// bank conflicts.
__device__ __forceinline__ int p_off(int h, int g) { return h * kPRowBytes + 16 * (g ^ ((h >> 1) & 3)); }

__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) char*)(p));
}

// Operand vectors are assembled only from whole registers: packed pairs and
// whole-vector bit casts. (Building a bf16 vector one element at a time is
// lowered incorrectly by the gfx950 code generator of this toolchain: it
// duplicates or misaligns elements.)
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

// Per-lane LDS byte offsets inside a tile. Every operand read of a tile is
// one of these bases plus a compile-time constant, so the reads use the LDS
// instruction's immediate offset instead of one address register each.
struct LdsBases {
  int qk[2][2];  // [token block mt][k-step parity]: row 16mt + c, chunk (4(s&1) + g) ^ f
  int pv[2][4];  // [row r0 / r1][m & 3]: rows 4g + c/4 (+16), chunk of dims 128w + 16m + 4(c&3)
};

__device__ __forceinline__ LdsBases lds_bases(int w, int g, int c) {
  LdsBases L;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = 16 * mt + c;
#pragma unroll
    for (int par = 0; par < 2; ++par) L.qk[mt][par] = row * (kRowChunks * 16) + swz(row, 4 * par + g) * 16;
  }
  const int r0 = 4 * g + (c >> 2);
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = r0 + 16 * rr;
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4)
      L.pv[rr][m4] = row * (kRowChunks * 16) + 256 * w + swz(row, 2 * m4 + ((c & 3) >> 1)) * 16 + 8 * (c & 1);
  }
  return L;
}

// Q^T operand of the QK role: lane (g, c) holds q[16w + c][32s + 8g .. +8]
// for k-step s. All loads are issued before the first wait, so their
// latencies overlap. The registers are then made opaque: otherwise the
// compiler re-loads these read-only values inside the tile loop, or defers
// the wait for them into the loop, where (not knowing the tile loads issued
// from inline assembly) its vmcnt count would also wait for those.
__device__ __forceinline__ void load_q(const uint16_t* qhead, int g, bf16x8 (&qreg)[kQSteps]) {
  const uint16_t* qp = qhead + 8 * g;
#pragma unroll
  for (int s = 0; s < kQSteps; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
#pragma unroll
  for (int s = 0; s < kQSteps; ++s) asm volatile("" : "+v"(qreg[s]));
}

template <int N>
__device__ __forceinline__ void wait_ahead(int ahead) {
  // at most `ahead` further tiles of N loads each may still be in flight
  if (ahead >= 3) cpa::wait_vmcnt<3 * N>();
  else if (ahead == 2) cpa::wait_vmcnt<2 * N>();
  else if (ahead == 1) cpa::wait_vmcnt<N>();
  else cpa::wait_vmcnt<0>();
}

// QK of one tile into sacc (K operands read kAhead k-steps ahead); hook(s)
// runs at k-step s; vpre(m) runs at the last kAheadV k-steps.
template <typename Hook, typename VPre>
__device__ __forceinline__ void qk_tile(const char* tile, const LdsBases& L, const bf16x8 (&qreg)[kQSteps],
                                        f32x4 (&sacc)[2], Hook&& hook, VPre&& vpre) {
  constexpr int kAhead = 4;
  constexpr int kAheadV = 4;
  sacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ka[kQSteps][2];
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      ka[s][mt] = *reinterpret_cast<const bf16x8*>(tile + L.qk[mt][s & 1] + 128 * (s >> 1));
#pragma unroll
  for (int s = 0; s < kQSteps; ++s) {
    hook(s);
    if (s + kAhead < kQSteps) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        ka[s + kAhead][mt] =
            *reinterpret_cast<const bf16x8*>(tile + L.qk[mt][(s + kAhead) & 1] + 128 * ((s + kAhead) >> 1));
    }
    if (s >= kQSteps - kAheadV) vpre(s - (kQSteps - kAheadV));
    sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s][0], qreg[s], sacc[0], 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s][1], qreg[s], sacc[1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Online softmax of the QK-role head 16w + c over one tile, in pieces so the
// pieces can sit between the MFMAs of the PV step. Branch free: a lane moves
// its reference max only when a score exceeds it by more than 2^8 (always
// on the first tile); alpha is the factor the head's O and sum take.
struct Soft {
  float x[8];
  float mx, alpha, psum;
  float pf[8];
};

// FP8 cache: the per-token scales of the 8 tokens whose scores a lane holds
// (element j: token 16 (j / 4) + 4g + j % 4 of the tile). The scale
// multiplies the score (s = scale_t q.e_t) and P (p_t scale_t multiplies e_t
// in PV); the bf16 path passes none.
struct TokScale {
  float v[8];
};

// Scores stay unscaled (raw dot products; times the token scale for FP8)
// until the exponential, where one FMA applies the softmax scale and
// subtracts the reference: the max is taken over raw scores (the scale is
// positive) and scaled once. The mask (ragged last tile, or selection bits)
// is applied only where it can matter. kMask: bit t of vmask says whether
// token t of the tile is a selection (index-list attention); without it the
// first nvalid tokens are.
template <bool kFp8, bool kMask = false>
__device__ __forceinline__ void soft_scores(Soft& sm, const f32x4 (&sacc)[2], int nvalid, int g, float scale_log2,
                                            const TokScale& ts, uint32_t vmask = 0xffffffffu) {
  (void)scale_log2;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.x[4 * mt + i] = kFp8 ? sacc[mt][i] * ts.v[4 * mt + i] : sacc[mt][i];
  if (kMask || nvalid < kBN) {  // wave-uniform
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 16 * (j >> 2) + 4 * g + (j & 3);
      const bool keep = kMask ? (t < nvalid && ((vmask >> t) & 1u)) : t < nvalid;
      sm.x[j] = keep ? sm.x[j] : -INFINITY;
    }
  }
  sm.mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) sm.mx = fmaxf(sm.mx, sm.x[j]);
}

template <typename St>
__device__ __forceinline__ void soft_ref(Soft& sm, St& st, float scale_log2) {
  const float mx = max4_rows(sm.mx) * scale_log2;
  const bool move = mx > st.m_run + 8.f;
  const float m_new = move ? mx : st.m_run;
  sm.alpha = move ? __builtin_amdgcn_exp2f(st.m_run - m_new) : 1.f;  // 0 on the first tile
  st.m_run = m_new;
  st.l_run *= sm.alpha;
  sm.psum = 0.f;
}

// kMask: a head may have seen no selected token yet (reference max still
// -inf, every score -inf); its probabilities are then 0, not -inf - -inf.
template <bool kFp8, int J0, bool kMask = false, typename St>
__device__ __forceinline__ void soft_exp(Soft& sm, const St& st, const TokScale& ts, float scale_log2) {
  const float mref = (kMask && st.m_run == -INFINITY) ? 0.f : st.m_run;
#pragma unroll
  for (int j = J0; j < J0 + 4; ++j) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sm.x[j], scale_log2, -mref));
    sm.psum += p;
    sm.pf[j] = kFp8 ? p * ts.v[j] : p;
  }
}

template <typename St>
__device__ __forceinline__ void soft_store(Soft& sm, St& st, char* pbuf, float* abuf, int w, int g, int c) {
  st.l_run += sm.psum;
  // P^T chunk of this lane: head 16w + c, k-elements 8g..8g+7 in score order
  *reinterpret_cast<bf16x8*>(pbuf + p_off(16 * w + c, g)) = pack8(sm.pf);
  abuf[16 * w + c] = sm.alpha;  // the head's four lane groups hold the same value
}

// ---- index-list (sparse) attention: the LDS ring of list entries ----
// (Long Context 2.4: a sparse-attention query brings its own list.) Entry
// values outside [0, nrows) are no selection: their scores are masked and
// their loads read row 0. A loading wavefront copies the entries of a tile
// into its own ring slot with one 4-byte-per-lane direct load (lane l: entry
// l mod 32), five tiles ahead of use, so the index values never pass
// through registers the compiler would have to wait for (see ws_pv_gather).
constexpr int kIdxSlots = 5;
constexpr int kIdxSlotBytes = 256;                          // 64 lanes x 4 B
constexpr int kIdxRingBytes = 4 * kIdxSlots * kIdxSlotBytes;  // per workgroup (the 4 PV wavefronts)

}  // namespace mla
}  // namespace cpa
