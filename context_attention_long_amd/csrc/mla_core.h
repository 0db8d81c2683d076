// Attention of one query (64 heads) over a contiguous range of an MLA latent
// cache, on one 4-wavefront workgroup: the shared core of the split-KV
// decode kernel and the MLA prefill kernel.
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 1.3 and 3.2-3.4 -- all heads of a query read one latent vector per token;
// vLLM GLM-5.3 post, footnote 1 -- QK runs over the 576 latent dims and PV
// over 512 (the value of a token is the first 512 dims of its latent). FP8
// entries are e4m3 * scale_t. The result is the unnormalised running state
// (O, running max, running sum) of the online softmax over the range.
//
// Design (gfx950):
//  * 32-token tiles of the latent are staged in LDS by direct global -> LDS
//    loads: bf16 keeps 4 stages (3 tiles in flight while one is consumed),
//    FP8 keeps 4 raw stages plus 2 converted bf16 tiles; the next tile's
//    loads are spread over the QK steps of the current one;
//  * QK: wave w computes S^T = K Q^T for heads 16w..16w+15 with
//    v_mfma_f32_16x16x32_bf16 (A = 16 tokens x 32 dims from the LDS tile,
//    B = Q^T held in registers for the whole range); each lane ends with 8
//    scores of one head, the head's row max takes two row-swap permutes;
//  * the wave turns its scores into bf16 probabilities P and writes them to
//    LDS (one 16-byte store per lane) together with each head's rescale
//    factor; one barrier later
//  * PV: wave w accumulates O^T for value dims [128w, 128w+128) of all 64
//    heads: A = V^T read from the same latent tile with ds_read_b64_tr_b16
//    (each read feeds 4 MFMAs, one per head block), B = P^T from LDS. The
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

namespace cpa {
namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kH = 64;          // query heads sharing the latent
constexpr int kDk = 576;        // QK dims (latent)
constexpr int kDv = 512;        // PV dims (leading part of the latent)
constexpr int kBN = 32;         // tokens per LDS tile
constexpr int kThreads = 256;   // 4 wavefronts
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

// Maximum / sum over the four lanes l, l^16, l^32, l^48 (one head's four
// score groups), with the gfx950 row-swap permutes instead of LDS round trips.
__device__ __forceinline__ float max4_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum4_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

struct State {
  f32x4 oacc[kMv][4];  // PV role: O^T dims 128w + 16m + 4g + i, head 16 hb + c
  float m_run;         // QK role: running reference max of head 16w + c (log2 domain)
  float l_run;         // QK role: this lane's share of that head's running sum
};

__device__ __forceinline__ void init_state(State& st) {
#pragma unroll
  for (int m = 0; m < kMv; ++m)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      st.oacc[m][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(st.oacc[m][hb]));
    }
  st.m_run = -INFINITY;
  st.l_run = 0.f;
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

// Tokens [t0, t1) of a bf16 latent cache (`base` = token 0, `c_t` elements
// per token) through the core. Stage i % 4 holds tile i; tokens past t1 in
// the last tile re-read token t1 - 1 and are masked.
// ---- bf16 pipeline: one barrier per tile ----
// Step i, after the barrier that publishes P_i (and tile i+1):
//   S_{i+1} = K_{i+1} Q^T                      (QK role, MFMA)
//   O += V_i^T P_i, rescaled by alpha_i first   (PV role, MFMA)
//   softmax(S_{i+1}) -> P_{i+1}, alpha_{i+1}    (VALU, placed between the PV
//                                                MFMAs so it runs in their shadow)
// P and alpha are double buffered (P_{i+1} goes to the buffer P_{i-1} used,
// which every wave finished reading before the barrier), so one barrier per
// tile orders everything: the tile stages, the P exchange and the reuse.

// QK of one tile into sacc; hook(s) runs at k-step s; vpre(m) at the last
// kAheadV steps issues the first V operand reads of the tile PV works on.
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

// kMask: bit t of vmask says whether token t of the tile is a selection
// (index-list attention); without it the first nvalid tokens are.
template <bool kFp8, bool kMask = false>
__device__ __forceinline__ void soft_scores(Soft& sm, const f32x4 (&sacc)[2], int nvalid, int g, float scale_log2,
                                            const TokScale& ts, uint32_t vmask = 0xffffffffu) {
  sm.mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g + i;
      float v = sacc[mt][i] * scale_log2;
      if constexpr (kFp8) v *= ts.v[4 * mt + i];
      if constexpr (kMask)
        v = (t < nvalid && ((vmask >> t) & 1u)) ? v : -INFINITY;
      else
        v = (t < nvalid) ? v : -INFINITY;
      sm.x[4 * mt + i] = v;
      sm.mx = fmaxf(sm.mx, v);
    }
}

template <typename St>
__device__ __forceinline__ void soft_ref(Soft& sm, St& st) {
  const float mx = max4_rows(sm.mx);
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
__device__ __forceinline__ void soft_exp(Soft& sm, const St& st, const TokScale& ts) {
  const float mref = (kMask && st.m_run == -INFINITY) ? 0.f : st.m_run;
#pragma unroll
  for (int j = J0; j < J0 + 4; ++j) {
    const float p = __builtin_amdgcn_exp2f(sm.x[j] - mref);
    sm.psum += p;
    sm.pf[j] = kFp8 ? p * ts.v[j] : p;
  }
}

template <typename St>
__device__ __forceinline__ void soft_store(Soft& sm, St& st, char* pbuf, float* abuf, int w, int g, int c) {
  st.l_run += sm.psum;
  // P^T chunk of this lane: head 16w + c, k-elements 8g..8g+7 in score order
  *reinterpret_cast<bf16x8*>(pbuf + p_off(16 * w + c, g)) = pack8(sm.pf);
  if (g == 0) abuf[16 * w + c] = sm.alpha;
}

// Interleave `n` MFMAs of the current scheduling region with the VALU work
// placed in it (1 MFMA, then up to `v` VALU instructions).
template <int N, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

// One pipeline step (see above). kNext: tile nxt exists (QK + softmax of it);
// ts: the token scales of tile nxt (FP8).
// pv_hook(m) runs in PV m-step m (the FP8 path converts its next tile there,
// where the LDS is far less busy than during QK).
// kMask / vmask: selection bits of tile nxt (see soft_scores).
template <bool kNext, bool kFp8 = false, bool kMask = false, typename Hook, typename PvHook>
__device__ __forceinline__ void pipe_step(const char* cur, const char* nxt, int nvalid_nxt, int buf, int w, int g,
                                          int c, const LdsBases& L, const bf16x8 (&qreg)[kQSteps], float scale_log2,
                                          State& st, const Lds& S, Hook&& hook, PvHook&& pv_hook,
                                          const TokScale& ts = TokScale{}, uint32_t vmask = 0xffffffffu) {
  constexpr int kAheadV = 4;
  bf16x8 va[kMv];
  auto load_v = [&](int m) {
    va[m] = join_tr(lds_read_tr(cur + L.pv[0][m & 3] + 128 * (m >> 2)),
                    lds_read_tr(cur + L.pv[1][m & 3] + 128 * (m >> 2)));
  };
  // P_i and alpha_i are read first: their LDS latency then hides behind the
  // QK MFMAs instead of stalling the start of PV
  const float* acur = S.alpha + kH * buf;
  const char* pcur = S.p + kH * kPRowBytes * buf;
  float al[4];
  bf16x8 pb[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    al[hb] = acur[16 * hb + c];
    pb[hb] = *reinterpret_cast<const bf16x8*>(pcur + p_off(16 * hb + c, g));
  }
  f32x4 sacc[2];
  if constexpr (kNext) {
    qk_tile(nxt, L, qreg, sacc, hook, load_v);
  } else {
#pragma unroll
    for (int m = 0; m < kAheadV; ++m) load_v(m);
  }
  // ---- alpha_i: rescale O (rare) ----
  if (__any(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
    for (int m = 0; m < kMv; ++m)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        asm volatile("" : "+a"(st.oacc[m][hb]));
        st.oacc[m][hb] *= al[hb];
        asm volatile("" : "+a"(st.oacc[m][hb]));
      }
  }
  // ---- PV_i with softmax_{i+1} in the MFMA shadows ----
  Soft sm;
#pragma unroll
  for (int m = 0; m < kMv; ++m) {
    if (m + kAheadV < kMv) load_v(m + kAheadV);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      st.oacc[m][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[m], pb[hb], st.oacc[m][hb], 0, 0, 0);
      asm volatile("" : "+a"(st.oacc[m][hb]));
    }
    if constexpr (kNext) {
      if (m == 0) soft_scores<kFp8, kMask>(sm, sacc, nvalid_nxt, g, scale_log2, ts, vmask);
      if (m == 1) soft_ref(sm, st);
      if (m == 2) soft_exp<kFp8, 0, kMask>(sm, st, ts);
      if (m == 3) soft_exp<kFp8, 4, kMask>(sm, st, ts);
      if (m == 4) soft_store(sm, st, S.p + kH * kPRowBytes * (buf ^ 1), S.alpha + kH * (buf ^ 1), w, g, c);
      if (m <= 4) interleave_mfma_valu<4, 6>();
    }
    pv_hook(m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Tokens [t0, t1) of a bf16 latent cache (`base` = token 0, `c_t` elements
// per token) through the core. Step i consumes tile (i + rot) mod ntiles:
// the softmax state does not depend on the order of the tiles, and a
// workgroup-specific rotation keeps the many workgroups that stream equally
// aligned ranges at the same rate from addressing the same HBM channels in
// lockstep. Stage i % 4 holds step i's tile; tokens past t1 in the last tile
// re-read token t1 - 1 and are masked. Needs S.p and S.alpha with room for
// two buffers.
template <Policy P>
__device__ __forceinline__ void run_bf16(const uint16_t* base, int64_t c_t, int64_t t0, int64_t t1, int w, int g,
                                         int c, const LdsBases& L, const bf16x8 (&qreg)[kQSteps], float scale_log2,
                                         State& st, const Lds& S, uint32_t rot_seed = 0) {
  const int tid = threadIdx.x;
  const int ntok = (int)(t1 - t0);
  const int ntiles = (ntok + kBN - 1) / kBN;
  if (ntiles <= 0) return;
  const int rot = (int)(rot_seed % (uint32_t)ntiles);
  auto phys = [&](int i) { const int t = i + rot; return t >= ntiles ? t - ntiles : t; };
  uint32_t toff[kLdChunks];  // byte offset of this thread's chunks inside a full tile
#pragma unroll
  for (int k = 0; k < kLdChunks; ++k) {
    const int Pc = tid + kThreads * k;
    const int row = Pc / kRowChunks, pc = Pc % kRowChunks;
    toff[k] = (uint32_t)((row * c_t + swz(row, pc) * 8) * 2);
  }
  auto tile_ptr = [&](int i) -> const char* { return S.tiles + (i & 3) * kTileBytes; };
  auto stage = [&](int i) { return S.tiles + (i & 3) * kTileBytes + 64 * w * 16; };
  auto issue = [&](int i) {
    const int64_t tok0 = t0 + (int64_t)phys(i) * kBN;
    char* dst0 = stage(i);
    if (tok0 + kBN <= t1) {
      const uint16_t* tb = base + tok0 * c_t;
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k) lds_dma16_sbase<P>(tb, toff[k], lds_addr(dst0 + kThreads * k * 16));
    } else {
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k) {
        const int Pc = tid + kThreads * k;
        const int row = Pc / kRowChunks, pc = Pc % kRowChunks;
        const int64_t tok = min(tok0 + row, t1 - 1);
        lds_dma16<P>(base + tok * c_t + swz(row, pc) * 8, lds_addr(dst0 + kThreads * k * 16));
      }
    }
  };
  auto nvalid = [&](int i) { return min(kBN, ntok - kBN * phys(i)); };
  for (int i = 0; i < 3 && i < ntiles; ++i) issue(i);
  // ---- prologue: S_0 and P_0 ----
  wait_ahead<kLdChunks>(min(2, ntiles - 1));  // tile 0 landed
  __syncthreads();
  {
    f32x4 sacc[2];
    qk_tile(tile_ptr(0), L, qreg, sacc, [](int) {}, [](int) {});
    Soft sm;
    const TokScale none{};
    soft_scores<false>(sm, sacc, nvalid(0), g, scale_log2, none);
    soft_ref(sm, st);
    soft_exp<false, 0>(sm, st, none);
    soft_exp<false, 4>(sm, st, none);
    soft_store(sm, st, S.p, S.alpha, w, g, c);
  }
  // ---- steady state ----
  for (int i = 0; i + 1 < ntiles; ++i) {
    wait_ahead<kLdChunks>(min(1, ntiles - 2 - i));  // tile i+1 landed
    __syncthreads();  // P_i and tile i+1 visible; every wave is done with tile i-1 and P_{i-1}
    // tile i+3 goes into the stage tile i-1 used: a full tile's loads are
    // spread over the QK steps of tile i+1 (one every other step), the
    // clamped last tile is issued at once
    const int64_t nxt0 = t0 + (int64_t)phys(i + 3 < ntiles ? i + 3 : 0) * kBN;
    const bool spread = (i + 3 < ntiles) && (nxt0 + kBN <= t1);
    if (i + 3 < ntiles && !spread) issue(i + 3);
    const uint64_t ntb = uniform_ptr(base + nxt0 * c_t);
    const uint32_t ndst = __builtin_amdgcn_readfirstlane(lds_addr(stage(i + 3)));
    pipe_step<true>(tile_ptr(i), tile_ptr(i + 1), nvalid(i + 1), i & 1, w, g, c, L, qreg, scale_log2, st, S,
                    [&](int s) {
                      if (spread && (s & 1) == 0 && (s >> 1) < kLdChunks)
                        lds_dma16_s<P>(ntb, toff[s >> 1], ndst + kThreads * (s >> 1) * 16);
                    },
                    [](int) {});
  }
  __syncthreads();  // P of the last tile visible
  pipe_step<false>(tile_ptr(ntiles - 1), nullptr, 0, (ntiles - 1) & 1, w, g, c, L, qreg, scale_log2, st, S,
                   [](int) {}, [](int) {});
}

// Tokens [t0, t1) of an FP8 E4M3 latent cache with one fp32 scale per token
// (entry = e4m3 * scale_t), through the same pipeline as bf16. The cache
// bytes stream into registers two tiles ahead of use (nontemporal vector
// loads: each thread holds 9 units of 8 bytes of a tile); during the PV
// MFMAs of step i each unit of tile i+2 is converted to bf16 exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and written to its swizzled LDS
// position, and its register is refilled with tile i+4. Three bf16 stages:
// tile i (PV), tile i+1 (QK), tile i+2 (being written). The scales are
// loaded into registers one step ahead of the softmax that folds them in.
// Tile order rotated as in run_bf16. kPol = kStream marks the loads
// nontemporal (a range read once), kReuse leaves them cached (a range other
// workgroups read too).
template <Policy kPol = Policy::kStream>
__device__ __forceinline__ void run_fp8(const uint8_t* base, int64_t c_t, const float* sbase, int64_t s_t, int64_t t0,
                                        int64_t t1, int w, int g, int c, const LdsBases& L,
                                        const bf16x8 (&qreg)[kQSteps], float scale_log2, State& st, const Lds& S,
                                        uint32_t rot_seed = 0) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x;
  const int ntok = (int)(t1 - t0);
  const int ntiles = (ntok + kBN - 1) / kBN;
  if (ntiles <= 0) return;
  const int rot = (int)(rot_seed % (uint32_t)ntiles);
  auto phys = [&](int i) { const int t = i + rot; return t >= ntiles ? t - ntiles : t; };
  auto nvalid = [&](int i) { return min(kBN, ntok - kBN * phys(i)); };
  auto stage = [&](int i) -> char* { return S.tiles + (i % 3) * kTileBytes; };
  // unit j of this thread: 8 cache bytes of row u / 72, chunk u % 72 (u = tid + 256 j)
  uint32_t goff[kLdChunks], loff[kLdChunks];
  int urow[kLdChunks];
#pragma unroll
  for (int j = 0; j < kLdChunks; ++j) {
    const int u = tid + kThreads * j;
    const int row = u / kRowChunks, ch = u % kRowChunks;
    urow[j] = row;
    goff[j] = (uint32_t)(ch * 8);
    loff[j] = (uint32_t)(row * (kRowChunks * 16) + swz(row, ch) * 16);
  }
  u32x2 raw[2][kLdChunks];
  TokScale tsc[2];
  // Addresses: a wavefront-uniform tile base plus a 32-bit lane offset; rows
  // past the range's last token re-read it (lim = last valid row). The host
  // bounds the token stride so that 32 rows fit 32-bit offsets.
  const uint32_t ct32 = (uint32_t)c_t, st32 = (uint32_t)s_t;
  auto load_unit = [&](int i, int j, u32x2& r) {
    const int64_t tok0 = t0 + (int64_t)phys(i) * kBN;
    const int lim = (int)min((int64_t)(kBN - 1), t1 - 1 - tok0);
    const uint8_t* tb = base + tok0 * c_t;
    const uint32_t off = (uint32_t)min(urow[j], lim) * ct32 + goff[j];
    if constexpr (kPol == Policy::kStream)
      r = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tb + off));
    else
      r = *reinterpret_cast<const u32x2*>(tb + off);
  };
  auto load_scales = [&](int i, TokScale& ts) {
    const int64_t tok0 = t0 + (int64_t)phys(i) * kBN;
    const int lim = (int)min((int64_t)(kBN - 1), t1 - 1 - tok0);
    const float* sb = sbase + tok0 * s_t;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if constexpr (kPol == Policy::kStream)
        ts.v[j] = __builtin_nontemporal_load(sb + (uint32_t)min(16 * (j >> 2) + 4 * g + (j & 3), lim) * st32);
      else
        ts.v[j] = sb[(uint32_t)min(16 * (j >> 2) + 4 * g + (j & 3), lim) * st32];
  };
  auto convert_unit = [&](const u32x2& r, int j, char* tile) {
    const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r[0], 1.0f, false));
    const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r[0], 1.0f, true));
    const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r[1], 1.0f, false));
    const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r[1], 1.0f, true));
    *reinterpret_cast<uint4*>(tile + loff[j]) = make_uint4(o0, o1, o2, o3);
  };

  // ---- prologue: tiles 0, 1 converted; tiles 2, 3 in flight; S_0 and P_0 ----
  auto clampt = [&](int i) { return min(i, ntiles - 1); };
#pragma unroll
  for (int j = 0; j < kLdChunks; ++j) load_unit(0, j, raw[0][j]);
  load_scales(0, tsc[0]);
#pragma unroll
  for (int j = 0; j < kLdChunks; ++j) load_unit(clampt(1), j, raw[1][j]);
  load_scales(clampt(1), tsc[1]);
#pragma unroll
  for (int j = 0; j < kLdChunks; ++j) {
    convert_unit(raw[0][j], j, stage(0));
    load_unit(clampt(2), j, raw[0][j]);
  }
#pragma unroll
  for (int j = 0; j < kLdChunks; ++j) {
    convert_unit(raw[1][j], j, stage(1));
    load_unit(clampt(3), j, raw[1][j]);
  }
  __syncthreads();
  {
    f32x4 sacc[2];
    qk_tile(stage(0), L, qreg, sacc, [](int) {}, [](int) {});
    Soft sm;
    soft_scores<true>(sm, sacc, nvalid(0), g, scale_log2, tsc[0]);
    soft_ref(sm, st);
    soft_exp<true, 0>(sm, st, tsc[0]);
    soft_exp<true, 4>(sm, st, tsc[0]);
    soft_store(sm, st, S.p, S.alpha, w, g, c);
  }
  // ---- steady state, two steps per trip so the register sets are static ----
  // The loads and conversions of a step are unconditional (past the last
  // tile they re-read the last tile and write a stage nobody reads again):
  // loads under a branch make the compiler's wait placement fall back to
  // waiting for every outstanding load, which would drain the stream.
  auto step = [&](int i, auto parity) {
    constexpr int P = decltype(parity)::value;  // i & 1
    __syncthreads();  // P_i and bf16 tile i+1 visible; every wave is done with tile i-1 and P_{i-1}
    const int conv_t = min(i + 2, ntiles - 1), refill_t = min(i + 4, ntiles - 1);
    char* dst = stage(i + 2);
    pipe_step<true, true>(stage(i), stage(i + 1), nvalid(i + 1), P, w, g, c, L, qreg, scale_log2, st, S,
                          [&](int s) {
                            if (s == 1) load_scales(conv_t, tsc[P]);  // tile i's scales are spent
                          },
                          [&](int m) {  // units 0-1 at m-step 0, one per m-step after
#pragma unroll
                            for (int j = (m == 0 ? 0 : m + 1); j <= m + 1; ++j) {
                              convert_unit(raw[P][j], j, dst);
                              load_unit(refill_t, j, raw[P][j]);
                            }
                          },
                          tsc[P ^ 1]);
  };
  int i = 0;
  for (; i + 2 < ntiles; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
  }
  if (i + 1 < ntiles) {
    step(i, std::integral_constant<int, 0>{});
    ++i;
  }
  __syncthreads();  // P of the last tile visible
  pipe_step<false>(stage(ntiles - 1), nullptr, 0, (ntiles - 1) & 1, w, g, c, L, qreg, scale_log2, st, S, [](int) {},
                   [](int) {});
}

// ---- index-list (sparse) attention ----
// The tokens are the cache rows named by entries [0, ntok) of an index list
// (Long Context 2.4: a sparse-attention query brings its own list). Entry
// values outside [0, nrows) are no selection: their scores are masked and
// their loads read row 0. Each wavefront copies the entries of a tile into
// its own LDS ring slot with one 4-byte-per-lane direct load (lane l: entry
// l mod 32), five tiles ahead of use, so the index values never pass through
// registers the compiler would have to wait for. Per step i, in this order:
// the entries of tile i+5, then the nine row loads of tile i+3 (addresses
// from the ring, spread over the QK steps of tile i+1). Since vector-memory
// loads complete in issue order, the wait at the top of step i for tile i+1
// (at most 1 + 9 loads issued after it) also covers the entries of tiles up
// to i+3; the ring slot of tile i is rewritten (step i) only after its last
// readers (the address reads of step i-3, the selection mask of step i-1).
constexpr int kIdxSlots = 5;
constexpr int kIdxSlotBytes = 256;                          // 64 lanes x 4 B
constexpr int kIdxRingBytes = 4 * kIdxSlots * kIdxSlotBytes;  // per workgroup (4 waves)

template <Policy P>
__device__ __forceinline__ void run_bf16_gather(const uint16_t* base, int64_t c_t, const int32_t* ilist, int ntok,
                                                int nrows, int w, int g, int c, const LdsBases& L,
                                                const bf16x8 (&qreg)[kQSteps], float scale_log2, State& st,
                                                const Lds& S, char* ring, uint32_t rot_seed = 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int ntiles = (ntok + kBN - 1) / kBN;
  if (ntiles <= 0) return;
  const int rot = (int)(rot_seed % (uint32_t)ntiles);
  auto phys = [&](int i) { const int t = i + rot; return t >= ntiles ? t - ntiles : t; };
  auto nvalid = [&](int i) { return min(kBN, ntok - kBN * phys(i)); };
  const uint32_t rowbytes = (uint32_t)c_t * 2u;  // the host bounds nrows * rowbytes below 2^32
  // this thread's chunks of a tile: tile row (high half) and swizzled source byte offset
  uint32_t rinfo[kLdChunks];
#pragma unroll
  for (int k = 0; k < kLdChunks; ++k) {
    const int Pc = tid + kThreads * k;
    const int row = Pc / kRowChunks, pc = Pc % kRowChunks;
    rinfo[k] = ((uint32_t)row << 16) | (uint32_t)(swz(row, pc) * 16);
  }
  const char* wring = ring + w * (kIdxSlots * kIdxSlotBytes);
  const uint32_t wring_lds = __builtin_amdgcn_readfirstlane(lds_addr(wring));
  const uint64_t ibase = uniform_ptr(ilist), cbase = uniform_ptr(base);
  auto slot = [&](int T) { return (T % kIdxSlots) * kIdxSlotBytes; };
  auto issue_idx = [&](int T) {
    const int Tc = T < ntiles ? T : ntiles - 1;  // past the end: re-read the last tile's entries
    const int e = min(kBN * phys(Tc) + (lane & 31), ntok - 1);
    lds_dma4_s<Policy::kReuse>(ibase, (uint32_t)e * 4u, wring_lds + (uint32_t)slot(T));
  };
  auto row_of = [&](int T, int row) -> uint32_t {
    const int v = *reinterpret_cast<const int*>(wring + slot(T) + 4 * row);
    return (uint32_t)v < (uint32_t)nrows ? (uint32_t)v : 0u;
  };
  auto offsets = [&](int T, uint32_t (&voff)[kLdChunks]) {
#pragma unroll
    for (int k = 0; k < kLdChunks; ++k) voff[k] = row_of(T, (int)(rinfo[k] >> 16)) * rowbytes + (rinfo[k] & 0xffffu);
  };
  auto tile_mask = [&](int T) -> uint32_t {
    const int v = *reinterpret_cast<const int*>(wring + slot(T) + 4 * (lane & 31));
    return (uint32_t)__ballot((uint32_t)v < (uint32_t)nrows);
  };
  auto tile_ptr = [&](int i) -> const char* { return S.tiles + (i & 3) * kTileBytes; };
  auto dst = [&](int i) {
    return __builtin_amdgcn_readfirstlane(lds_addr(S.tiles + (i & 3) * kTileBytes + 64 * w * 16));
  };
  auto issue_tile = [&](int T) {
    uint32_t voff[kLdChunks];
    offsets(T, voff);
    const uint32_t d = dst(T);
#pragma unroll
    for (int k = 0; k < kLdChunks; ++k) lds_dma16_s<P>(cbase, voff[k], d + kThreads * k * 16);
  };
  // ---- prologue: entries of tiles 0..4, rows of tiles 0..2 ----
  issue_idx(0);
  issue_idx(1);
  issue_idx(2);
  cpa::wait_vmcnt<2>();  // entries of tile 0
  issue_tile(0);
  issue_idx(3);
  if (ntiles > 1) {
    cpa::wait_vmcnt<11>();  // entries of tile 1 (then: 2, rows 0, 3)
    issue_tile(1);
  }
  issue_idx(4);
  if (ntiles > 2) {
    cpa::wait_vmcnt<20>();  // entries of tile 2 (then: rows 0, 3, rows 1, 4)
    issue_tile(2);
  }
  // rows of tile 0 landed (after them: entries 3, rows 1, entries 4, rows 2)
  if (ntiles > 2) cpa::wait_vmcnt<20>();
  else if (ntiles == 2) cpa::wait_vmcnt<11>();
  else cpa::wait_vmcnt<2>();
  __syncthreads();
  {
    f32x4 sacc[2];
    qk_tile(tile_ptr(0), L, qreg, sacc, [](int) {}, [](int) {});
    Soft sm;
    const TokScale none{};
    soft_scores<false, true>(sm, sacc, nvalid(0), g, scale_log2, none, tile_mask(0));
    soft_ref(sm, st);
    soft_exp<false, 0, true>(sm, st, none);
    soft_exp<false, 4, true>(sm, st, none);
    soft_store(sm, st, S.p, S.alpha, w, g, c);
  }
  // ---- steady state ----
  for (int i = 0; i + 1 < ntiles; ++i) {
    // rows of tile i+1 landed: after them only the entries of tile i+4 and the rows of tile i+2
    if (i + 2 < ntiles) cpa::wait_vmcnt<10>();
    else cpa::wait_vmcnt<1>();
    __syncthreads();  // P_i and tile i+1 visible; every wave is done with tile i-1 and P_{i-1}
    issue_idx(i + 5);
    const bool more = i + 3 < ntiles;
    uint32_t voff[kLdChunks];
    offsets(i + 3, voff);
    const uint32_t ndst = dst(i + 3);
    pipe_step<true, false, true>(tile_ptr(i), tile_ptr(i + 1), nvalid(i + 1), i & 1, w, g, c, L, qreg, scale_log2,
                                 st, S,
                                 [&](int s) {
                                   if (more && (s & 1) == 0 && (s >> 1) < kLdChunks)
                                     lds_dma16_s<P>(cbase, voff[s >> 1], ndst + kThreads * (s >> 1) * 16);
                                 },
                                 [](int) {}, TokScale{}, tile_mask(i + 1));
  }
  __syncthreads();  // P of the last tile visible
  pipe_step<false>(tile_ptr(ntiles - 1), nullptr, 0, (ntiles - 1) & 1, w, g, c, L, qreg, scale_log2, st, S,
                   [](int) {}, [](int) {});
  cpa::wait_vmcnt<0>();  // entry loads issued past the last tile have landed
}

// Closes the range: the softmax sum of every head into S.lsum (one barrier).
// Returns this lane's QK-role head total (head 16w + c).
__device__ __forceinline__ float finish(const State& st, int w, int g, int c, const Lds& S) {
  const float l = sum4_rows(st.l_run);
  if (g == 0) S.lsum[16 * w + c] = l;
  __syncthreads();
  return l;
}

}  // namespace mla
}  // namespace cpa
