// Split-KV decode over a token-sharded MLA latent cache (bf16, or OCP FP8
// E4M3 with one fp32 scale per token).
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 3.2-3.4 -- a rank attends each request's single query over its own share
// of the cache and reports partial output + LSE; 1.3 and the vLLM DCP post,
// 5.3 -- one latent vector per token is read by all heads; vLLM GLM-5.3
// post, footnote 1 -- QK runs over the 576 latent dims and PV over 512 (the
// value of a token is the first 512 dims of its latent). FP8 entries are
// e4m3 * scale_t.
//
// Design (gfx950):
//  * one workgroup = 4 wavefronts per (request, split); wave w owns query
//    heads 16w..16w+15, so every latent tile staged in LDS serves all 64
//    heads and each cache byte is read from HBM once;
//  * QK as S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32
//    dims straight from the row-major LDS tile (16-byte reads), B = Q^T held
//    in registers for the whole split (18 k-steps); each lane ends with 8
//    scores of one head, so the running max needs two cross-lane steps;
//  * PV as O^T = V^T P^T: B = P^T comes from the score registers with no
//    shuffle (the 32 tokens of the k-step are ordered to match the score
//    layout), A = V^T is read from the same LDS tile with ds_read_b64_tr_b16
//    (transposing 16-bit reads), so one LDS copy feeds both products;
//  * the output accumulator O^T [512 x 16 heads] stays in registers; each
//    lane's column is one head, so the softmax rescale is lane-local;
//  * the cache streams from HBM by direct global -> LDS loads: bf16 keeps 4
//    tile stages (3 tiles in flight per CU while one is consumed); FP8 keeps
//    3 stages of 64 raw tokens plus one bf16 tile, converted e4m3 -> bf16
//    exactly once per CU; the per-token scale is folded into the score
//    (s = scale_t q.e_t) and into P (p_t * scale_t multiplies e_t in PV),
//    never into K itself;
//  * LDS rows are 72 chunks of 16 bytes, XOR-swizzled inside aligned groups
//    of 8 chunks so that the 16 rows one MFMA operand read touches fall in
//    distinct banks.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_dma.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kH = 64;          // query heads sharing the latent
constexpr int kDk = 576;        // QK dims (latent)
constexpr int kDv = 512;        // PV dims (leading part of the latent)
constexpr int kBN = 32;         // tokens per LDS tile
constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kRowChunks = kDk / 8;               // 72 chunks of 16 B per bf16 row
constexpr int kTileChunks = kBN * kRowChunks;     // 2304
constexpr int kTileBytes = kTileChunks * 16;      // 36864
constexpr int kLdChunks = kTileChunks / kThreads; // 9 chunks per thread (bf16)
constexpr int kFp8RowChunks = kDk / 16;           // 36 source chunks per fp8 row
constexpr int kFp8TileChunks = kBN * kFp8RowChunks;  // 1152
constexpr int kFp8LdChunks = (kFp8TileChunks + kThreads - 1) / kThreads;  // 5
constexpr float kLn2 = 0.69314718055994531f;

static_assert(kTileChunks % kThreads == 0, "tile must split evenly over the threads");

// Physical 16-byte chunk of logical chunk `c` in LDS row `r` (XOR inside the
// aligned group of 8 chunks). gfx950 LDS has 64 four-byte banks (256 B per
// clock); a row is 1152 B, so rows alternate between the two 128-byte bank
// halves and the XOR must separate the rows one read pass touches. With
// f(r) = bits (b0, b2, b1) of r both operand reads run at the full LDS rate:
// the 16-byte K reads (16 rows x 4 chunks) and the 8-byte transposing V
// reads (4 rows x 2 chunks per 16 lanes); the previous f(r) = (r ^ r>>3) & 7
// halved the K read rate (measured with a microbenchmark of these patterns).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r & 1) | ((r & 2) << 1) | ((r & 4) >> 1)); }

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

// Per-lane LDS byte offsets inside a tile. Every operand read of a tile is
// one of these bases plus a compile-time constant, so the reads use the LDS
// instruction's immediate offset instead of one address register each.
struct LdsBases {
  int qk[2][2];  // [token block mt][k-step parity]: row 16mt + c, chunk (4(s&1) + g) ^ f
  int pv[2][4];  // [row r0 / r1][m & 3]: rows 4g + c/4 (+16), chunk (2(m&3) + (c&3)/2) ^ f
};

__device__ __forceinline__ LdsBases lds_bases(int g, int c) {
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
      L.pv[rr][m4] = row * (kRowChunks * 16) + swz(row, 2 * m4 + ((c & 3) >> 1)) * 16 + 8 * (c & 1);
  }
  return L;
}

struct State {
  f32x4 oacc[kDv / 16];
  float m_run;  // running max of this lane's head (log2 domain)
  float l_run;  // this lane's share of the running sum
};

// Maximum over the four lanes l, l^16, l^32, l^48 (one head's four score
// groups), with the gfx950 row-swap permutes instead of LDS round trips.
__device__ __forceinline__ float max4_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One 32-token tile: scores, online softmax update, PV accumulation.
// hook(s) runs at the start of QK k-step s (the caller issues the next
// tile's loads there, spread over the MFMA work).
template <bool kFp8, typename Hook>
__device__ __forceinline__ void consume_tile(const char* tile, const float* scales, int nvalid, int g,
                                             const LdsBases& L, const bf16x8 (&qreg)[kDk / 32],
                                             float scale_log2, State& st, Hook&& hook) {
  constexpr int kSteps = kDk / 32;  // 18
  constexpr int kAhead = 4;
  constexpr int kMt = kDv / 16;     // 32 PV m-tiles
  constexpr int kAheadV = 4;        // V operands read ahead; the first ones load during the last QK steps
  bf16x8 va[kMt];
  auto load_v = [&](int m) {
    va[m] = join_tr(lds_read_tr(tile + L.pv[0][m & 3] + 128 * (m >> 2)),
                    lds_read_tr(tile + L.pv[1][m & 3] + 128 * (m >> 2)));
  };
  // ---- S^T = K Q^T: two 16-token blocks, chains interleaved ----
  // K operands are read kAhead k-steps ahead of their MFMAs (the last
  // kAheadV steps also read the first V operands); a scheduling barrier closes every
  // step so the reads cannot sink next to their use and LDS latency overlaps
  // MFMA work.
  f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  bf16x8 ka[kSteps][2];
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      ka[s][mt] = *reinterpret_cast<const bf16x8*>(tile + L.qk[mt][s & 1] + 128 * (s >> 1));
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    hook(s);
    if (s + kAhead < kSteps) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        ka[s + kAhead][mt] =
            *reinterpret_cast<const bf16x8*>(tile + L.qk[mt][(s + kAhead) & 1] + 128 * ((s + kAhead) >> 1));
    }
    if (s >= kSteps - kAheadV) load_v(s - (kSteps - kAheadV));
    sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s][0], qreg[s], sacc[0], 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s][1], qreg[s], sacc[1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- online softmax (log2 domain) ----
  float x[8];
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g + i;
      float v = sacc[mt][i] * scale_log2;
      if constexpr (kFp8) v *= scales[t];
      v = (t < nvalid) ? v : -INFINITY;
      x[4 * mt + i] = v;
      mx = fmaxf(mx, v);
    }
  mx = max4_rows(mx);
  // Lazy rescale: the reference max m_run only moves when a score exceeds it
  // by more than 2^8; until then p = 2^(s - m_run) <= 256, and O and l share
  // the same reference, so the result is unchanged. The first tile always
  // sets it (m_run = -inf).
  if (__any(mx > st.m_run + 8.f)) {
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);  // 0 on the first tile
    st.m_run = m_new;
    st.l_run *= alpha;
#pragma unroll
    for (int m = 0; m < kDv / 16; ++m) {
      // (the opaque step first keeps the AGPR -> VGPR copies inside this rare
      // branch; otherwise they are hoisted into every tile)
      asm volatile("" : "+a"(st.oacc[m]));
      st.oacc[m] *= alpha;
      asm volatile("" : "+a"(st.oacc[m]));
    }
  }
  const float m_new = st.m_run;
  float psum = 0.f;
  float pf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(x[j] - m_new);
    psum += p;
    float pv = p;
    if constexpr (kFp8) pv *= scales[16 * (j >> 2) + 4 * g + (j & 3)];
    pf[j] = pv;
  }
  const bf16x8 pb = pack8(pf);
  st.l_run += psum;
  // ---- O^T += V^T P^T: V^T operands read kAheadV m-tiles ahead (same scheme) ----
#pragma unroll
  for (int m = 0; m < kMt; ++m) {
    if (m + kAheadV < kMt) load_v(m + kAheadV);
    st.oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[m], pb, st.oacc[m], 0, 0, 0);
    // keep the accumulator in AGPRs across the tile loop (otherwise it is
    // copied between AGPRs and VGPRs every tile)
    asm volatile("" : "+a"(st.oacc[m]));
    __builtin_amdgcn_sched_barrier(0);
  }
}

constexpr int kStageBytes = kTileBytes;               // 36 KB: one 32-token bf16 tile
constexpr int kRawBytes = kBN * kDk;                   // 18 KB: one 32-token FP8 tile
constexpr int kRawWaveLoads = kRawBytes / 1024;        // 18 wave-wide 16-byte loads per tile
static_assert(kRawWaveLoads * 1024 == kRawBytes && kDk % 16 == 0, "raw FP8 tile layout");

// FP8 -> bf16 of one raw 32-token tile into a bf16 tile (swizzled layout),
// each byte converted once per workgroup; the tile's scales travel with it.
__device__ __forceinline__ void convert_tile(const char* raw, const float* sc_in, char* tile, float* sc_out) {
  const int tid = threadIdx.x;
  for (int S = tid; S < kBN * kFp8RowChunks; S += kThreads) {
    const int row = S / kFp8RowChunks, sc16 = S % kFp8RowChunks;
    const uint4 r = *reinterpret_cast<const uint4*>(raw + row * kDk + sc16 * 16);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, false));
      o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, true));
    }
    char* rowp = tile + row * (kRowChunks * 16);
    *reinterpret_cast<uint4*>(rowp + swz(row, 2 * sc16) * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(rowp + swz(row, 2 * sc16 + 1) * 16) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  if (tid < kBN) sc_out[tid] = sc_in[tid];
}

template <int N>
__device__ __forceinline__ void wait_ahead(int ahead) {
  // at most `ahead` further tiles of N loads each may still be in flight
  if (ahead >= 3) cpa::wait_vmcnt<3 * N>();
  else if (ahead == 2) cpa::wait_vmcnt<2 * N>();
  else if (ahead == 1) cpa::wait_vmcnt<N>();
  else cpa::wait_vmcnt<0>();
}

template <bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void decode_mla_kernel(cpa::DecodeMlaArgs a) {
  // bf16: 4 tile stages. FP8: 4 raw stages (18 KB) + 2 bf16 tiles, in the same bytes.
  __shared__ __attribute__((aligned(16))) char smem[4 * kStageBytes];
  __shared__ float rscale[4][4][64];  // FP8: [raw stage][wave copy][token]
  __shared__ float bscale[2][kBN];    // FP8: scales of the two bf16 tiles

  const int split = blockIdx.x % a.nsplit;
  const int b = blockIdx.x / a.nsplit;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int h = 16 * w + c;  // this lane's head (column of S^T and O^T)

  int64_t beg = a.kv_begin[b], end = a.kv_end[b];
  beg = beg < 0 ? 0 : (beg > a.Lmax ? a.Lmax : beg);
  end = end < beg ? beg : (end > a.Lmax ? a.Lmax : end);
  const int64_t len = end - beg;
  const int64_t t0 = beg + len * split / a.nsplit;
  const int64_t t1 = beg + len * (split + 1) / a.nsplit;
  const int ntok = (int)(t1 - t0);
  const int ntiles = (ntok + kBN - 1) / kBN;

  // Q^T operand: lane holds q[h][32s + 8g .. +8] for k-step s
  // (opaque after loading: otherwise the compiler re-loads these read-only
  // values from memory inside the tile loop instead of keeping them)
  bf16x8 qreg[kDk / 32];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h + 8 * g;
#pragma unroll
    for (int s = 0; s < kDk / 32; ++s) {
      qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
      asm volatile("" : "+v"(qreg[s]));
    }
  }

  State st;
#pragma unroll
  for (int m = 0; m < kDv / 16; ++m) {
    st.oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    asm volatile("" : "+a"(st.oacc[m]));
  }
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  const LdsBases L = lds_bases(g, c);

  if constexpr (!kFp8) {
    // ---- bf16: stage i % 4 holds tile i ----
    const uint16_t* base = reinterpret_cast<const uint16_t*>(a.cache) + (int64_t)b * a.c_b;
    uint32_t toff[kLdChunks];  // byte offset of this thread's chunks inside a full tile
#pragma unroll
    for (int k = 0; k < kLdChunks; ++k) {
      const int P = tid + kThreads * k;
      const int row = P / kRowChunks, pc = P % kRowChunks;
      toff[k] = (uint32_t)((row * a.c_t + swz(row, pc) * 8) * 2);
    }
    auto issue = [&](int i) {
      const int64_t tok0 = t0 + (int64_t)i * kBN;
      char* dst0 = smem + (i & 3) * kStageBytes + 64 * w * 16;
      if (tok0 + kBN <= t1) {
        const uint16_t* tb = base + tok0 * a.c_t;
#pragma unroll
        for (int k = 0; k < kLdChunks; ++k) cpa::lds_dma16_sbase<cpa::Policy::kStream>(tb, toff[k], cpa::lds_addr(dst0 + kThreads * k * 16));
      } else {  // last tile: tokens past the split re-read its last token (masked)
#pragma unroll
        for (int k = 0; k < kLdChunks; ++k) {
          const int P = tid + kThreads * k;
          const int row = P / kRowChunks, pc = P % kRowChunks;
          const int64_t tok = min(tok0 + row, t1 - 1);
          cpa::lds_dma16<cpa::Policy::kStream>(base + tok * a.c_t + swz(row, pc) * 8, cpa::lds_addr(dst0 + kThreads * k * 16));
        }
      }
    };
    for (int i = 0; i < 3 && i < ntiles; ++i) issue(i);
    for (int i = 0; i < ntiles; ++i) {
      wait_ahead<kLdChunks>(min(2, ntiles - 1 - i));  // tile i landed
      __syncthreads();  // tile i visible to all; every wave is done with tile i-1
      // tile i+3 goes into the stage tile i-1 used: a full tile's loads are
      // spread over the QK steps of tile i (one every other step), the
      // clamped last tile is issued at once
      const int64_t nxt0 = t0 + (int64_t)(i + 3) * kBN;
      const bool spread = (i + 3 < ntiles) && (nxt0 + kBN <= t1);
      if (i + 3 < ntiles && !spread) issue(i + 3);
      const uint16_t* ntb = base + nxt0 * a.c_t;
      char* ndst = smem + ((i + 3) & 3) * kStageBytes + 64 * w * 16;
      consume_tile<false>(smem + (i & 3) * kStageBytes, nullptr, min(kBN, ntok - kBN * i), g, L, qreg,
                          a.scale_log2, st, [&](int s) {
                            if (spread && (s & 1) == 0 && (s >> 1) < kLdChunks)
                              cpa::lds_dma16_sbase<cpa::Policy::kStream>(ntb, toff[s >> 1], cpa::lds_addr(ndst + kThreads * (s >> 1) * 16));
                          });
    }
  } else {
    // ---- FP8: raw stage u % 4 holds the e4m3 bytes of tile u; bf16 tile u % 2 ----
    char* raw = smem;                       // 4 x 18 KB
    char* btile = smem + 4 * kRawBytes;     // 2 x 36 KB
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)b * a.c_b;
    const float* sbase = a.kv_scale + (int64_t)b * a.s_b;
    // wave w issues the tile's wave-loads w, w+4, ... (5 for waves 0-1, 4 for 2-3)
    // plus one load of the tile's scales: per-wave counts for the waits
    const int n_mine = (kRawWaveLoads - w + 3) / 4;
    uint32_t roff[5];  // byte offset of this lane's 16-byte pieces inside a full raw tile
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int B = (w + 4 * k) * 1024 + 16 * lane;  // LDS byte of the piece, row-major [32][576]
      roff[k] = (uint32_t)((B / kDk) * a.c_t + (B % kDk));
    }
    auto issue = [&](int u) {
      const int64_t tok0 = t0 + (int64_t)u * kBN;
      char* dst = raw + (u & 3) * kRawBytes;
      if (tok0 + kBN <= t1) {
        const uint8_t* tb = base + tok0 * a.c_t;
#pragma unroll
        for (int k = 0; k < 5; ++k)
          if (k < n_mine) cpa::lds_dma16_sbase<cpa::Policy::kStream>(tb, roff[k], cpa::lds_addr(dst + (w + 4 * k) * 1024));
      } else {  // last tile: past the split, re-read its last token (masked)
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          if (k < n_mine) {
            const int B = (w + 4 * k) * 1024 + 16 * lane;
            const int64_t tok = min(tok0 + B / kDk, t1 - 1);
            cpa::lds_dma16<cpa::Policy::kStream>(base + tok * a.c_t + (B % kDk), cpa::lds_addr(dst + (w + 4 * k) * 1024));
          }
        }
      }
      const int64_t tok = min(tok0 + lane, t1 - 1);
      cpa::lds_dma4<cpa::Policy::kStream>(sbase + tok * a.s_t, cpa::lds_addr(&rscale[u & 3][w][0]));
    };
    auto wait_raw = [&](int ahead) {
      if (w < 2) wait_ahead<6>(ahead);  // 5 cache loads + 1 scale load per tile
      else wait_ahead<5>(ahead);
    };
    for (int u = 0; u < 4 && u < ntiles; ++u) issue(u);
    if (ntiles > 0) {
      wait_raw(min(3, ntiles - 1));  // raw 0 landed
      __syncthreads();
      convert_tile(raw, &rscale[0][0][0], btile, bscale[0]);
    }
    for (int u = 0; u < ntiles; ++u) {
      if (u + 1 < ntiles) wait_raw(min(u + 3, ntiles - 1) - (u + 1));  // raw u+1 landed
      __syncthreads();  // bf16 tile u complete; raw u+1 visible; tile u-1 and raw u fully consumed
      if (u + 4 < ntiles) issue(u + 4);  // into the raw stage of tile u
      if (u + 1 < ntiles)
        convert_tile(raw + ((u + 1) & 3) * kRawBytes, &rscale[(u + 1) & 3][0][0], btile + ((u + 1) & 1) * kStageBytes,
                     bscale[(u + 1) & 1]);
      consume_tile<true>(btile + (u & 1) * kStageBytes, bscale[u & 1], min(kBN, ntok - kBN * u), g, L, qreg,
                         a.scale_log2, st, [](int) {});
    }
  }

  // ---- finish: combine the four lanes of each head, normalise, store ----
  float l_run = st.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* op = a.o + (int64_t)split * a.o_s + (int64_t)b * a.o_b + (int64_t)h * a.o_h + 4 * g;
#pragma unroll
  for (int m = 0; m < kDv / 16; ++m) {
    const f32x4 v = st.oacc[m] * inv;
    *reinterpret_cast<f32x4*>(op + 16 * m) = v;
  }
  if (g == 0)
    a.lse[(int64_t)split * a.l_s + (int64_t)b * a.l_b + (int64_t)h * a.l_h] =
        l_run > 0.f ? (st.m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

}  // namespace

namespace cpa {

int launch_decode_mla(const DecodeMlaArgs& a, void* stream) {
  const dim3 grid((unsigned)((int64_t)a.B * a.nsplit));
  if (a.fp8)
    hipLaunchKernelGGL(decode_mla_kernel<true>, grid, dim3(kThreads), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(decode_mla_kernel<false>, grid, dim3(kThreads), 0, (hipStream_t)stream, a);
  return hipGetLastError();
}

}  // namespace cpa
