// Split-KV decode for GQA caches (f32, bf16, or FP8 E4M3 with a per-token
// scale), Q >= 1 query rows per request.
//
// What it computes: "How GPUs Share a Long Context During LLM Inference",
// 3.2-3.4: a rank runs attention of each request's new query over its own
// share of the cache and reports the partial output with its LSE; vLLM
// "Decode Context Parallelism", 4.1 and 5.4: the GQA kv heads are broadcast
// to their query heads (query head h reads kv head h / (Hq / Hkv)). FP8
// entries (1.2) are code * scale_t, the token's scale applying to its key
// and its value: s_t = scale_t q.k_t and p_t scale_t weights the value codes.
//
// Work decomposition (gfx950). One workgroup of four wavefronts per (query
// row, kv head, block of up to 16 query heads, split); the split is an even
// share of the row's [begin, end) range. Decode is HBM-bound (a few FLOP
// per cache byte), so the design is about streaming:
//  * Every wavefront runs its own pipeline over the split's tiles w, w + 4,
//    w + 8, ... (32 tokens for bf16 / FP8 rows up to 256 bytes, else 16):
//    direct global -> LDS loads (16 bytes per lane) into two stages that
//    only it reads, waited with its own vmcnt, so the main loop has no
//    barrier. The host sizes the split for one workgroup per CU: more
//    concurrent streams (two workgroups per CU, eight wavefronts per
//    workgroup, deeper stages) all measured slower on the whole-machine
//    stream.
//  * Both contractions run on MFMA with the 16 query heads as the N
//    dimension (heads past the group are zero columns): S^T = K Q^T with
//    16x16x32 bf16 (an f32 query against a bf16 / FP8 cache as bf16 hi + lo
//    parts, two MFMAs; f32 cache: 16x16x4 f32, which keeps fp32 products),
//    then O^T += V^T P^T with 16x16x16 bf16 (16x16x4 f32). Each lane ends
//    QK with four token scores of one head, which are exactly the B operand
//    of the PV MFMA, and every O^T value it accumulates belongs to that
//    same head, so the online softmax rescale is per lane.
//  * FP8 codes are converted in registers (E4M3 values are exact in bf16);
//    the token scale multiplies the score and the probability.
//  * K and V tiles are row-major with the 16-byte units of each row
//    XOR-swizzled by a bit permutation of the row index (swz), so every QK
//    operand read and every transposing V read touches each LDS bank the
//    minimum number of times, while each load instruction still fetches
//    whole cache rows: 1 KB of consecutive row bytes. (Loading 64-byte
//    pieces of 16 rows per instruction instead, which a unit-major tile
//    needs, streamed at 4.7 TB/s against 5.8-6.0 for whole rows.)
//  * The four wavefronts' states are merged in LDS at the end (the same
//    exact combine as the split merge) and written as the split's
//    normalised output and natural-log LSE.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_dma.h"
#include "paged.h"
#include "wave_ops.h"

namespace {

using cpa::Policy;
using cpa::max4_rows;
using cpa::sum4_rows;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

enum Dt { kF32 = 0, kBf16 = 1, kFp8 = 2 };

constexpr int kMaxThreads = 256;
constexpr int kHB = 16;   // query heads per workgroup (MFMA columns)
constexpr float kLn2 = 0.69314718055994531f;

template <int DT, int D>
struct Cfg {
  static constexpr int esz = DT == kF32 ? 4 : (DT == kBf16 ? 2 : 1);
  static constexpr int row = D * esz;             // bytes of one token's K (or V) row
  // tokens per tile: two 16-token MFMA blocks for rows up to 256 bytes (bf16
  // and FP8 caches), one for longer rows and f32 -- a tile carries 8 KB or
  // more of K + V, so the per-tile work (waits, softmax reductions) is
  // spread over enough bytes
  static constexpr int tok = (DT != kF32 && row <= 256) ? 32 : 16;
  static constexpr int nb = tok / 16;             // MFMA row blocks per tile
  static constexpr int kv_bytes = tok * row;      // K (or V) part of a tile
  static constexpr int loads = kv_bytes / 1024;   // wave-wide 16-byte loads per part
  static constexpr int scale_bytes = DT == kFp8 ? 4 * tok : 0;
  static constexpr int tile = 2 * kv_bytes + scale_bytes;
  static constexpr int stages = tile <= 4096 + 128 ? 4 : (tile <= 16384 + 128 ? 2 : 1);
  // wavefronts per workgroup, each with its own pipeline (eight, where they
  // fit, streamed the FP8 d = 128 cache at 4.5 TB/s against 4.9 with four)
  static constexpr int waves = 4;
  static constexpr int threads = 64 * waves;
  static constexpr int vm = 2 * loads + (DT == kFp8 ? 1 : 0);  // vector-memory ops per tile
  static constexpr int nacc = D / 16;             // O^T accumulators (16 dims x 16 heads each)
  static constexpr int stage_lds = waves * stages * tile;
  static constexpr int merge_lds = waves * kHB * (D + 3) * 4;  // O rows of D + 1, max, sum
  static constexpr int lds = stage_lds > merge_lds ? stage_lds : merge_lds;
  static_assert(loads >= 1 && kv_bytes % 1024 == 0, "whole wave-wide loads per tile part");
  static_assert((stages - 1) * vm <= 63, "vmcnt range");
  static_assert(D % 64 == 0, "head dim 64, 128 or 256");
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
}

// v rounded to the nearest bf16 (ties to even), as a float; finite inputs.
__device__ __forceinline__ float bf16_round(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

// Four E4M3 codes (one 32-bit word) -> four bf16 values, exactly.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true))};
}

template <typename T>
__device__ __forceinline__ T lds_ld(const char* p) {
  return *reinterpret_cast<const T*>(p);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) char*)(p));
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(__attribute__((address_space(3))) char*)(p));
}

// Wait until at most n of this wavefront's vector-memory operations are
// outstanding (n < 64; a run-time count, resolved by a switch).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define CPA_W(k) case k: cpa::wait_vmcnt<k>(); break;
    CPA_W(0) CPA_W(1) CPA_W(2) CPA_W(3) CPA_W(4) CPA_W(5) CPA_W(6) CPA_W(7) CPA_W(8) CPA_W(9)
    CPA_W(10) CPA_W(11) CPA_W(12) CPA_W(13) CPA_W(14) CPA_W(15) CPA_W(16) CPA_W(17) CPA_W(18)
    CPA_W(19) CPA_W(20) CPA_W(21) CPA_W(22) CPA_W(23) CPA_W(24) CPA_W(25) CPA_W(26) CPA_W(27)
    CPA_W(28) CPA_W(29) CPA_W(30) CPA_W(31) CPA_W(32)
#undef CPA_W
    default: cpa::wait_vmcnt<0>(); break;
  }
}

// Tiles are row-major (16 rows of `kRow` bytes) with the 16-byte units of
// row t stored XOR-swizzled: slot u of the row holds unit u ^ swz(t). The
// LDS has 64 banks of 4 bytes; a 16-byte read is served in four passes of
// 16 lanes (the lanes of one half-wave whose quad index (lane >> 2) & 7 has
// even, or odd, parity; measured), an 8-byte read (plain or transposing) in
// two passes of 32 consecutive lanes. The swizzle is a linear map of the
// row's low bits, found by search over every pass of every operand read of
// the nine dtype / head-dim tiles, under which each pass touches each bank
// once: the QK reads (16-byte: rows c, units 4k + g; FP8 8-byte: 16 rows,
// one unit half), the bf16 transposing V reads (rows 0..7 or 8..15, two
// units), the FP8 ones (8 rows, units n and n + 1) and the f32 V reads
// (16-byte: rows 4g + e, units 16N + c). Each load instruction still
// fetches whole rows (1 KB of consecutive row bytes).
template <int kRow>
__device__ __forceinline__ int swz(int t) {
  if constexpr (kRow >= 256)  // 16 units per 256 B: t0, t1, t0 ^ t2, t2 ^ t3
    return (t & 1) | (t & 2) | (((t ^ (t >> 2)) & 1) << 2) | ((((t >> 2) ^ (t >> 3)) & 1) << 3);
  else if constexpr (kRow == 128)  // 2 rows per 256 B: t1, t1 ^ t2, t1 ^ t3
    return ((t >> 1) & 1) | ((((t >> 1) ^ (t >> 2)) & 1) << 1) | ((((t >> 1) ^ (t >> 3)) & 1) << 2);
  else return (((t >> 2) & 1) << 1) | ((t >> 3) & 1);  // 64-byte rows: 4 rows per 256 B
}

template <int kRow>
__device__ __forceinline__ int tile_off(int t, int u) {
  return t * kRow + 16 * (u ^ swz<kRow>(t));
}

// kPaged: K, V and the scales are pools read through a block table (paged.h).
template <int DT, int D, bool kPaged>
__global__ __launch_bounds__(kMaxThreads) void decode_gqa_kernel(cpa::DecodeGqaArgs a) {
  using C = Cfg<DT, D>;
  __shared__ __attribute__((aligned(16))) char smem[C::lds];
  __shared__ int pages_s[kPaged ? cpa::kPageCap : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

  // ---- work unit: blockIdx = (u / 8) * 8Q + 8k + u % 8 keeps the Q rows of
  // one unit on one XCD (they read the same tiles through its L2) ----
  const int G = a.Hq / a.Hkv, HB = (G + kHB - 1) / kHB;
  const int64_t bx = blockIdx.x;
  const int64_t u = bx / (8 * (int64_t)a.Q) * 8 + bx % 8;
  const int k = (int)(bx / 8 % a.Q);
  const int64_t n_units = (int64_t)a.B * a.Hkv * HB * a.nsplit;
  if (u >= n_units) return;
  // the kv head varies fastest: the workgroups of one (request, head block,
  // split) -- consecutive block indices, on different XCDs -- read the same
  // tokens' rows of the Hkv heads at the same time
  const int kvh = (int)(u % a.Hkv);
  int64_t rest = u / a.Hkv;
  const int split = (int)(rest % a.nsplit);
  rest /= a.nsplit;
  const int hb = (int)(rest % HB);
  const int b = (int)(rest / HB);
  const int row = b * a.Q + k;
  const int h0 = kvh * G + hb * kHB;      // first query head of the block
  const int nh = min(kHB, G - hb * kHB);  // heads in the block

  int64_t beg = a.kv_begin[b], end = a.kv_end[row];
  beg = beg < 0 ? 0 : (beg > a.Lmax ? a.Lmax : beg);
  end = end < beg ? beg : (end > a.Lmax ? a.Lmax : end);
  const int64_t len = end - beg;
  const int64_t t0 = beg + len * split / a.nsplit;
  const int64_t t1 = beg + len * (split + 1) / a.nsplit;
  constexpr int kTok = C::tok;
  const int nt_all = (int)((t1 - t0 + kTok - 1) / kTok);
  constexpr int kWaves = C::waves;
  const int nt = nt_all > w ? (nt_all - w + kWaves - 1) / kWaves : 0;  // tiles w, w + waves, ...
  cpa::PagedRows pr{};
  if constexpr (kPaged) {
    pr = cpa::load_pages(pages_s, a.block_table + (int64_t)b * a.bt_b, t0, t1, a.page_shift, a.n_pages, tid,
                         kWaves * 64);
    __syncthreads();
  }

  // ---- this wavefront's loads ----
  const uint64_t kb = cpa::uniform_ptr(reinterpret_cast<const char*>(a.k) +
                                       ((int64_t)b * a.k_b + (int64_t)kvh * a.k_h) * C::esz);
  const uint64_t vb = cpa::uniform_ptr(reinterpret_cast<const char*>(a.v) +
                                       ((int64_t)b * a.v_b + (int64_t)kvh * a.v_h) * C::esz);
  const uint32_t kt = (uint32_t)(a.k_t * C::esz), vt = (uint32_t)(a.v_t * C::esz);  // token strides (bytes)
  char* wlds = smem + w * C::stages * C::tile;
  // cache policy: the Q rows of a request share tiles through L2; FP8 tiles
  // also stream faster without the nontemporal hint (4.9 against 4.6 TB/s
  // at 8 requests x 8 kv heads x 16384 tokens), bf16 faster with it (5.7
  // against 5.0)
  const bool reuse = a.Q > 1 || DT == kFp8;
  auto dma = [&](uint64_t base, uint32_t off, uint32_t dst) {
    if (reuse) cpa::lds_dma16_s<Policy::kReuse>(base, off, dst);
    else cpa::lds_dma16_s<Policy::kStream>(base, off, dst);
  };
  auto issue = [&](int j) {  // tile w + 4j into stage j % stages
    const int64_t tok0 = t0 + (int64_t)(w + kWaves * j) * kTok;
    const int lim = (int)min((int64_t)(kTok - 1), t1 - 1 - tok0);  // last valid row of the tile
    char* st = wlds + (j % C::stages) * C::tile;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wavefront's reads of the stage are done
    const uint64_t kbase = cpa::uniform_ptr(reinterpret_cast<const void*>(kb + (uint64_t)tok0 * kt));
    const uint64_t vbase = cpa::uniform_ptr(reinterpret_cast<const void*>(vb + (uint64_t)tok0 * vt));
    const uint32_t kdst = __builtin_amdgcn_readfirstlane(cpa::lds_addr(st));
    const uint32_t vdst = __builtin_amdgcn_readfirstlane(cpa::lds_addr(st + C::kv_bytes));
    // load i fills tile bytes 1024 i + 16 l: row t, slot u of it, which holds
    // the row's unit u ^ swz(t) (rows past a ragged end re-read the last
    // valid row; they are masked)
#pragma unroll
    for (int i = 0; i < C::loads; ++i) {
      const int q = 1024 * i + 16 * lane, t = q / C::row;
      const uint32_t src = 16u * (uint32_t)(((q % C::row) >> 4) ^ swz<C::row>(t));
      const uint32_t rr = (uint32_t)min(t, lim);
      if constexpr (kPaged) {  // every row its own pool row: 64-bit addresses
        const uint64_t prow = (uint64_t)pr.row(tok0 + rr);
        const char* ks = reinterpret_cast<const char*>(kb + prow * kt + src);
        const char* vs = reinterpret_cast<const char*>(vb + prow * vt + src);
        if (reuse) {
          cpa::lds_dma16<Policy::kReuse>(ks, kdst + 1024 * i);
          cpa::lds_dma16<Policy::kReuse>(vs, vdst + 1024 * i);
        } else {
          cpa::lds_dma16<Policy::kStream>(ks, kdst + 1024 * i);
          cpa::lds_dma16<Policy::kStream>(vs, vdst + 1024 * i);
        }
      } else {
        dma(kbase, rr * kt + src, kdst + 1024 * i);
        dma(vbase, rr * vt + src, vdst + 1024 * i);
      }
    }
    if constexpr (DT == kFp8) {
      const int64_t srow = kPaged ? pr.row(tok0 + min(lane, lim)) : tok0 + min(lane, lim);
      const float* sp = a.kv_scale + (int64_t)b * a.s_b + srow * a.s_t;
      const uint32_t sdst = __builtin_amdgcn_readfirstlane(cpa::lds_addr(st + 2 * C::kv_bytes));
      if (lane < kTok) {
        if (reuse) cpa::lds_dma4<Policy::kReuse>(sp, sdst);
        else cpa::lds_dma4<Policy::kStream>(sp, sdst);
      }
    }
  };
  const int pro = min(nt, C::stages);
  for (int j = 0; j < pro; ++j) issue(j);

  // ---- query operands (heads past the block are zero columns) ----
  const bool qbf = a.q_bf16 != 0;
  // every lane loads a valid head's row (lanes past the block reuse the
  // last head and are zeroed afterwards): unconditional loads issue back to
  // back instead of one guarded round trip per element
  const int64_t qrow = (int64_t)b * a.q_b + (int64_t)k * a.q_q + (int64_t)(h0 + min(c, nh - 1)) * a.q_h;
  const float qmask = c < nh ? 1.f : 0.f;
  // the lane's query values: f32 path dims 16 m + 4 g + x (index 4 m + x),
  // bf16 path dims 32 s + 8 g + e (index 8 s + e); one branch on the query
  // dtype around all the loads
  constexpr int kQv = D / 4;
  float qv[kQv];
  auto qdim = [&](int i) { return DT == kF32 ? 16 * (i >> 2) + 4 * g + (i & 3) : 32 * (i >> 3) + 8 * g + (i & 7); };
  if (qbf) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow;
#pragma unroll
    for (int i = 0; i < kQv; ++i) qv[i] = __uint_as_float((uint32_t)qp[qdim(i)] << 16);
  } else {
    const float* qp = reinterpret_cast<const float*>(a.q) + qrow;
#pragma unroll
    for (int i = 0; i < kQv; ++i) qv[i] = qp[qdim(i)];
  }
#pragma unroll
  for (int i = 0; i < kQv; ++i) qv[i] *= qmask;
  // bf16 path: an f32 query is split into bf16 hi + lo parts (q = hi + lo to
  // 2^-16 relative), two MFMAs per k-step; f32 path: the values themselves
  bf16x8 qb[D / 32], qlo[D / 32];
  float qf[D / 16][4];
  if constexpr (DT == kF32) {
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
#pragma unroll
      for (int x = 0; x < 4; ++x) qf[m][x] = qv[4 * m + x];
  } else {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const float* v = qv + 8 * s;
      float r[8];
      qb[s] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                                                    pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])));
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = v[e] - bf16_round(v[e]);  // exact; 0 for a bf16 query
      qlo[s] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]),
                                                     pack_bf16(r[4], r[5]), pack_bf16(r[6], r[7])));
    }
  }

  // ---- main loop: this wavefront's tiles ----
  f32x4 acc[C::nacc];
#pragma unroll
  for (int n = 0; n < C::nacc; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = a.scale_log2;
  for (int j = 0; j < nt; ++j) {
    // tile j landed: the loads of the tiles issued after it may be in flight
    const int after = min(nt, j + C::stages) - (j + 1);
    wait_vm(after * C::vm);
    const char* T = wlds + (j % C::stages) * C::tile;
    const char* V = T + C::kv_bytes;
    const int64_t tok0 = t0 + (int64_t)(w + kWaves * j) * kTok;
    const int lim = (int)min((int64_t)(kTok - 1), t1 - 1 - tok0);

    // S^T per 16-token block bk (16 tokens x 16 heads): lane (head c, group
    // g) gets tokens 16 bk + 4g .. + 3
    f32x4 s[C::nb];
#pragma unroll
    for (int bk = 0; bk < C::nb; ++bk) {
      const char* Tb = T + 16 * bk * C::row;
      s[bk] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DT == kF32) {
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
          const f32x4 kv = lds_ld<f32x4>(Tb + tile_off<C::row>(c, 4 * m + g));  // dims 16m + 4g .. + 3 of token c
#pragma unroll
          for (int x = 0; x < 4; ++x) s[bk] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[x], qf[m][x], s[bk], 0, 0, 0);
        }
      } else if constexpr (DT == kBf16) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 kv = lds_ld<bf16x8>(Tb + tile_off<C::row>(c, 4 * ks + g));  // dims 32ks + 8g .. + 7
          s[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[ks], s[bk], 0, 0, 0);
          if (!qbf) s[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[ks], s[bk], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const u32x2 raw = lds_ld<u32x2>(Tb + tile_off<C::row>(c, 2 * ks + (g >> 1)) + 8 * (g & 1));
          const u32x2 lo = fp8x4_to_bf16(raw[0]), hi = fp8x4_to_bf16(raw[1]);
          const bf16x8 kv = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], hi[0], hi[1]));
          s[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[ks], s[bk], 0, 0, 0);
          if (!qbf) s[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[ks], s[bk], 0, 0, 0);
        }
      }
    }

    // online softmax (log2 domain) of head c over the tile
    f32x4 ts[C::nb];
    float x[C::nb][4];
    float mx = -INFINITY;
#pragma unroll
    for (int bk = 0; bk < C::nb; ++bk) {
      ts[bk] = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (DT == kFp8) ts[bk] = lds_ld<f32x4>(T + 2 * C::kv_bytes + 64 * bk + 16 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[bk][i] = s[bk][i] * ts[bk][i] * sl2;
        if (lim < kTok - 1 && 16 * bk + 4 * g + i > lim) x[bk][i] = -INFINITY;
        mx = fmaxf(mx, x[bk][i]);
      }
    }
    const float mt = max4_rows(mx);
    // the reference max moves only when a score passes it by 2^8 (p <= 256
    // meanwhile; O and the sum share the reference), so rescaling is rare
    const float m_new = mt > m_run + 8.f ? mt : m_run;  // finite: every tile holds a valid token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
    float p[C::nb][4], psum = 0.f;
#pragma unroll
    for (int bk = 0; bk < C::nb; ++bk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[bk][i] = __builtin_amdgcn_exp2f(x[bk][i] - m_new);
        psum += p[bk][i];
      }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int n = 0; n < C::nacc; ++n) acc[n] *= alpha;
    }

    // O^T += V^T P^T, block by block
#pragma unroll
    for (int bk = 0; bk < C::nb; ++bk) {
      const char* Vb = V + 16 * bk * C::row;
      if constexpr (DT == kF32) {
        // k-step e takes token 4g + e of every group; lane (c, g) reads dims
        // 64N + 4c .. + 3, feeding MFMA (N, x) at row c (dim 64N + 4c + x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int N = 0; N < D / 64; ++N) {
            const f32x4 vv = lds_ld<f32x4>(Vb + tile_off<C::row>(4 * g + e, 16 * N + c));
#pragma unroll
            for (int xx = 0; xx < 4; ++xx)
              acc[4 * N + xx] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[xx], p[bk][e], acc[4 * N + xx], 0, 0, 0);
          }
      } else {
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = p[bk][i] * ts[bk][i];
        const i16x4 pb = __builtin_bit_cast(i16x4, u32x2{pack_bf16(pw[0], pw[1]), pack_bf16(pw[2], pw[3])});
        if constexpr (DT == kBf16) {
          // lane 4j + i of group g addresses token 4g + j, dims 16n + 4i .. + 3
          const int tk = 4 * g + (c >> 2);
#pragma unroll
          for (int n = 0; n < C::nacc; ++n) {
            const i16x4 va = lds_read_tr16(Vb + tile_off<C::row>(tk, 2 * n + ((c & 3) >> 1)) + 8 * (c & 1));
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[n], 0, 0, 0);
          }
        } else {
          // lanes 2j, 2j + 1 of group g address row j: token 4g + (j & 3),
          // dims of unit n + (j >> 2); one read feeds n-blocks n and n + 1
          const int jr = c >> 1, tk = 4 * g + (jr & 3);
#pragma unroll
          for (int n = 0; n < C::nacc; n += 2) {
            const i32x2 raw = lds_read_tr8(Vb + tile_off<C::row>(tk, n + (jr >> 2)) + 8 * (c & 1));
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, fp8x4_to_bf16(raw[0])), pb,
                                                                acc[n], 0, 0, 0);
            acc[n + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(i16x4, fp8x4_to_bf16(raw[1])), pb, acc[n + 1], 0, 0, 0);
          }
        }
      }
    }
    if (j + C::stages < nt) issue(j + C::stages);
  }

  // ---- merge the wavefronts' states and write the split's result ----
  const float l_run = sum4_rows(l_part);
  __syncthreads();  // every wavefront is done with its stages
  // [waves][16][D + 1] unnormalised O: the odd row stride puts the 16 heads
  // a store instruction writes in different banks
  constexpr int Dp = D + 1;
  float* mo = reinterpret_cast<float*>(smem);
  float* mm = mo + kWaves * kHB * Dp;               // [waves][16] running max
  float* ml = mm + kWaves * kHB;                    // [waves][16] running sum
#pragma unroll
  for (int n = 0; n < C::nacc; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // lane (head c, group g) holds O^T rows 4g + r of accumulator n
      const int d = DT == kF32 ? 64 * (n / 4) + 4 * (4 * g + r) + (n % 4) : 16 * n + 4 * g + r;
      mo[(w * kHB + c) * Dp + d] = acc[n][r];
    }
  if (g == 0) {
    mm[w * kHB + c] = m_run;
    ml[w * kHB + c] = l_run;
  }
  __syncthreads();
  float* o = a.o + (int64_t)split * a.o_s + (int64_t)row * a.o_b;
  for (int e = tid; e < nh * D; e += C::threads) {
    const int h = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, mm[v * kHB + h]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float f = __builtin_amdgcn_exp2f(mm[v * kHB + h] - M);  // 0 for an empty wavefront
        num += f * mo[(v * kHB + h) * Dp + d];
        den += f * ml[v * kHB + h];
      }
    }
    o[(int64_t)(h0 + h) * a.o_h + d] = den > 0.f ? num / den : 0.f;
    if (d == 0) {
      a.lse[(int64_t)split * a.l_s + (int64_t)row * a.l_b + (int64_t)(h0 + h) * a.l_h] =
          den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
    }
  }
}

template <int DT, bool kPaged>
int launch_dt(const cpa::DecodeGqaArgs& a, dim3 grid, hipStream_t st) {
  switch (a.D) {
    case 64:
      hipLaunchKernelGGL((decode_gqa_kernel<DT, 64, kPaged>), grid, dim3(Cfg<DT, 64>::threads), 0, st, a);
      break;
    case 128:
      hipLaunchKernelGGL((decode_gqa_kernel<DT, 128, kPaged>), grid, dim3(Cfg<DT, 128>::threads), 0, st, a);
      break;
    case 256:
      hipLaunchKernelGGL((decode_gqa_kernel<DT, 256, kPaged>), grid, dim3(Cfg<DT, 256>::threads), 0, st, a);
      break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <bool kPaged>
int launch_paging(const cpa::DecodeGqaArgs& a, dim3 grid, hipStream_t st) {
  if (a.kv_dtype == CPA_F32) return launch_dt<kF32, kPaged>(a, grid, st);
  if (a.kv_dtype == CPA_BF16) return launch_dt<kBf16, kPaged>(a, grid, st);
  return launch_dt<kFp8, kPaged>(a, grid, st);
}

}  // namespace

namespace cpa {

int gqa_head_blocks(int G) { return (G + kHB - 1) / kHB; }

int launch_decode_gqa(const DecodeGqaArgs& a, void* stream) {
  const int64_t units = (int64_t)a.B * a.Hkv * gqa_head_blocks(a.Hq / a.Hkv) * a.nsplit;
  const dim3 grid((unsigned)((units + 7) / 8 * 8 * a.Q));
  hipStream_t st = (hipStream_t)stream;
  return a.block_table != nullptr ? launch_paging<true>(a, grid, st) : launch_paging<false>(a, grid, st);
}

}  // namespace cpa
