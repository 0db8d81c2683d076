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
//  * FP8: the tile is converted e4m3 -> bf16 exactly while it is written to
//    LDS; the per-token scale is folded into the score (s = scale_t q.e_t)
//    and into P (p_t * scale_t multiplies e_t in PV), never into K itself;
//  * LDS rows are 72 chunks of 16 bytes, XOR-swizzled inside aligned groups
//    of 8 chunks so that the 16 rows one MFMA operand read touches fall in
//    distinct banks.
#include <hip/hip_runtime.h>

#include "internal.h"

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

// Physical 16-byte chunk of logical chunk `c` in LDS row `r`.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

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

template <bool kFp8>
struct TileLoader {
  // registers holding the next tile while the current one is consumed
  uint4 r[kFp8 ? kFp8LdChunks : kLdChunks];
  float sc;
  // per-thread element offsets of its chunks inside a tile (loop invariant)
  uint32_t goff[kFp8 ? kFp8LdChunks : kLdChunks];

  __device__ __forceinline__ void init(const cpa::DecodeMlaArgs& a) {
    const int tid = threadIdx.x;
    if constexpr (!kFp8) {
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k) {
        const int P = tid + kThreads * k;
        const int row = P / kRowChunks, pc = P % kRowChunks;
        goff[k] = (uint32_t)(row * a.c_t + swz(row, pc) * 8);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kFp8LdChunks; ++k) {
        const int S = tid + kThreads * k;
        const int row = S / kFp8RowChunks, sc16 = S % kFp8RowChunks;
        goff[k] = (uint32_t)(row * a.c_t + sc16 * 16);
      }
    }
  }

  __device__ __forceinline__ void load(const cpa::DecodeMlaArgs& a, int b, int64_t tok0, int nvalid) {
    const int tid = threadIdx.x;
    if constexpr (!kFp8) {
      const uint16_t* base = reinterpret_cast<const uint16_t*>(a.cache) + (int64_t)b * a.c_b + tok0 * a.c_t;
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k) {
        const int row = (tid + kThreads * k) / kRowChunks;
        if (nvalid == kBN || row < nvalid)
          r[k] = *reinterpret_cast<const uint4*>(base + goff[k]);
        else
          r[k] = make_uint4(0, 0, 0, 0);
      }
    } else {
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)b * a.c_b + tok0 * a.c_t;
#pragma unroll
      for (int k = 0; k < kFp8LdChunks; ++k) {
        const int S = tid + kThreads * k;
        const int row = S / kFp8RowChunks;
        if (S < kFp8TileChunks && (nvalid == kBN || row < nvalid))
          r[k] = *reinterpret_cast<const uint4*>(base + goff[k]);
        else
          r[k] = make_uint4(0, 0, 0, 0);
      }
      sc = (tid < nvalid) ? a.kv_scale[(int64_t)b * a.s_b + (tok0 + tid) * a.s_t] : 0.f;
    }
  }

  __device__ __forceinline__ void store(char* tile, float* scales) {
    const int tid = threadIdx.x;
    if constexpr (!kFp8) {
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k)
        *reinterpret_cast<uint4*>(tile + (tid + kThreads * k) * 16) = r[k];
    } else {
#pragma unroll
      for (int k = 0; k < kFp8LdChunks; ++k) {
        const int S = tid + kThreads * k;
        if (S < kFp8TileChunks) {
          const int row = S / kFp8RowChunks, sc16 = S % kFp8RowChunks;
          const uint32_t w[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
          uint32_t o[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, false);
            bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, true);
            o[2 * q] = __builtin_bit_cast(uint32_t, lo);
            o[2 * q + 1] = __builtin_bit_cast(uint32_t, hi);
          }
          char* rowp = tile + row * (kRowChunks * 16);
          *reinterpret_cast<uint4*>(rowp + swz(row, 2 * sc16) * 16) = make_uint4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<uint4*>(rowp + swz(row, 2 * sc16 + 1) * 16) = make_uint4(o[4], o[5], o[6], o[7]);
        }
      }
      if (tid < kBN) scales[tid] = sc;
    }
  }
};

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

// One 32-token tile: scores, online softmax update, PV accumulation.
template <bool kFp8>
__device__ __forceinline__ void consume_tile(const char* tile, const float* scales, int nvalid, int g,
                                             const LdsBases& L, const bf16x8 (&qreg)[kDk / 32],
                                             float scale_log2, State& st) {
  // ---- S^T = K Q^T: two 16-token blocks ----
  f32x4 sacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDk / 32; ++s) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(tile + L.qk[mt][s & 1] + 128 * (s >> 1));
      sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[s], sacc[mt], 0, 0, 0);
    }
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
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m_run, mx);
  const float alpha = exp2f(st.m_run - m_new);  // 0 on the first tile
  st.m_run = m_new;
  float psum = 0.f;
  float pf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = exp2f(x[j] - m_new);
    psum += p;
    float pv = p;
    if constexpr (kFp8) pv *= scales[16 * (j >> 2) + 4 * g + (j & 3)];
    pf[j] = pv;
  }
  const bf16x8 pb = pack8(pf);
  st.l_run = st.l_run * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int m = 0; m < kDv / 16; ++m) st.oacc[m] *= alpha;
  }
  // ---- O^T += V^T P^T ----
#pragma unroll
  for (int m = 0; m < kDv / 16; ++m) {
    const i16x4 v0 = lds_read_tr(tile + L.pv[0][m & 3] + 128 * (m >> 2));
    const i16x4 v1 = lds_read_tr(tile + L.pv[1][m & 3] + 128 * (m >> 2));
    const bf16x8 va = join_tr(v0, v1);
    st.oacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, st.oacc[m], 0, 0, 0);
  }
}

template <bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void decode_mla_kernel(cpa::DecodeMlaArgs a) {
  __shared__ __attribute__((aligned(16))) char tiles[2][kTileBytes];
  __shared__ float scales[2][kBN];

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
  const int ntiles = (int)((t1 - t0 + kBN - 1) / kBN);

  // Q^T operand: lane holds q[h][32s + 8g .. +8] for k-step s
  bf16x8 qreg[kDk / 32];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_b + (int64_t)h * a.q_h + 8 * g;
#pragma unroll
    for (int s = 0; s < kDk / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  }

  State st;
#pragma unroll
  for (int m = 0; m < kDv / 16; ++m) st.oacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  const LdsBases L = lds_bases(g, c);

  auto tile_valid = [&](int it) {
    const int64_t tk = t0 + (int64_t)it * kBN;
    return (int)(t1 - tk < kBN ? t1 - tk : kBN);
  };

  TileLoader<kFp8> ld;
  ld.init(a);
  if (ntiles > 0) {
    ld.load(a, b, t0, tile_valid(0));
    ld.store(tiles[0], scales[0]);
    if (ntiles > 1) ld.load(a, b, t0 + kBN, tile_valid(1));
  }
  // Two tiles per trip so each stage's LDS base is a compile-time constant.
  for (int it = 0; it < ntiles; it += 2) {
    __syncthreads();  // tile `it` (stage 0) visible; stage 1 free
    if (it + 1 < ntiles) {
      ld.store(tiles[1], scales[1]);
      if (it + 2 < ntiles) ld.load(a, b, t0 + (int64_t)(it + 2) * kBN, tile_valid(it + 2));
    }
    consume_tile<kFp8>(tiles[0], scales[0], tile_valid(it), g, L, qreg, a.scale_log2, st);
    if (it + 1 >= ntiles) break;
    __syncthreads();  // tile `it + 1` (stage 1) visible; stage 0 free
    if (it + 2 < ntiles) {
      ld.store(tiles[0], scales[0]);
      if (it + 3 < ntiles) ld.load(a, b, t0 + (int64_t)(it + 3) * kBN, tile_valid(it + 3));
    }
    consume_tile<kFp8>(tiles[1], scales[1], tile_valid(it + 1), g, L, qreg, a.scale_log2, st);
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
