// Wave-specialised variant of the MLA core: 8 wavefronts, two per SIMD.
//
// Same computation as mla_core.h (attention of one query's 64 heads over a
// contiguous range of a latent cache, 32-token LDS tiles, one barrier per
// tile, P exchanged through LDS), split by role so that every SIMD runs two
// independent instruction streams:
//  * QK wavefronts 0-3: wave w computes the scores of heads 16w..16w+15
//    (36 MFMAs per tile, K from LDS, Q^T in registers), the online softmax,
//    and stores P and the per-head rescale factor;
//  * PV wavefronts 4-7: wave w accumulates O^T for value dims
//    128w..128w+127 of all heads (32 MFMAs per tile, V^T from LDS with
//    transposing reads, P^T from LDS) and issues the direct global -> LDS
//    loads of the tiles.
// With one wavefront per SIMD the in-order issue left the matrix unit idle
// whenever the wave waited on an LDS operand, a dependent softmax step or
// the barrier; here the other role's wavefront issues meanwhile. Each role
// holds only its own state (Q^T and the softmax statistics, or O), which
// keeps both within the 256 registers a wavefront gets at two per SIMD.
//
// Step i (after the barrier that publishes P_i and tile i+1):
//   QK: S_{i+1} = K_{i+1} Q^T, softmax -> P_{i+1}, alpha_{i+1}
//   PV: O = alpha_i O + V_i^T P_i; loads of tile i+3 into tile i-1's stage
#pragma once

#include <type_traits>

#include "mla_core.h"

namespace cpa {
namespace mla {

constexpr int kWsThreads = 512;  // 4 QK + 4 PV wavefronts

struct QkStat {
  float m_run;  // running reference max of head 16w + c (log2 domain)
  float l_run;  // this lane's share of the head's running sum
};

// The tile sequence of a range: step i consumes tile (i + rot) mod ntiles.
// The rotation is a per-workgroup hash, so workgroups that start together do
// not all read the same tile offsets of their ranges at once (the order of
// tiles does not change the result beyond rounding: online softmax).
struct Tiles {
  int64_t t0, t1;
  int ntok, ntiles, rot;
  __device__ __forceinline__ Tiles(int64_t a, int64_t b, uint32_t rot_seed) : t0(a), t1(b) {
    ntok = (int)(b - a);
    ntiles = ntok > 0 ? (ntok + kBN - 1) / kBN : 0;
    rot = ntiles > 0 ? (int)(rot_seed % (uint32_t)ntiles) : 0;
  }
  __device__ __forceinline__ int phys(int i) const {
    const int t = i + rot;
    return t >= ntiles ? t - ntiles : t;
  }
  __device__ __forceinline__ int nvalid(int i) const { return min(kBN, ntok - kBN * phys(i)); }
};

__device__ __forceinline__ const char* ws_tile(const Lds& S, int i) { return S.tiles + (i & 3) * kTileBytes; }

// QK role. Barriers: 1 (tile 0) + (ntiles - 1) (loop) + 1 (after the loop).
// tile(i): LDS bf16 tile of step i. kMask: mask(i) gives the selection bits
// of tile i (index lists).
template <bool kMask = false, typename TileFn, typename MaskFn>
__device__ __forceinline__ void ws_qk(const Tiles& T, int w, int g, int c, const LdsBases& L,
                                      const bf16x8 (&qreg)[kQSteps], float scale_log2, QkStat& st, const Lds& S,
                                      TileFn&& tile, MaskFn&& mask) {
  if (T.ntiles <= 0) return;
  const TokScale tsc{};  // unused: bf16 caches carry no scale
  auto step = [&](int i, auto parity) {  // scores and P of tile i; parity = i & 1
    constexpr int P = decltype(parity)::value;
    f32x4 sacc[2];
    qk_tile(tile(i), L, qreg, sacc, [](int) {}, [](int) {});
    Soft sm;
    soft_scores<false, kMask>(sm, sacc, T.nvalid(i), g, scale_log2, tsc, kMask ? mask(i) : 0xffffffffu);
    soft_ref(sm, st, scale_log2);
    soft_exp<false, 0, kMask>(sm, st, tsc, scale_log2);
    soft_exp<false, 4, kMask>(sm, st, tsc, scale_log2);
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

// PV role, bf16 cache rows `base` (row 0) with `c_t` elements per row;
// rows.row(t) is the row of token t (the token itself, or its row in a paged
// pool: every load then takes its own address). tp = thread index inside the
// role (0..255).
template <Policy P, typename Rows = LinearRows>
__device__ __forceinline__ void ws_pv(const Tiles& T, const uint16_t* base, int64_t c_t, int tp, int w, int g, int c,
                                      const LdsBases& L, f32x4 (&oacc)[kMv][4], const Lds& S,
                                      const Rows& rows = Rows{}) {
  if (T.ntiles <= 0) return;
  uint32_t toff[kLdChunks];  // byte offset of this thread's chunks inside a full tile
#pragma unroll
  for (int k = 0; k < kLdChunks; ++k) {
    const int Pc = tp + kThreads * k;
    const int row = Pc / kRowChunks, pc = Pc % kRowChunks;
    toff[k] = (uint32_t)((row * c_t + swz(row, pc) * 8) * 2);
  }
  auto stage = [&](int i) { return S.tiles + (i & 3) * kTileBytes + 64 * w * 16; };
  auto issue = [&](int i) {  // all loads of tile i at once
    const int64_t tok0 = T.t0 + (int64_t)T.phys(i) * kBN;
    char* dst0 = stage(i);
    if (tok0 + kBN <= T.t1 && rows.consecutive(tok0, tok0 + kBN - 1)) {  // one base, per-thread offsets
      const uint16_t* tb = base + rows.row(tok0) * c_t;
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k) lds_dma16_sbase<P>(tb, toff[k], lds_addr(dst0 + kThreads * k * 16));
    } else {
#pragma unroll
      for (int k = 0; k < kLdChunks; ++k) {
        const int Pc = tp + kThreads * k;
        const int row = Pc / kRowChunks, pc = Pc % kRowChunks;
        const int64_t tok = min(tok0 + row, T.t1 - 1);
        lds_dma16<P>(base + rows.row(tok) * c_t + swz(row, pc) * 8, lds_addr(dst0 + kThreads * k * 16));
      }
    }
  };
  const int n = T.ntiles;
  for (int i = 0; i < 3 && i < n; ++i) issue(i);
  wait_ahead<kLdChunks>(min(2, n - 1));  // tile 0 landed
  __syncthreads();

  // O = alpha_i O + V_i^T P_i, with the loads of tile `nxt` spread over the
  // m-steps when it is a full tile (hook at m-step m)
  constexpr int kAheadV = 4;
  auto pv = [&](int i, auto&& hook) {
    const char* cur = ws_tile(S, i);
    const float* acur = S.alpha + kH * (i & 1);
    const char* pcur = S.p + kH * kPRowBytes * (i & 1);
    float al[4];
    bf16x8 pb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      al[hb] = acur[16 * hb + c];
      pb[hb] = *reinterpret_cast<const bf16x8*>(pcur + p_off(16 * hb + c, g));
    }
    bf16x8 va[kMv];
    auto load_v = [&](int m) {
      va[m] = join_tr(lds_read_tr(cur + L.pv[0][m & 3] + 128 * (m >> 2)),
                      lds_read_tr(cur + L.pv[1][m & 3] + 128 * (m >> 2)));
    };
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
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        oacc[m][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[m], pb[hb], oacc[m][hb], 0, 0, 0);
    }
  };

  for (int i = 0; i + 1 < n; ++i) {
    wait_ahead<kLdChunks>(min(1, n - 2 - i));  // tile i+1 landed
    __syncthreads();                            // P_i visible; every wave is done with tile i-1
    // tile i+3 goes into the stage tile i-1 used: a full tile's loads are
    // spread over the m-steps (two at the first), the clamped last tile is
    // issued at once
    const int64_t nxt0 = T.t0 + (int64_t)T.phys(i + 3 < n ? i + 3 : 0) * kBN;
    const bool spread = (i + 3 < n) && (nxt0 + kBN <= T.t1) && rows.consecutive(nxt0, nxt0 + kBN - 1);
    if (i + 3 < n && !spread) issue(i + 3);
    const uint64_t ntb = uniform_ptr(base + (Rows::kLinear ? nxt0 : (spread ? rows.row(nxt0) : 0)) * c_t);
    const uint32_t ndst = __builtin_amdgcn_readfirstlane(lds_addr(stage(i + 3)));
    pv(i, [&](int m) {
      if (spread) {
        if (m == 0) lds_dma16_s<P>(ntb, toff[0], ndst);
        lds_dma16_s<P>(ntb, toff[m + 1], ndst + kThreads * (m + 1) * 16);
      }
    });
  }
  __syncthreads();  // P of the last tile visible
  pv(n - 1, [](int) {});
}

// PV role of index-list (sparse) attention: the rows of a tile are the cache
// rows named by list entries (index ring: mla_core.h, kIdxSlots). Each PV
// wavefront copies the 32 entries of a tile into its own LDS
// ring slot (one 4-byte direct load per lane), five tiles ahead; per step
// i: the entries of tile i+5, then the nine row loads of tile i+3 with
// addresses from the ring (spread over the m-steps). Vector-memory loads
// complete in issue order, so the wait for tile i+1 (at most 1 + 9 later
// loads) also covers the entries of tiles up to i+3. The QK wavefronts read
// the selection bits of a tile from the ring of the PV wavefront with the
// same index after the barrier that publishes the tile.
template <Policy P>
__device__ __forceinline__ void ws_pv_gather(const Tiles& T, const uint16_t* base, int64_t c_t, const int32_t* ilist,
                                             int nrows, int tp, int w, int g, int c, const LdsBases& L,
                                             f32x4 (&oacc)[kMv][4], const Lds& S, char* ring) {
  if (T.ntiles <= 0) return;
  const int lane = tp & 63;
  const int n = T.ntiles;
  const uint32_t rowbytes = (uint32_t)c_t * 2u;  // the host bounds nrows * rowbytes below 2^32
  uint32_t rinfo[kLdChunks];  // tile row (high half) and swizzled source byte offset of this thread's chunks
#pragma unroll
  for (int k = 0; k < kLdChunks; ++k) {
    const int Pc = tp + kThreads * k;
    const int row = Pc / kRowChunks, pc = Pc % kRowChunks;
    rinfo[k] = ((uint32_t)row << 16) | (uint32_t)(swz(row, pc) * 16);
  }
  const char* wring = ring + w * (kIdxSlots * kIdxSlotBytes);
  const uint32_t wring_lds = __builtin_amdgcn_readfirstlane(lds_addr(wring));
  const uint64_t ibase = uniform_ptr(ilist), cbase = uniform_ptr(base);
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
  auto offsets = [&](int t, uint32_t (&voff)[kLdChunks]) {
#pragma unroll
    for (int k = 0; k < kLdChunks; ++k) voff[k] = row_of(t, (int)(rinfo[k] >> 16)) * rowbytes + (rinfo[k] & 0xffffu);
  };
  auto dst = [&](int t) {
    return __builtin_amdgcn_readfirstlane(lds_addr(S.tiles + (t & 3) * kTileBytes + 64 * w * 16));
  };
  auto issue_tile = [&](int t) {
    uint32_t voff[kLdChunks];
    offsets(t, voff);
    const uint32_t d = dst(t);
#pragma unroll
    for (int k = 0; k < kLdChunks; ++k) lds_dma16_s<P>(cbase, voff[k], d + kThreads * k * 16);
  };
  // ---- prologue: entries of tiles 0..4, rows of tiles 0..2 ----
  issue_idx(0);
  issue_idx(1);
  issue_idx(2);
  wait_vmcnt<2>();  // entries of tile 0
  issue_tile(0);
  issue_idx(3);
  if (n > 1) {
    wait_vmcnt<11>();  // entries of tile 1 (then: 2, rows 0, 3)
    issue_tile(1);
  }
  issue_idx(4);
  if (n > 2) {
    wait_vmcnt<20>();  // entries of tile 2 (then: rows 0, 3, rows 1, 4)
    issue_tile(2);
  }
  // rows of tile 0 landed (after them: entries 3, rows 1, entries 4, rows 2)
  if (n > 2) wait_vmcnt<20>();
  else if (n == 2) wait_vmcnt<11>();
  else wait_vmcnt<2>();
  __syncthreads();

  constexpr int kAheadV = 4;
  auto pv = [&](int i, auto&& hook) {
    const char* cur = ws_tile(S, i);
    const float* acur = S.alpha + kH * (i & 1);
    const char* pcur = S.p + kH * kPRowBytes * (i & 1);
    float al[4];
    bf16x8 pb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      al[hb] = acur[16 * hb + c];
      pb[hb] = *reinterpret_cast<const bf16x8*>(pcur + p_off(16 * hb + c, g));
    }
    bf16x8 va[kMv];
    auto load_v = [&](int m) {
      va[m] = join_tr(lds_read_tr(cur + L.pv[0][m & 3] + 128 * (m >> 2)),
                      lds_read_tr(cur + L.pv[1][m & 3] + 128 * (m >> 2)));
    };
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
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        oacc[m][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[m], pb[hb], oacc[m][hb], 0, 0, 0);
    }
  };
  for (int i = 0; i + 1 < n; ++i) {
    // rows of tile i+1 landed: after them only the entries of tile i+4 and the rows of tile i+2
    if (i + 2 < n) wait_vmcnt<10>();
    else wait_vmcnt<1>();
    __syncthreads();  // P_i and tile i+1 visible; every wave is done with tile i-1 and P_{i-1}
    issue_idx(i + 5);
    const bool more = i + 3 < n;
    uint32_t voff[kLdChunks];
    offsets(i + 3, voff);
    const uint32_t ndst = dst(i + 3);
    pv(i, [&](int m) {
      if (more) {
        if (m == 0) lds_dma16_s<P>(cbase, voff[0], ndst);
        lds_dma16_s<P>(cbase, voff[m + 1], ndst + kThreads * (m + 1) * 16);
      }
    });
  }
  __syncthreads();  // P of the last tile visible
  pv(n - 1, [](int) {});
  wait_vmcnt<0>();  // entry loads issued past the last tile have landed
}

}  // namespace mla
}  // namespace cpa
