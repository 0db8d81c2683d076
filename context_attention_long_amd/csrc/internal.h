// Internal declarations of libcpattn: error state, tensor views handed to the
// kernels, and the kernel launchers. Not part of the ABI.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "cpattn.h"

namespace cpa {

// Thread-local last-error message (cpa_last_error).
void clear_error();
cpa_status fail(cpa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// ---- kernel-side argument blocks (plain data, passed by value) ----

struct MergeArgs {
  const float* o;       // [S, N, H, Dv]
  const float* lse;     // [S, N, H]
  void* out;            // [N, H, Dv] f32 or bf16
  float* lse_out;       // [N, H] or null
  int64_t o_s, o_n, o_h;        // element strides of o (Dv contiguous)
  int64_t l_s, l_n, l_h;        // strides of lse
  int64_t out_n, out_h;         // strides of out
  int64_t lo_n, lo_h;           // strides of lse_out
  int32_t S, N, H, Dv;
  int32_t out_bf16;
};

struct DecodeGqaArgs {
  const void* q;        // [B, Hq, D] f32 or bf16
  const void* k;        // [B, Lmax, Hkv, D] f32, bf16 or E4M3 bytes
  const void* v;        // [B, Lmax, Hkv, D] same dtype as k
  const float* kv_scale;  // [B, Lmax] per-token scale of an FP8 cache (key and value), else null
  int64_t s_b, s_t;
  const int32_t* kv_begin;
  const int32_t* kv_end;
  float* o;             // [nsplit, B, Hq, D] (or o_part when nsplit == 1)
  float* lse;           // [nsplit, B, Hq]
  int64_t q_b, q_h;
  int64_t k_b, k_t, k_h;
  int64_t v_b, v_t, v_h;
  int64_t o_s, o_b, o_h;        // strides of the partial output
  int64_t l_s, l_b, l_h;
  int32_t B, Hq, Hkv, D, Lmax, nsplit;
  int32_t q_bf16, kv_dtype;
  float scale_log2;             // softmax scale * log2(e)
  // Q query rows per request (speculative / MTP decode): row k of request b
  // is q + b*q_b + k*q_q, reads [kv_begin[b], kv_end[b*Q + k]) and writes
  // output row b*Q + k (strides o_b / l_b then step one row).
  int32_t Q;
  int64_t q_q;
  // Paged cache when block_table is set (paged.h): token t of request b is
  // pool row block_table[b*bt_b + (t >> page_shift)] * 2^page_shift +
  // (t & (2^page_shift - 1)); k_b, v_b and s_b are then 0.
  const int32_t* block_table;
  int64_t bt_b;
  int32_t page_shift, n_pages;
};

struct DecodeMlaArgs {
  const uint16_t* q;    // [B, H, 576] bf16
  const void* cache;    // [B, Lmax, 576] bf16 words or E4M3 bytes (one kv head)
  const float* kv_scale;  // [B, Lmax] (FP8) or null
  const int32_t* kv_begin;
  const int32_t* kv_end;
  float* o;             // [nsplit, B, H, 512]
  float* lse;           // [nsplit, B, H]
  int64_t q_b, q_h;
  int64_t c_b, c_t;     // cache strides (elements of its dtype)
  int64_t s_b, s_t;     // kv_scale strides
  int64_t o_s, o_b, o_h;
  int64_t l_s, l_b, l_h;
  int32_t B, H, Lmax, nsplit;
  int32_t fp8;
  float scale_log2;
  // Q query rows per request, as in DecodeGqaArgs.
  int32_t Q;
  int64_t q_q;
  // Paged cache, as in DecodeGqaArgs (c_b and s_b are then 0).
  const int32_t* block_table;
  int64_t bt_b;
  int32_t page_shift, n_pages;
};

struct SparseMlaArgs {
  const uint16_t* q;      // [N, 64, 576] bf16
  const void* cache;      // [B, Lmax, 576] bf16 words or E4M3 bytes (one kv head)
  const float* kv_scale;  // [B, Lmax] per-token scale of an FP8 cache, else null
  int64_t s_b, s_t;
  const int32_t* req;     // [N] request of each query, or null (query n -> request n)
  const int32_t* idx;     // [N, K] selected cache rows
  const int32_t* n_idx;   // [N] entries that count, or null (all K)
  float* o;               // [nsplit, N, 64, 512]
  float* lse;             // [nsplit, N, 64]
  int64_t q_n, q_h;
  int64_t c_b, c_t;       // cache strides (elements)
  int64_t i_n;            // idx row stride (entries)
  int64_t o_s, o_n, o_h;
  int64_t l_s, l_n, l_h;
  int32_t N, B, K, Lmax, nsplit;
  int32_t reuse;          // several queries share a request's rows: cached loads
  int32_t fp8;
  float scale_log2;
};

struct TopkLocalArgs {
  const float* scores;    // [N, L] (row stride s_n)
  const int32_t* n_valid; // [N] or null (all L)
  float* out_score;       // [N, k]
  int32_t* out_id;        // [N, k] global ids
  int32_t* out_row;       // [N, k] local rows
  int32_t* out_count;     // [N]
  int64_t s_n, id_base, id_stride;
  int32_t N, L, k;
};

struct TopkMergeArgs {
  const float* cand_score;  // [P, N, k_in]
  const int32_t* cand_id;   // [P, N, k_in]
  const int32_t* cand_row;  // [P, N, k_in]
  const int32_t* cand_count;  // [P, N] or null (all k_in)
  int32_t* out_id;          // [N, k]
  int32_t* owner_row;       // [P, N, k]
  int32_t* owner_count;     // [P, N]
  int32_t P, N, k_in, k;
};

struct PrefillGqaArgs {
  const uint16_t* q;    // [n_local, Hq, 128] bf16
  const uint16_t* k;    // [T_kv, Hkv, 128]
  const uint16_t* v;    // [T_kv, Hkv, 128]
  void* out;            // [n_local, Hq, 128] bf16 or f32
  float* lse;           // [n_local, Hq]
  int64_t q_n, q_h, k_t, k_h, v_t, v_h, o_n, o_h, l_n, l_h;
  int32_t Hkv, G, out_bf16;
  float scale_log2;
};

struct PrefillMlaArgs {
  const uint16_t* q;    // [n_local, 64, 576] bf16
  const uint16_t* lat;  // [T_kv, 1, 576] latent (value = first 512 dims)
  void* out;            // [n_local, 64, 512] bf16 or f32
  float* lse;           // [n_local, 64]
  int64_t q_n, q_h, k_t, o_n, o_h, l_n, l_h;
  int32_t out_bf16;
  float scale_log2;
};

struct CacheWriteArgs {
  const char* src;      // [n, row] bytes
  const int64_t* slot;  // [n]
  const int32_t* req;   // [n]
  char* dst;            // [B, Lmax, row] bytes
  int64_t n, src_row, dst_b, dst_row, row_bytes;  // byte strides and row size
  int32_t C, rank, n_repl, B;
  int64_t Lmax;
  int32_t vec16;        // 16-byte lanes (row size and strides multiples of 16)
};

// ---- library-owned scratch of the entry points that allocate nothing ----
// Bytes of the per-device scratch array (noalloc.hip): the split states of
// one decode launch, e.g. 4 splits of 64 requests x 64 heads x 512 dims
// (33.6 MB) fit; 2 splits of 200 requests (52 MB) do not.
constexpr size_t kNoAllocScratchBytes = (size_t)48 << 20;

// Paged decode: page ids of one split a workgroup keeps in LDS. The host
// picks enough splits that no split touches more pages.
constexpr int kPageCap = 1024;
// Device address of the current device's scratch array (looked up once per
// device); returns hipSuccess or the lookup's error.
int noalloc_scratch(void** ptr);

// ---- launchers (return hipSuccess or the launch error) ----
int launch_merge(const MergeArgs& a, void* stream);
int launch_decode_gqa(const DecodeGqaArgs& a, void* stream);
// Query-head blocks (workgroups per kv head and split) of a GQA group of G heads.
int gqa_head_blocks(int G);
int launch_decode_mla(const DecodeMlaArgs& a, void* stream);
int launch_prefill_gqa(const PrefillGqaArgs& a, const cpa_segment* seg, int n_seg, void* stream);
int launch_prefill_mla(const PrefillMlaArgs& a, const cpa_segment* seg, int n_seg, void* stream);
int launch_cache_write_rr(const CacheWriteArgs& a, void* stream);
int launch_sparse_mla(const SparseMlaArgs& a, void* stream);
int launch_topk_local(const TopkLocalArgs& a, void* stream);
int launch_topk_merge(const TopkMergeArgs& a, void* stream);

}  // namespace cpa
