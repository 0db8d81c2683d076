// Host-side shard planners: zigzag and interleave prefill plans, contiguous
// decode shards.
//
// Zigzag -- SGLang "Prefill context parallelism" docs, "Zigzag strategy";
// "How GPUs Share a Long Context During LLM Inference", 2.3: 2C contiguous
// blocks per request, rank r keeps blocks r and 2C-1-r, early blocks take the
// remainder (one extra token each), the split restarts per request, a cached
// prefix is read by both blocks but not split.
// Interleave -- same docs, "Interleave strategy"; the same article, 2.4:
// rank r keeps flattened new-token indices r, r+C, ... across the batch.
// Contiguous decode shards -- vLLM "Decode Context Parallelism" post,
// section 4.
//
// Everything here is plain host C++ (no HIP), pure and synchronous.
#include <climits>
#include <cstdint>
#include <vector>

#include "internal.h"

namespace {

struct Req {
  int64_t new_len, prefix, cu_new, cu_kv;
};

cpa_status read_batch(int32_t C, int32_t rank, int32_t n_req, const int32_t* new_len,
                      const int32_t* prefix_len, cpa_plan* out, std::vector<Req>& reqs) {
  if (out == nullptr) return cpa::fail(CPA_E_INVAL, "plan: out is NULL");
  if (C < 1) return cpa::fail(CPA_E_INVAL, "plan: C = %d must be >= 1", C);
  if (rank < 0 || rank >= C) return cpa::fail(CPA_E_INVAL, "plan: rank %d not in [0, %d)", rank, C);
  if (n_req < 0) return cpa::fail(CPA_E_INVAL, "plan: n_req = %d < 0", n_req);
  if (n_req > 0 && new_len == nullptr) return cpa::fail(CPA_E_INVAL, "plan: new_len is NULL");
  reqs.resize(n_req);
  int64_t cu_new = 0, cu_kv = 0;
  for (int32_t j = 0; j < n_req; ++j) {
    int64_t L = new_len[j];
    int64_t P = prefix_len ? prefix_len[j] : 0;
    if (L < 0 || P < 0) return cpa::fail(CPA_E_INVAL, "plan: request %d has a negative length", j);
    if (L + P > INT32_MAX)
      return cpa::fail(CPA_E_INVAL, "plan: request %d has %lld tokens (positions must fit int32)", j,
                       (long long)(L + P));
    reqs[j] = Req{L, P, cu_new, cu_kv};
    cu_new += L;
    cu_kv += L + P;
  }
  if (cu_new > INT32_MAX) return cpa::fail(CPA_E_INVAL, "plan: batch has more than 2^31-1 new tokens");
  return CPA_OK;
}

// Length and start of block b (0 <= b < 2C) of an L-token request.
inline void zz_block(int64_t L, int32_t C, int32_t b, int64_t* start, int64_t* len) {
  const int64_t nb = 2 * (int64_t)C;
  const int64_t base = L / nb, rem = L % nb;
  *len = base + (b < rem ? 1 : 0);
  *start = (int64_t)b * base + (b < rem ? b : rem);
}

inline int64_t zz_rank_rows(int64_t L, int32_t C, int32_t r) {
  int64_t s, a, b;
  zz_block(L, C, r, &s, &a);
  zz_block(L, C, 2 * C - 1 - r, &s, &b);
  return a + b;
}

}  // namespace

extern "C" cpa_status cp_plan_zigzag(int32_t C, int32_t rank, int32_t n_req, const int32_t* new_len,
                                     const int32_t* prefix_len, cpa_plan* out) {
  cpa::clear_error();
  std::vector<Req> reqs;
  cpa_status st = read_batch(C, rank, n_req, new_len, prefix_len, out, reqs);
  if (st != CPA_OK) return st;
  // sizes: rows and segments of this rank, largest share over all ranks
  int64_t n_local = 0, n_seg = 0;
  std::vector<int64_t> per_rank(C, 0);
  for (const Req& q : reqs) {
    for (int32_t r = 0; r < C; ++r) per_rank[r] += zz_rank_rows(q.new_len, C, r);
    for (int32_t b : {rank, 2 * C - 1 - rank}) {
      int64_t s, n;
      zz_block(q.new_len, C, b, &s, &n);
      n_local += n;
      n_seg += n > 0;
    }
  }
  int64_t n_padded = 0;
  for (int64_t x : per_rank) n_padded = x > n_padded ? x : n_padded;
  out->n_local = n_local;
  out->n_seg = n_seg;
  out->n_padded = n_padded;
  if (out->cap_local < n_local || out->cap_seg < n_seg)
    return cpa::fail(CPA_E_CAPACITY, "plan: need %lld rows and %lld segments, have %lld and %lld",
                     (long long)n_local, (long long)n_seg, (long long)out->cap_local,
                     (long long)out->cap_seg);
  if ((n_local > 0 && (!out->tok_index || !out->pos_id || !out->req_id)) || (n_seg > 0 && !out->seg))
    return cpa::fail(CPA_E_INVAL, "plan: output arrays are NULL");
  int64_t row = 0, sg = 0;
  for (int32_t j = 0; j < n_req; ++j) {
    const Req& q = reqs[j];
    for (int32_t b : {rank, 2 * C - 1 - rank}) {
      int64_t start, n;
      zz_block(q.new_len, C, b, &start, &n);
      if (n == 0) continue;
      cpa_segment& g = out->seg[sg++];
      g.req = j;
      g.q_row0 = (int32_t)row;
      g.q_len = (int32_t)n;
      g.pos0 = (int32_t)(q.prefix + start);
      g.pos_stride = 1;
      g.reserved = 0;
      g.kv_row0 = q.cu_kv;
      for (int64_t i = 0; i < n; ++i, ++row) {
        out->tok_index[row] = q.cu_new + start + i;
        out->pos_id[row] = (int32_t)(q.prefix + start + i);
        out->req_id[row] = j;
      }
    }
  }
  return CPA_OK;
}

extern "C" cpa_status cp_plan_interleave(int32_t C, int32_t rank, int32_t n_req,
                                         const int32_t* new_len, const int32_t* prefix_len,
                                         cpa_plan* out) {
  cpa::clear_error();
  std::vector<Req> reqs;
  cpa_status st = read_batch(C, rank, n_req, new_len, prefix_len, out, reqs);
  if (st != CPA_OK) return st;
  // first owned flattened index of each request and how many it owns
  auto first_owned = [&](const Req& q) { return q.cu_new + (((rank - q.cu_new) % C) + C) % C; };
  auto owned = [&](const Req& q) {
    const int64_t g0 = first_owned(q), end = q.cu_new + q.new_len;
    return g0 < end ? (end - 1 - g0) / C + 1 : (int64_t)0;
  };
  int64_t n_local = 0, n_seg = 0, T = 0;
  for (const Req& q : reqs) {
    const int64_t n = owned(q);
    n_local += n;
    n_seg += n > 0;
    T += q.new_len;
  }
  out->n_local = n_local;
  out->n_seg = n_seg;
  out->n_padded = (T + C - 1) / C;
  if (out->cap_local < n_local || out->cap_seg < n_seg)
    return cpa::fail(CPA_E_CAPACITY, "plan: need %lld rows and %lld segments, have %lld and %lld",
                     (long long)n_local, (long long)n_seg, (long long)out->cap_local,
                     (long long)out->cap_seg);
  if ((n_local > 0 && (!out->tok_index || !out->pos_id || !out->req_id)) || (n_seg > 0 && !out->seg))
    return cpa::fail(CPA_E_INVAL, "plan: output arrays are NULL");
  int64_t row = 0, sg = 0;
  for (int32_t j = 0; j < n_req; ++j) {
    const Req& q = reqs[j];
    const int64_t n = owned(q);
    if (n == 0) continue;
    const int64_t g0 = first_owned(q);
    cpa_segment& g = out->seg[sg++];
    g.req = j;
    g.q_row0 = (int32_t)row;
    g.q_len = (int32_t)n;
    g.pos0 = (int32_t)(q.prefix + (g0 - q.cu_new));
    g.pos_stride = C;
    g.reserved = 0;
    g.kv_row0 = q.cu_kv;
    for (int64_t i = 0; i < n; ++i, ++row) {
      const int64_t gi = g0 + i * C;
      out->tok_index[row] = gi;
      out->pos_id[row] = (int32_t)(q.prefix + (gi - q.cu_new));
      out->req_id[row] = j;
    }
  }
  return CPA_OK;
}

extern "C" cpa_status cp_decode_shards(int64_t L, int32_t C, int64_t* begin, int64_t* end) {
  cpa::clear_error();
  if (C < 1 || L < 0) return cpa::fail(CPA_E_INVAL, "decode shards: bad L = %lld or C = %d", (long long)L, C);
  if (!begin || !end) return cpa::fail(CPA_E_INVAL, "decode shards: NULL output");
  const int64_t base = L / C, rem = L % C;
  int64_t s = 0;
  for (int32_t c = 0; c < C; ++c) {
    const int64_t n = base + (c < rem ? 1 : 0);
    begin[c] = s;
    end[c] = s + n;
    s += n;
  }
  return CPA_OK;
}

// Round-robin decode storage -- "How GPUs Share a Long Context During LLM
// Inference", 3.1: slot p of a request lives on rank p mod C as row p / C;
// "DeepSeek-V4 Attention Inference Systems" notes, 5.3: entries replicated
// on every rank add their probability mass on one designated rank only.
// Local cache layout: rows [0, n_repl) replicated entries, then the rank's
// own slots in ascending order.
extern "C" cpa_status cp_round_robin_slot(int64_t slot, int32_t C, int32_t* rank, int64_t* row) {
  cpa::clear_error();
  if (C < 1 || slot < 0) return cpa::fail(CPA_E_INVAL, "round robin: bad slot %lld or C = %d", (long long)slot, C);
  if (!rank || !row) return cpa::fail(CPA_E_INVAL, "round robin: NULL output");
  *rank = (int32_t)(slot % C);
  *row = slot / C;
  return CPA_OK;
}

extern "C" cpa_status cp_plan_round_robin(int32_t C, int32_t rank, int32_t n_req, const int64_t* ctx_len,
                                          int32_t n_repl, int32_t repl_rank, int32_t* kv_begin, int32_t* kv_end,
                                          int64_t* max_local_rows) {
  cpa::clear_error();
  if (C < 1) return cpa::fail(CPA_E_INVAL, "round robin plan: C = %d must be >= 1", C);
  if (rank < 0 || rank >= C) return cpa::fail(CPA_E_INVAL, "round robin plan: rank %d not in [0, %d)", rank, C);
  if (repl_rank < 0 || repl_rank >= C)
    return cpa::fail(CPA_E_INVAL, "round robin plan: repl_rank %d not in [0, %d)", repl_rank, C);
  if (n_req < 0 || n_repl < 0) return cpa::fail(CPA_E_INVAL, "round robin plan: negative n_req or n_repl");
  if (n_req > 0 && (!ctx_len || !kv_begin || !kv_end))
    return cpa::fail(CPA_E_INVAL, "round robin plan: NULL array");
  int64_t mx = n_repl;
  for (int32_t b = 0; b < n_req; ++b) {
    const int64_t L = ctx_len[b];
    if (L < 0) return cpa::fail(CPA_E_INVAL, "round robin plan: request %d has a negative length", b);
    const int64_t own = L > rank ? (L - rank + C - 1) / C : 0;
    const int64_t end = n_repl + own;
    if (end > INT32_MAX) return cpa::fail(CPA_E_INVAL, "round robin plan: request %d needs more than 2^31-1 rows", b);
    kv_begin[b] = rank == repl_rank ? 0 : n_repl;
    kv_end[b] = (int32_t)end;
    mx = end > mx ? end : mx;
  }
  if (max_local_rows) *max_local_rows = mx;
  return CPA_OK;
}

// Multi-query decode ranges: the Q query rows of a request are its last Q
// slots (draft tokens already stored in the cache), and row k at slot
// p = L - Q + k reads the slots [0, p] (causal attention, "How GPUs Share a
// Long Context During LLM Inference", 1.1). On a rank this is the part of
// [0, p] the rank stores: for contiguous shards ("Decode Context
// Parallelism" post, 4) the prefix of the rank's chunk up to p, for
// round-robin storage (Long Context 3.1) its own slots <= p after the
// replicated rows, which every row sees.
extern "C" cpa_status cp_plan_multi_query(int32_t layout, int32_t C, int32_t rank, int32_t n_req,
                                          const int64_t* ctx_len, int32_t Q, int32_t n_repl, int32_t repl_rank,
                                          int32_t* kv_begin, int32_t* kv_end, int64_t* max_local_rows) {
  cpa::clear_error();
  if (layout != CPA_LAYOUT_CONTIGUOUS && layout != CPA_LAYOUT_ROUND_ROBIN)
    return cpa::fail(CPA_E_INVAL, "multi-query plan: unknown layout %d", layout);
  if (C < 1) return cpa::fail(CPA_E_INVAL, "multi-query plan: C = %d must be >= 1", C);
  if (rank < 0 || rank >= C) return cpa::fail(CPA_E_INVAL, "multi-query plan: rank %d not in [0, %d)", rank, C);
  if (Q < 1) return cpa::fail(CPA_E_INVAL, "multi-query plan: Q = %d must be >= 1", Q);
  if (n_req < 0 || n_repl < 0) return cpa::fail(CPA_E_INVAL, "multi-query plan: negative n_req or n_repl");
  if (layout == CPA_LAYOUT_CONTIGUOUS && (n_repl != 0 || repl_rank != 0))
    return cpa::fail(CPA_E_INVAL, "multi-query plan: contiguous shards take no replicated rows");
  if (repl_rank < 0 || repl_rank >= C)
    return cpa::fail(CPA_E_INVAL, "multi-query plan: repl_rank %d not in [0, %d)", repl_rank, C);
  if (n_req > 0 && (!ctx_len || !kv_begin || !kv_end)) return cpa::fail(CPA_E_INVAL, "multi-query plan: NULL array");
  int64_t mx = layout == CPA_LAYOUT_ROUND_ROBIN ? n_repl : 0;
  for (int32_t b = 0; b < n_req; ++b) {
    const int64_t L = ctx_len[b];
    if (L < Q) return cpa::fail(CPA_E_INVAL, "multi-query plan: request %d stores %lld < Q slots", b, (long long)L);
    int64_t rows;  // local rows this request needs
    if (layout == CPA_LAYOUT_CONTIGUOUS) {
      const int64_t base = L / C, rem = L % C;
      const int64_t s = rank * base + (rank < rem ? rank : rem);
      const int64_t e = s + base + (rank < rem ? 1 : 0);
      rows = e - s;
      kv_begin[b] = 0;
      for (int32_t k = 0; k < Q; ++k) {
        const int64_t lim = L - Q + k + 1;  // slots [0, lim) are visible
        kv_end[(int64_t)b * Q + k] = (int32_t)((lim < s ? s : (lim > e ? e : lim)) - s);
      }
    } else {
      rows = n_repl + (L > rank ? (L - rank + C - 1) / C : 0);
      kv_begin[b] = rank == repl_rank ? 0 : n_repl;
      for (int32_t k = 0; k < Q; ++k) {
        const int64_t lim = L - Q + k + 1;
        kv_end[(int64_t)b * Q + k] = (int32_t)(n_repl + (lim > rank ? (lim - rank + C - 1) / C : 0));
      }
    }
    if (rows > INT32_MAX) return cpa::fail(CPA_E_INVAL, "multi-query plan: request %d needs more than 2^31-1 rows", b);
    mx = rows > mx ? rows : mx;
  }
  if (max_local_rows) *max_local_rows = mx;
  return CPA_OK;
}
