/*
 * cpattn.h -- context-parallel attention shards for MI355X (gfx950).
 *
 * One rank's share of long-context attention, as the source pages state the
 * problem:
 *   - "How GPUs Share a Long Context During LLM Inference" (vincentzed.com),
 *     cited as Long Context below, sections 1-3;
 *   - SGLang documentation "Prefill context parallelism" (strategy interface,
 *     zigzag and interleave strategies);
 *   - vLLM "Decode Context Parallelism" post (contiguous token chunks, MLA and
 *     GQA backends);
 *   - "DeepSeek-V4 Attention Inference Systems" notes, section 5 (exact
 *     partial-softmax combine).
 *
 * Conventions shared by every call:
 *   - Plain C ABI. No exception crosses it. Every call returns a cpa_status;
 *     on failure cpa_last_error() returns a message for the calling thread.
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream), allocate nothing and own nothing: the
 *     caller owns every buffer and keeps it alive until the stream is done.
 *   - Tensors are described by cpa_tensor with strides in elements; the last
 *     dimension must be contiguous (stride 1) and the data pointer 16-byte
 *     aligned. Arguments are validated on the host before any launch; a
 *     validation failure launches nothing.
 *   - LSE is the natural log of the sum of exponentiated scores (Long
 *     Context 3.3); an empty key set gives O = 0 and LSE = -inf.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cpa_status {
  CPA_OK = 0,
  CPA_E_INVAL = 1,        /* null pointer, bad shape, dtype, stride or alignment */
  CPA_E_UNSUPPORTED = 2,  /* head dims or dtype combination the library has no kernel for */
  CPA_E_CAPACITY = 3,     /* a caller array or workspace is too small; sizes written back */
  CPA_E_HIP = 4           /* the HIP runtime reported an error at launch */
} cpa_status;

typedef enum cpa_dtype {
  CPA_F32 = 0,
  CPA_BF16 = 1,
  CPA_FP8_E4M3 = 2  /* OCP E4M3FN bytes: bias 7, max 448, no infinity */
} cpa_dtype;

typedef struct cpa_tensor {
  void* data;         /* device pointer */
  int32_t dtype;      /* cpa_dtype */
  int32_t ndim;       /* 1..4 */
  int64_t shape[4];
  int64_t stride[4];  /* elements; stride[ndim-1] must be 1 */
} cpa_tensor;

/*
 * A segment is a run of a rank's local query rows of one request whose
 * positions step by a constant: local row q_row0 + i (0 <= i < q_len) has
 * position pos0 + i * pos_stride inside its request (cached prefix
 * included) and reads keys 0 .. that position, diagonal included (Long
 * Context 1.1). In the packed full K/V, request `req` starts at row kv_row0
 * and holds its prefix and new tokens in original order, so the row reads
 * K/V rows [kv_row0, kv_row0 + pos0 + i * pos_stride + 1).
 *   zigzag:     stride 1, one segment per non-empty block; the block's
 *               reads stop at position pos0 + q_len (Long Context 2.3).
 *   interleave: stride C, one segment per request (each query's own causal
 *               extent, SGLang docs "Interleave strategy").
 */
typedef struct cpa_segment {
  int32_t req;
  int32_t q_row0;
  int32_t q_len;
  int32_t pos0;
  int32_t pos_stride;
  int32_t reserved;   /* set to 0 */
  int64_t kv_row0;
} cpa_segment;

/*
 * Output of the planners (host memory, owned by the caller). The planner
 * fills at most cap_local rows and cap_seg segments. It always writes
 * n_local, n_seg and n_padded; if either capacity is too small it writes
 * nothing else and returns CPA_E_CAPACITY, so a first call with zero
 * capacities (and NULL arrays) returns the sizes to allocate.
 */
typedef struct cpa_plan {
  int64_t* tok_index;   /* [cap_local] index into the batch's new tokens, flattened request by request */
  int32_t* pos_id;      /* [cap_local] original position inside the request, prefix included */
  int32_t* req_id;      /* [cap_local] request of the row */
  int64_t cap_local;
  cpa_segment* seg;     /* [cap_seg] */
  int64_t cap_seg;
  int64_t n_local;      /* rows owned by this rank */
  int64_t n_seg;        /* segments written */
  int64_t n_padded;     /* rows of the largest rank's share (padded buffer size) */
} cpa_plan;

/* Message of the last failed call on this thread ("" if none). */
const char* cpa_last_error(void);

/* ABI version of this library (major * 100 + minor). */
int32_t cpa_abi_version(void);

/*
 * Zigzag prefill plan. SGLang docs "Zigzag strategy"; Long Context 2.3.
 * Each request's new tokens are cut into 2C contiguous blocks, the first
 * (L mod 2C) blocks holding one extra token; rank `rank` takes blocks rank
 * and 2C-1-rank, request by request, early block first. A cached prefix is
 * not split and is read by both blocks. Host-only, synchronous, pure.
 *   C >= 1, 0 <= rank < C, n_req >= 0, new_len[n_req] >= 0,
 *   prefix_len[n_req] >= 0 or NULL for no prefix.
 * Errors: CPA_E_INVAL for bad arguments or a batch larger than 2^31-1 new
 * or packed tokens; CPA_E_CAPACITY as described at cpa_plan.
 */
cpa_status cp_plan_zigzag(int32_t C, int32_t rank, int32_t n_req, const int32_t* new_len,
                          const int32_t* prefix_len, cpa_plan* out);

/*
 * Interleave prefill plan. SGLang docs "Interleave strategy"; Long Context
 * 2.4. Rank `rank` owns flattened new-token indices rank, rank+C, ... of the
 * whole batch (no reset at request boundaries), in ascending order; position
 * ids keep their original values. One segment of stride C per request that
 * owns a row. n_padded = ceil(T / C). Arguments and errors as for
 * cp_plan_zigzag.
 */
cpa_status cp_plan_interleave(int32_t C, int32_t rank, int32_t n_req, const int32_t* new_len,
                              const int32_t* prefix_len, cpa_plan* out);

/*
 * Contiguous decode shards of an L-token context over C ranks (vLLM DCP
 * post, section 4: GPU c holds a contiguous chunk of token positions); the
 * early shards take the remainder. Writes begin[C], end[C] (host arrays).
 */
cpa_status cp_decode_shards(int64_t L, int32_t C, int64_t* begin, int64_t* end);

/*
 * Causal attention of a rank's local queries against their true causal
 * history (Long Context 2.1 and 2.3: partial Q against the full, gathered
 * K/V; the cached prefix included).
 *   q    [n_local, Hq, Dqk]  bf16   local queries in plan order
 *   k    [T_kv, Hkv, Dqk]    bf16   packed keys (see cpa_segment)
 *   v    [T_kv, Hkv, Dv]     bf16   packed values, or NULL for MLA, where the
 *                                   value of a token is the first Dv dims of
 *                                   its latent vector k (Long Context 1.3;
 *                                   vLLM GLM-5.3 post footnote 1: QK over 576,
 *                                   PV over 512)
 *   seg  [n_seg]             HOST   segments (e.g. from a planner); each is
 *                                   bounds-checked against q, k and out
 *   out  [n_local, Hq, Dv]   bf16 or f32 (written for rows covered by a segment)
 *   lse  [n_local, Hq]       f32
 * Query head h uses kv head h / (Hq / Hkv). Supported head dims: GQA
 * Dqk = Dv = 128; MLA (v NULL, Hkv = 1) Dqk = 576, Dv = 512.
 * Segments must not overlap in q rows. Rows not covered by a segment are not
 * written.
 */
cpa_status attn_prefill_shard(const cpa_tensor* q, const cpa_tensor* k, const cpa_tensor* v,
                              const cpa_segment* seg, int32_t n_seg, float softmax_scale,
                              const cpa_tensor* out, const cpa_tensor* lse, void* stream);

/*
 * Bytes of workspace attn_decode_shard needs for this shape (0 is possible).
 * max_shard_len is the longest kv_end - kv_begin of the batch.
 */
size_t attn_decode_workspace_size(int64_t batch, int32_t n_heads_q, int32_t head_dim_v,
                                  int64_t max_shard_len);

/*
 * Split-KV decode on one shard (Long Context 3.2-3.4; vLLM DCP post 4.1):
 * for request b and query head h, attention of the single query q[b, h]
 * over cache rows [kv_begin[b], kv_end[b]) of request b, emitting the
 * partial output and its LSE for the merge.
 *   q        [B, Hq, Dqk]          bf16 or f32
 *   kcache   [B, Lmax, Hkv, Dqk]   f32, bf16 or FP8 E4M3
 *   vcache   [B, Lmax, Hkv, Dv]    same dtype as kcache, or NULL for MLA
 *                                  (value = first Dv dims of the latent)
 *   kv_scale [B, Lmax] f32         per-token scale, required for FP8 and
 *                                  otherwise NULL: every entry of token t
 *                                  (its key and, for GQA, its value) is
 *                                  e4m3 * scale[b, t]
 *   kv_begin, kv_end [B] int32     DEVICE arrays; clamped to [0, Lmax] and
 *                                  an empty range gives O = 0, LSE = -inf
 *   max_shard_len                  upper bound of kv_end - kv_begin, used to
 *                                  size the internal split (any length is
 *                                  still processed in full)
 *   o_part   [B, Hq, Dv] f32, lse_part [B, Hq] f32
 *   workspace / ws_bytes           device scratch of at least
 *                                  attn_decode_workspace_size(...) bytes
 * Supported: MLA (Hkv = 1, Dqk = 576, Dv = 512, q bf16, cache bf16 or FP8)
 * and GQA (Dqk = Dv in {64, 128, 256}, any Hq / Hkv group, cache f32, bf16
 * or FP8; K/V data pointers and strides in bytes multiples of 16). Other
 * shapes return CPA_E_UNSUPPORTED, misaligned K/V CPA_E_INVAL.
 */
cpa_status attn_decode_shard(const cpa_tensor* q, const cpa_tensor* kcache, const cpa_tensor* vcache,
                             const cpa_tensor* kv_scale, const int32_t* kv_begin,
                             const int32_t* kv_end, int64_t max_shard_len, float softmax_scale,
                             const cpa_tensor* o_part, const cpa_tensor* lse_part, void* workspace,
                             size_t ws_bytes, void* stream);

/*
 * attn_decode_shard for callers that cannot allocate device memory (code
 * under HIP stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results as
 * attn_decode_shard, without workspace arguments. The internal split's
 * partial states live in a scratch array the library holds on every device
 * it runs on (48 MiB per device, kept until the process ends); the call
 * allocates nothing. A shape whose split states need more than that returns
 * CPA_E_CAPACITY (attn_decode_shard with a workspace takes any size). The
 * array is shared by every call on a GPU: calls that overlap on one GPU
 * (e.g. on two streams) race and must be serialised by the caller.
 */
cpa_status attn_decode_shard_noalloc(const cpa_tensor* q, const cpa_tensor* kcache, const cpa_tensor* vcache,
                                     const cpa_tensor* kv_scale, const int32_t* kv_begin, const int32_t* kv_end,
                                     int64_t max_shard_len, float softmax_scale, const cpa_tensor* o_part,
                                     const cpa_tensor* lse_part, void* stream);

/*
 * Split-KV decode over a paged cache ("DeepSeek-V4 Attention Inference
 * Systems", 1: logical cache blocks of a fixed size mapped to physical pages
 * of shared pools; 9.1: decode reads the paged cache directly). The same
 * computation and results as attn_decode_shard, where token t of request b
 * (t a logical position in [kv_begin[b], kv_end[b])) is the pool row
 *   block_table[b * bt_stride + t / page_size] * page_size + t % page_size.
 *   q           [B, Hq, Dqk]                   bf16 or f32, as attn_decode_shard
 *   kpool       [n_pages * page_size, Hkv, Dqk] f32, bf16 or FP8 E4M3
 *   vpool       [n_pages * page_size, Hkv, Dv]  same dtype, or NULL for MLA
 *   kv_scale    [n_pages * page_size] f32       per-row scale, FP8 only
 *   block_table DEVICE int32, B rows of n_blocks entries bt_stride apart;
 *               an entry outside [0, n_pages) is read as page 0
 *   page_size   a power of two in [1, 2^20]; logical positions are clamped
 *               to [0, n_blocks * page_size]
 *   max_shard_len  must bound kv_end - kv_begin here (it sizes the splits,
 *               and a split keeps the ids of the pages it touches on chip;
 *               a longer range is read in bounds but its result is not
 *               defined)
 *   workspace   at least attn_decode_paged_workspace_size(...) bytes
 * Supported shapes and dtypes as attn_decode_shard (one query row per
 * request). Pages can be shared between requests (e.g. a common prefix).
 * CPA_E_UNSUPPORTED when the pages of max_shard_len tokens do not fit the
 * split limit (1024 pages per split; 64 splits MLA, 256 GQA).
 */
size_t attn_decode_paged_workspace_size(int64_t batch, int32_t n_heads_q, int32_t head_dim_v,
                                        int64_t max_shard_len, int32_t page_size);
cpa_status attn_decode_shard_paged(const cpa_tensor* q, const cpa_tensor* kpool, const cpa_tensor* vpool,
                                   const cpa_tensor* kv_scale, const int32_t* block_table, int64_t bt_stride,
                                   int64_t n_blocks, int32_t page_size, const int32_t* kv_begin,
                                   const int32_t* kv_end, int64_t max_shard_len, float softmax_scale,
                                   const cpa_tensor* o_part, const cpa_tensor* lse_part, void* workspace,
                                   size_t ws_bytes, void* stream);

/*
 * Multi-query split-KV decode (speculative / MTP decode under decode CP:
 * Long Context 9 lists it; DeepSeek-V4 notes, 11, sweeps the query/spec
 * width 1, 2, 4, 8). Request b has Q query rows; row k attends cache rows
 * [kv_begin[b], kv_end[b*Q + k]) of its request -- causal among the draft
 * rows when the ends come from cp_plan_multi_query -- exactly as
 * attn_decode_shard attends its single query.
 *   q        [B, Q, Hq, Dqk]       bf16 or f32 (strides free, 16-byte aligned)
 *   kcache, vcache, kv_scale, max_shard_len, softmax_scale: as for
 *                                  attn_decode_shard
 *   kv_begin [B] int32, kv_end [B*Q] int32   DEVICE arrays, clamped to
 *                                  [0, Lmax]; an empty range gives O = 0,
 *                                  LSE = -inf
 *   o_part   [B, Q, Hq, Dv] f32, lse_part [B, Q, Hq] f32; for B > 1 and
 *            Q > 1 stride[0] must equal Q * stride[1] (the (b, k) pair is
 *            addressed as one row b*Q + k)
 *   workspace / ws_bytes           at least attn_decode_workspace_size(B*Q,
 *                                  Hq, Dv, max_shard_len) bytes
 * 1 <= Q <= 64. For MLA the Q rows of one (request, split) run as Q
 * workgroups on one XCD and read each cache tile through its shared L2, so
 * HBM traffic stays that of one query row. Q = 1 gives the same results as
 * attn_decode_shard. Errors as for attn_decode_shard, plus CPA_E_INVAL for a
 * bad Q or mismatched output shapes or strides.
 */
cpa_status attn_decode_shard_mq(const cpa_tensor* q, const cpa_tensor* kcache, const cpa_tensor* vcache,
                                const cpa_tensor* kv_scale, const int32_t* kv_begin,
                                const int32_t* kv_end, int64_t max_shard_len, float softmax_scale,
                                const cpa_tensor* o_part, const cpa_tensor* lse_part, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * Exact LSE merge of S partial states (Long Context 3.3; DeepSeek-V4 notes,
 * section 5): lse = log sum_c exp(lse_c), O = sum_c exp(lse_c - lse) O_c.
 *   o_parts   [S, N, H, Dv] f32
 *   lse_parts [S, N, H]     f32
 *   out       [N, H, Dv]    f32 or bf16
 *   lse_out   [N, H]        f32, or data NULL to skip
 * A state with LSE = -inf carries no mass; if all are -inf the row gets
 * O = 0 and LSE = -inf (no NaN). S = 1 copies.
 */
cpa_status attn_merge_states(int32_t n_states, const cpa_tensor* o_parts,
                             const cpa_tensor* lse_parts, const cpa_tensor* out,
                             const cpa_tensor* lse_out, void* stream);

/*
 * Round-robin decode storage (Long Context 3.1 and Figure 7: slot p of a
 * request lives on rank p mod C as local row p / C, and both the cache
 * write and the attention read translate a slot that way; DeepSeek-V4
 * notes, section 5: owner(j) = j mod P).
 *
 * cp_round_robin_slot: host, pure. *rank = slot % C, *row = slot / C.
 * CPA_E_INVAL if slot < 0, C < 1 or an output is NULL.
 */
cpa_status cp_round_robin_slot(int64_t slot, int32_t C, int32_t* rank, int64_t* row);

/*
 * cp_plan_round_robin: host, pure. The decode range of rank `rank` in its
 * round-robin local cache, per request. Local cache layout: rows
 * [0, n_repl) hold n_repl entries replicated on every rank (a local
 * window, attention sinks), rows n_repl, n_repl + 1, ... the rank's own
 * slots rank, rank + C, ... of the request in ascending order. Replicated
 * entries must add their probability mass once (DeepSeek-V4 notes, 5.3):
 * only repl_rank includes them.
 *   ctx_len  [n_req] int64  slots stored for each request (>= 0)
 *   kv_begin [n_req] int32  out: 0 on repl_rank, n_repl elsewhere
 *   kv_end   [n_req] int32  out: n_repl + number of own slots
 *   max_local_rows          out (may be NULL): rows a local cache needs
 * The ranges feed attn_decode_shard on that rank's local cache; the C
 * partial states merged with attn_merge_states equal attention over the
 * n_repl replicated entries and all ctx_len slots. CPA_E_INVAL on bad C,
 * rank, repl_rank, a negative count, NULL arrays or a range past 2^31-1.
 */
cpa_status cp_plan_round_robin(int32_t C, int32_t rank, int32_t n_req, const int64_t* ctx_len,
                               int32_t n_repl, int32_t repl_rank, int32_t* kv_begin, int32_t* kv_end,
                               int64_t* max_local_rows);

/*
 * Sparse (top-k index list) MLA attention (Long Context 2.4: a query of a
 * sparse-attention model brings its own list of selected tokens; vLLM
 * GLM-5.3 part 2, footnote 1: each query reads its 2,048 selected latent
 * rows for all 64 heads, QK over 576 dims and PV over 512). Query n attends
 * the cache rows idx[n, 0 .. n_idx[n]) of request req[n], emitting O and
 * its LSE, so lists split by owner across ranks combine exactly with
 * attn_merge_states (DeepSeek-V4 notes, 5.2).
 *   q       [N, 64, 576] bf16
 *   cache   [B, Lmax, 1, 576] bf16, or FP8 E4M3 (one latent per token;
 *           FP8 row strides multiples of 16 bytes)
 *   kv_scale [B, Lmax] f32 per-token scale, required for FP8 and otherwise
 *           NULL: entry = e4m3 * scale (as for attn_decode_shard)
 *   req     [N] int32 DEVICE, or NULL: query n uses request n (then N <= B)
 *   idx     DEVICE int32, row n at idx + n * idx_stride, k entries per row
 *           (idx_stride >= k); an entry outside [0, Lmax) is no selection
 *           (padding: skipped); an entry listed twice counts twice
 *   n_idx   [N] int32 DEVICE, or NULL: only the first n_idx[n] entries of
 *           row n count (clamped to [0, k))
 *   out     [N, 64, 512] f32, lse [N, 64] f32; a query with no selection,
 *           or whose request is outside [0, B), gets O = 0, LSE = -inf
 *   workspace / ws_bytes: at least attn_sparse_mla_workspace_size(N, k)
 *           bytes, 256-byte aligned (split states of long lists)
 * Rows are addressed with 32-bit offsets: one request's cache may span at
 * most 4 GiB. CPA_E_INVAL / CPA_E_UNSUPPORTED on shapes, dtypes, strides or
 * sizes outside these; CPA_E_CAPACITY for a short workspace.
 */
size_t attn_sparse_mla_workspace_size(int64_t n_queries, int32_t k);
cpa_status attn_sparse_mla(const cpa_tensor* q, const cpa_tensor* cache, const cpa_tensor* kv_scale,
                           const int32_t* req, const int32_t* idx, int64_t idx_stride, int32_t k,
                           const int32_t* n_idx, float softmax_scale, const cpa_tensor* out, const cpa_tensor* lse,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Exact distributed top-k for sparse attention with a split index
 * (DeepSeek-V4 notes, 5.2: each rank keeps a local top-k list of (score,
 * global id), the at most P x k candidates merge into the exact global top
 * k, the selected ids go to their owners; Long Context 4.1, Figure 11).
 * Order: higher score first; equal scores (-0 = +0) by lower global id; NaN
 * below every number. Using the same rule on every rank makes the union of
 * the local lists contain the global top k, so the merge is exact. All
 * arrays are DEVICE arrays, 4-byte aligned; both calls are asynchronous.
 *
 * attn_topk_local: for each of n_rows query rows, the best min(k, n) of the
 * rank's local entries 0 .. n-1 (n = n_valid[row], clamped to [0, L], or L
 * when n_valid is NULL), entry j having score scores[row * score_stride + j]
 * and global id id_base + j * id_stride (round robin: rank, C; contiguous
 * chunk: its first position, 1). Writes, in ascending local row order,
 * out_score / out_id / out_row [n_rows, k] (padded with -inf / -1 / -1) and
 * out_count [n_rows]. CPA_E_INVAL if a global id falls outside [0, 2^31), on
 * negative sizes, NULL arrays or misalignment.
 */
cpa_status attn_topk_local(const float* scores, int64_t score_stride, int32_t n_rows, int32_t L,
                           const int32_t* n_valid, int32_t k, int64_t id_base, int64_t id_stride, float* out_score,
                           int32_t* out_id, int32_t* out_row, int32_t* out_count, void* stream);

/*
 * attn_topk_merge: for each query row, the exact global top k of the P
 * ranks' lists (1 <= P <= 64). Candidates: cand_score / cand_id / cand_row [P, n_rows,
 * k_in] (rank p's list of that row: its first cand_count[p * n_rows + row]
 * entries, clamped to [0, k_in], or all k_in when cand_count is NULL).
 * Global ids must be distinct within a row. Writes out_id [n_rows, k]: the
 * selected global ids, grouped by rank (rank 0's first) and in each rank's
 * list order, padded with -1; owner_row [P, n_rows, k]: for each rank the
 * local rows (cand_row) of its selected entries, padded with -1 -- the
 * index lists its attn_sparse_mla call takes -- and owner_count [P, n_rows].
 */
cpa_status attn_topk_merge(int32_t P, int32_t n_rows, int32_t k_in, const float* cand_score, const int32_t* cand_id,
                           const int32_t* cand_row, const int32_t* cand_count, int32_t k, int32_t* out_id,
                           int32_t* owner_row, int32_t* owner_count, void* stream);

/* Cache layouts of decode CP. */
#define CPA_LAYOUT_CONTIGUOUS 0  /* rank c holds the c-th contiguous chunk (cp_decode_shards) */
#define CPA_LAYOUT_ROUND_ROBIN 1 /* slot p on rank p % C, row p / C (cp_plan_round_robin) */

/*
 * cp_plan_multi_query: host, pure. Per-row decode ranges of rank `rank` for
 * multi-query (speculative / MTP) decode. A request stores ctx_len[b] slots
 * whose last Q are its query rows (draft tokens already written to the
 * cache); row k sits at slot p = ctx_len[b] - Q + k and, attention being
 * causal (Long Context 1.1), sees slots [0, p].
 *   layout   CPA_LAYOUT_CONTIGUOUS: the rank's local cache holds slots
 *            [begin, end) of cp_decode_shards(ctx_len[b], C) from row 0;
 *            kv_begin = 0, kv_end[b*Q + k] = rows of that chunk below p + 1.
 *            n_repl and repl_rank must be 0.
 *            CPA_LAYOUT_ROUND_ROBIN: local cache as for cp_plan_round_robin;
 *            kv_begin as there, kv_end[b*Q + k] = n_repl + own slots <= p
 *            (replicated rows are seen by every query row).
 *   ctx_len  [n_req] int64 (>= Q)
 *   kv_begin [n_req] int32, kv_end [n_req * Q] int32 (out, host)
 *   max_local_rows  out (may be NULL): rows a local cache needs
 * Merging the C ranks' attn_decode_shard_mq states with attn_merge_states
 * gives each query row causal attention over its request. CPA_E_INVAL on a
 * bad layout, C, rank, Q < 1, repl_rank, a length below Q, NULL arrays or a
 * range past 2^31-1.
 */
cpa_status cp_plan_multi_query(int32_t layout, int32_t C, int32_t rank, int32_t n_req, const int64_t* ctx_len,
                               int32_t Q, int32_t n_repl, int32_t repl_rank, int32_t* kv_begin, int32_t* kv_end,
                               int64_t* max_local_rows);

/*
 * attn_cache_write_round_robin: device, asynchronous. Writes entries into
 * rank `rank`'s round-robin local cache (Long Context 3.1: the cache write
 * translates a slot into a GPU and a row). Entry i (row i of src) of
 * request req[i] at slot slot[i] is copied to dst[req[i], n_repl + slot[i] / C]
 * when slot[i] % C == rank; entries owned by other ranks, with a negative
 * slot or request, a request >= B, or a row past Lmax_local are skipped.
 *   src  [n, W]                any dtype (bytes are copied)
 *   slot [n] int64, req [n] int32: device arrays, 8- and 4-byte aligned
 *   dst  [B, Lmax_local, W]    same dtype as src
 * Row size and row strides must be multiples of 4 bytes (16 bytes gives
 * 16-byte copies). The FP8 cache's per-token scales are written by a second
 * call with W = 1 f32 rows. Entries with equal (req, slot) race.
 */
cpa_status attn_cache_write_round_robin(int32_t C, int32_t rank, int32_t n_repl, const cpa_tensor* src,
                                        const int64_t* slot, const int32_t* req, const cpa_tensor* dst,
                                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
