// Host-side checks of libcpattn built with AddressSanitizer and
// UndefinedBehaviorSanitizer: the planners on valid, edge and invalid
// inputs, and the argument validation of every device call (descriptors
// point at addresses that are never dereferenced; the kernel launchers are
// counting stubs). Any memory error or undefined behaviour aborts the run;
// a wrong status or a launch behind a rejected call fails it. Prints
// "host checks passed" on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <random>
#include <set>
#include <vector>

#include "cpattn.h"

namespace cpa {
extern int g_launches;
}

static int g_fail = 0;

#define CHECK(cond)                                                                       \
  do {                                                                                    \
    if (!(cond)) {                                                                        \
      std::fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
                   cpa_last_error());                                                     \
      ++g_fail;                                                                           \
    }                                                                                     \
  } while (0)

// A status and whether the call reached a kernel launcher.
#define EXPECT_CALL(call, status, launched)                                                      \
  do {                                                                                           \
    const int before = cpa::g_launches;                                                          \
    const cpa_status st_ = (call);                                                               \
    if (st_ != (status) || (cpa::g_launches > before) != (launched)) {                           \
      std::fprintf(stderr, "%s:%d: %s -> status %d (want %d), launched %d (want %d): %s\n",     \
                   __FILE__, __LINE__, #call, (int)st_, (int)(status), cpa::g_launches > before, \
                   (int)(launched), cpa_last_error());                                           \
      ++g_fail;                                                                                  \
    }                                                                                            \
  } while (0)

// Device addresses are never dereferenced on the host: any aligned value works.
static void* dev(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t)1 << 20 | off); }

static cpa_tensor tensor(int dtype, std::initializer_list<int64_t> shape, uintptr_t off = 0) {
  cpa_tensor t{};
  t.data = dev(off);
  t.dtype = dtype;
  t.ndim = (int32_t)shape.size();
  int i = 0;
  for (int64_t s : shape) t.shape[i++] = s;
  int64_t st = 1;
  for (int d = t.ndim - 1; d >= 0; --d) {
    t.stride[d] = st;
    st *= t.shape[d];
  }
  return t;
}

// ---------------------------------------------------------------- planners

static void check_prefill_planners() {
  std::mt19937 rng(7);
  for (int trial = 0; trial < 300; ++trial) {
    const int C = 1 + (int)(rng() % 9);
    const int n_req = (int)(rng() % 7);
    std::vector<int32_t> len(n_req), pre(n_req);
    int64_t total = 0;
    for (int i = 0; i < n_req; ++i) {
      len[i] = (int32_t)(rng() % 60);
      pre[i] = (int32_t)(rng() % 3 == 0 ? rng() % 50 : 0);
      total += len[i];
    }
    for (int kind = 0; kind < 2; ++kind) {
      std::set<int64_t> seen;
      int64_t owned = 0;
      for (int r = 0; r < C; ++r) {
        cpa_plan p{};
        auto plan = [&](cpa_plan* out) {
          return kind ? cp_plan_interleave(C, r, n_req, len.data(), pre.data(), out)
                      : cp_plan_zigzag(C, r, n_req, len.data(), pre.data(), out);
        };
        const cpa_status s0 = plan(&p);
        CHECK(s0 == CPA_OK || s0 == CPA_E_CAPACITY);
        std::vector<int64_t> tok(p.n_local + 1, -7);
        std::vector<int32_t> pos(p.n_local + 1, -7), req(p.n_local + 1, -7);
        std::vector<cpa_segment> seg(p.n_seg + 1);
        p.tok_index = tok.data();
        p.pos_id = pos.data();
        p.req_id = req.data();
        p.seg = seg.data();
        p.cap_local = p.n_local;
        p.cap_seg = p.n_seg;
        CHECK(plan(&p) == CPA_OK);
        CHECK(tok[p.n_local] == -7 && pos[p.n_local] == -7);  // nothing written past the count
        for (int64_t i = 0; i < p.n_local; ++i) {
          CHECK(tok[i] >= 0 && tok[i] < total);
          CHECK(seen.insert(tok[i]).second);
        }
        owned += p.n_local;
        if (p.n_local > 0) {  // a capacity one short writes only the sizes
          std::vector<int64_t> t2(p.n_local, -9);
          cpa_plan q = p;
          q.tok_index = t2.data();
          q.cap_local = p.n_local - 1;
          CHECK(plan(&q) == CPA_E_CAPACITY && q.n_local == p.n_local && t2[0] == -9);
        }
      }
      CHECK(owned == total);
    }
  }
  cpa_plan p{};
  const int32_t one[1] = {4}, neg[1] = {-1}, big[1] = {2147483647 - 10}, pre[1] = {100};
  CHECK(cp_plan_zigzag(0, 0, 1, one, nullptr, &p) == CPA_E_INVAL);
  CHECK(cp_plan_zigzag(4, 4, 1, one, nullptr, &p) == CPA_E_INVAL);
  CHECK(cp_plan_interleave(4, -1, 1, one, nullptr, &p) == CPA_E_INVAL);
  CHECK(cp_plan_interleave(4, 0, 1, neg, nullptr, &p) == CPA_E_INVAL);
  CHECK(cp_plan_zigzag(2, 0, 1, big, pre, &p) == CPA_E_INVAL);
  CHECK(cp_plan_zigzag(2, 0, 1, nullptr, nullptr, &p) == CPA_E_INVAL);
  CHECK(cp_plan_zigzag(2, 0, 1, one, nullptr, nullptr) == CPA_E_INVAL);
  CHECK(cp_plan_interleave(2, 0, 0, nullptr, nullptr, &p) == CPA_OK && p.n_local == 0);
}

static void check_decode_planners() {
  for (int64_t L = 0; L <= 70; ++L)
    for (int C = 1; C <= 9; ++C) {
      std::vector<int64_t> b(C + 1, -3), e(C + 1, -3);
      CHECK(cp_decode_shards(L, C, b.data(), e.data()) == CPA_OK);
      int64_t at = 0;
      for (int c = 0; c < C; ++c) {
        CHECK(b[c] == at && e[c] >= b[c]);
        at = e[c];
      }
      CHECK(at == L && b[C] == -3);
    }
  int64_t b4[4], e4[4];
  CHECK(cp_decode_shards(-1, 4, b4, e4) == CPA_E_INVAL);
  CHECK(cp_decode_shards(10, 0, b4, e4) == CPA_E_INVAL);
  CHECK(cp_decode_shards(10, 4, nullptr, e4) == CPA_E_INVAL);

  int32_t rank;
  int64_t row;
  for (int64_t slot = 0; slot < 200; slot += 7) {
    CHECK(cp_round_robin_slot(slot, 8, &rank, &row) == CPA_OK && rank == slot % 8 && row == slot / 8);
  }
  CHECK(cp_round_robin_slot(-1, 8, &rank, &row) == CPA_E_INVAL);
  CHECK(cp_round_robin_slot(5, 0, &rank, &row) == CPA_E_INVAL);
  CHECK(cp_round_robin_slot(5, 8, nullptr, &row) == CPA_E_INVAL);

  const int64_t ctx[4] = {0, 1, 17, 1000};
  for (int C = 1; C <= 8; ++C)
    for (int n_repl = 0; n_repl <= 3; ++n_repl) {
      int64_t own_total = 0;
      for (int r = 0; r < C; ++r) {
        int32_t kb[5] = {-5, -5, -5, -5, -5}, ke[5] = {-5, -5, -5, -5, -5};
        int64_t rows = -1;
        CHECK(cp_plan_round_robin(C, r, 4, ctx, n_repl, 0, kb, ke, &rows) == CPA_OK);
        CHECK(kb[4] == -5 && ke[4] == -5);
        for (int i = 0; i < 4; ++i) {
          CHECK(kb[i] == (r == 0 ? 0 : n_repl) && ke[i] >= n_repl && ke[i] <= rows);
          own_total += ke[i] - n_repl;
        }
      }
      CHECK(own_total == 0 + 1 + 17 + 1000);
      for (int layout = 0; layout < 2; ++layout)
        for (int Q = 1; Q <= 4; ++Q) {
          const int64_t ctx_q[3] = {4, 9, 300};
          int32_t kb[3], ke[12];
          int64_t rows;
          const int nr = layout ? n_repl : 0;
          CHECK(cp_plan_multi_query(layout, C, C - 1, 3, ctx_q, Q, nr, 0, kb, ke, &rows) == CPA_OK);
        }
    }
  int32_t kb[4], ke[16];
  CHECK(cp_plan_round_robin(0, 0, 4, ctx, 0, 0, kb, ke, nullptr) == CPA_E_INVAL);
  CHECK(cp_plan_round_robin(4, 4, 4, ctx, 0, 0, kb, ke, nullptr) == CPA_E_INVAL);
  CHECK(cp_plan_round_robin(4, 0, 4, ctx, 1, 9, kb, ke, nullptr) == CPA_E_INVAL);
  CHECK(cp_plan_round_robin(4, 0, 4, nullptr, 0, 0, kb, ke, nullptr) == CPA_E_INVAL);
  const int64_t short_ctx[2] = {1, 8};
  CHECK(cp_plan_multi_query(0, 4, 0, 2, short_ctx, 2, 0, 0, kb, ke, nullptr) == CPA_E_INVAL);  // length < Q
  CHECK(cp_plan_multi_query(0, 4, 0, 2, ctx + 2, 0, 0, 0, kb, ke, nullptr) == CPA_E_INVAL);    // Q < 1
  CHECK(cp_plan_multi_query(7, 4, 0, 2, ctx + 2, 1, 0, 0, kb, ke, nullptr) == CPA_E_INVAL);    // layout
  CHECK(cp_plan_multi_query(0, 4, 0, 2, ctx + 2, 1, 2, 0, kb, ke, nullptr) == CPA_E_INVAL);    // repl on contiguous
}

// ------------------------------------------------------------ device calls

static void check_merge() {
  cpa_tensor o = tensor(CPA_F32, {3, 5, 8, 64}), l = tensor(CPA_F32, {3, 5, 8}), out = tensor(CPA_F32, {5, 8, 64});
  cpa_tensor lo = tensor(CPA_F32, {5, 8});
  EXPECT_CALL(attn_merge_states(3, &o, &l, &out, &lo, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_merge_states(3, &o, &l, &out, nullptr, nullptr), CPA_OK, true);
  cpa_tensor outb = tensor(CPA_BF16, {5, 8, 64});
  EXPECT_CALL(attn_merge_states(3, &o, &l, &outb, &lo, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_merge_states(3, nullptr, &l, &out, nullptr, nullptr), CPA_E_INVAL, false);
  cpa_tensor lbad = tensor(CPA_F32, {3, 5, 9});
  EXPECT_CALL(attn_merge_states(3, &o, &lbad, &out, nullptr, nullptr), CPA_E_INVAL, false);
  cpa_tensor omis = o;
  omis.data = dev(4);  // not 16-byte aligned
  EXPECT_CALL(attn_merge_states(3, &omis, &l, &out, nullptr, nullptr), CPA_E_INVAL, false);
  cpa_tensor ostr = o;
  ostr.stride[3] = 2;  // last dimension not contiguous
  EXPECT_CALL(attn_merge_states(3, &ostr, &l, &out, nullptr, nullptr), CPA_E_INVAL, false);
  EXPECT_CALL(attn_merge_states(4, &o, &l, &out, nullptr, nullptr), CPA_E_INVAL, false);  // n_states != shape
  cpa_tensor oi = o;
  oi.dtype = CPA_BF16;  // partial states are f32 only
  EXPECT_CALL(attn_merge_states(3, &oi, &l, &out, nullptr, nullptr), CPA_E_UNSUPPORTED, false);
}

static void check_prefill() {
  const int n_local = 100, T = 300;
  cpa_tensor q = tensor(CPA_BF16, {n_local, 32, 128}), k = tensor(CPA_BF16, {T, 8, 128}),
             v = tensor(CPA_BF16, {T, 8, 128}), out = tensor(CPA_BF16, {n_local, 32, 128}),
             lse = tensor(CPA_F32, {n_local, 32});
  cpa_segment seg[2] = {{0, 0, 60, 0, 1, 0, 0}, {1, 60, 40, 5, 1, 0, 100}};
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, seg, 2, 0.1f, &out, &lse, nullptr), CPA_OK, true);
  std::vector<cpa_segment> many;
  for (int i = 0; i < 100; ++i) many.push_back({i, i, 1, i, 1, 0, 0});  // more than one launch's worth
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, many.data(), (int32_t)many.size(), 0.1f, &out, &lse, nullptr),
              CPA_OK, true);
  cpa_segment past_q[1] = {{0, 90, 20, 0, 1, 0, 0}};  // rows 90..109 > n_local
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, past_q, 1, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  cpa_segment past_kv[1] = {{0, 0, 10, 295, 1, 0, 0}};  // reads keys up to 304 > T
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, past_kv, 1, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  cpa_segment overlap[2] = {{0, 0, 50, 0, 1, 0, 0}, {1, 49, 10, 0, 1, 0, 100}};
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, overlap, 2, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  cpa_segment negs[1] = {{0, 0, 10, -1, 1, 0, 0}};
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, negs, 1, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  cpa_segment huge[1] = {{0, 0, 2, 2147483000, 2000000, 0, 0}};  // position overflows int32
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, huge, 1, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  EXPECT_CALL(attn_prefill_shard(&q, &k, &v, nullptr, 1, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  cpa_tensor q64 = tensor(CPA_BF16, {n_local, 32, 64});
  EXPECT_CALL(attn_prefill_shard(&q64, &k, &v, seg, 2, 0.1f, &out, &lse, nullptr), CPA_E_INVAL, false);
  // MLA: latent keys, no values
  cpa_tensor qm = tensor(CPA_BF16, {n_local, 64, 576}), lat = tensor(CPA_BF16, {T, 1, 576}),
             om = tensor(CPA_F32, {n_local, 64, 512}), lm = tensor(CPA_F32, {n_local, 64});
  EXPECT_CALL(attn_prefill_shard(&qm, &lat, nullptr, seg, 2, 0.05f, &om, &lm, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_prefill_shard(&qm, &lat, nullptr, seg, 2, -1.f, &om, &lm, nullptr), CPA_E_INVAL, false);
}

// Decode over a paged cache: pools of whole pages, a block table per request.
static void check_decode_paged(int B, int L, const int32_t* kb, const int32_t* ke, void* ws, size_t big) {
  const int ps = 64, nb = (L + ps - 1) / ps, n_pages = 2 * B * nb;
  const int32_t* table = static_cast<const int32_t*>(dev(128));
  cpa_tensor qm = tensor(CPA_BF16, {B, 64, 576}), pool = tensor(CPA_BF16, {(int64_t)n_pages * ps, 1, 576}),
             om = tensor(CPA_F32, {B, 64, 512}), lm = tensor(CPA_F32, {B, 64});
  const size_t need = attn_decode_paged_workspace_size(B, 64, 512, L, ps);
  CHECK(need > 0 && attn_decode_paged_workspace_size(B, 64, 512, L, 48) == 0);
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, table, nb, nb, ps, kb, ke, L, 0.05f, &om, &lm, ws,
                                      need, nullptr),
              CPA_OK, true);
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, table, nb, nb, ps, kb, ke, L, 0.05f, &om, &lm, ws,
                                      4096, nullptr),
              CPA_E_CAPACITY, false);
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, table, nb, nb, 48, kb, ke, L, 0.05f, &om, &lm, ws,
                                      big, nullptr),
              CPA_E_INVAL, false);  // page size not a power of two
  cpa_tensor ragged = tensor(CPA_BF16, {(int64_t)n_pages * ps + 5, 1, 576});
  EXPECT_CALL(attn_decode_shard_paged(&qm, &ragged, nullptr, nullptr, table, nb, nb, ps, kb, ke, L, 0.05f, &om, &lm,
                                      ws, big, nullptr),
              CPA_E_INVAL, false);  // pool rows not whole pages
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, nullptr, nb, nb, ps, kb, ke, L, 0.05f, &om, &lm,
                                      ws, big, nullptr),
              CPA_E_INVAL, false);
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, table, nb - 1, nb, ps, kb, ke, L, 0.05f, &om, &lm,
                                      ws, big, nullptr),
              CPA_E_INVAL, false);  // table row stride < n_blocks
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, table, (int64_t)1 << 26, (int64_t)1 << 26, ps, kb,
                                      ke, L, 0.05f, &om, &lm, ws, big, nullptr),
              CPA_E_INVAL, false);  // n_blocks x page size past 2^31
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool, nullptr, nullptr, table, nb, nb, ps, kb, ke, (int64_t)nb * ps + 1,
                                      0.05f, &om, &lm, ws, big, nullptr),
              CPA_OK, true);  // a bound past the table is allowed: positions clamp to it
  // 16-token pages: 1022 pages per split cover 16352 tokens, so a
  // 1.1M-token shard needs more splits than the MLA merge takes
  const int nb16 = 70000;
  cpa_tensor pool16 = tensor(CPA_BF16, {(int64_t)nb16 * 16, 1, 576});
  EXPECT_CALL(attn_decode_shard_paged(&qm, &pool16, nullptr, nullptr, table, nb16, nb16, 16, kb, ke,
                                      (int64_t)nb16 * 16, 0.05f, &om, &lm, ws, big, nullptr),
              CPA_E_UNSUPPORTED, false);
  // FP8 GQA pools with the per-row scale of the pool
  cpa_tensor q = tensor(CPA_BF16, {B, 32, 128}), kf = tensor(CPA_FP8_E4M3, {(int64_t)n_pages * ps, 8, 128}),
             vf = tensor(CPA_FP8_E4M3, {(int64_t)n_pages * ps, 8, 128}), o = tensor(CPA_F32, {B, 32, 128}),
             l = tensor(CPA_F32, {B, 32}), sc = tensor(CPA_F32, {(int64_t)n_pages * ps}),
             sshort = tensor(CPA_F32, {(int64_t)n_pages * ps - 1}), vshort = tensor(CPA_FP8_E4M3, {(int64_t)ps, 8, 128});
  EXPECT_CALL(attn_decode_shard_paged(&q, &kf, &vf, &sc, table, nb + 3, nb, ps, kb, ke, L, 0.1f, &o, &l, ws, big,
                                      nullptr),
              CPA_OK, true);
  EXPECT_CALL(attn_decode_shard_paged(&q, &kf, &vf, &sshort, table, nb, nb, ps, kb, ke, L, 0.1f, &o, &l, ws, big,
                                      nullptr),
              CPA_E_INVAL, false);
  EXPECT_CALL(attn_decode_shard_paged(&q, &kf, &vf, nullptr, table, nb, nb, ps, kb, ke, L, 0.1f, &o, &l, ws, big,
                                      nullptr),
              CPA_E_INVAL, false);  // FP8 without its scales
  EXPECT_CALL(attn_decode_shard_paged(&q, &kf, &vshort, &sc, table, nb, nb, ps, kb, ke, L, 0.1f, &o, &l, ws, big,
                                      nullptr),
              CPA_E_INVAL, false);  // value pool of another size
}

static void check_decode() {
  const int B = 6, L = 5000;
  const size_t big = (size_t)1 << 34;  // workspace bytes (never touched)
  // GQA bf16, d = 128
  cpa_tensor q = tensor(CPA_BF16, {B, 32, 128}), kc = tensor(CPA_BF16, {B, L, 8, 128}),
             vc = tensor(CPA_BF16, {B, L, 8, 128}), o = tensor(CPA_F32, {B, 32, 128}),
             l = tensor(CPA_F32, {B, 32});
  const int32_t* kb = static_cast<const int32_t*>(dev());
  const int32_t* ke = static_cast<const int32_t*>(dev(64));
  void* ws = dev(4096);
  const size_t need = attn_decode_workspace_size(B, 32, 128, L);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, nullptr, kb, ke, L, 0.1f, &o, &l, ws, need, nullptr), CPA_OK, true);
  // attn_decode_workspace_size is an upper bound over kv-head counts; this
  // shape splits 6 ways (48 units), so a few KB of workspace are too short
  CHECK(need >= (size_t)6 * B * 32 * 128 * 4);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, nullptr, kb, ke, L, 0.1f, &o, &l, ws, 4096, nullptr), CPA_E_CAPACITY,
              false);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, nullptr, kb, ke, L, 0.1f, &o, &l, dev(8), need, nullptr), CPA_E_INVAL,
              false);  // workspace not 256-byte aligned
  // FP8 GQA needs its per-token scale; the scale is only for FP8
  cpa_tensor kf = tensor(CPA_FP8_E4M3, {B, L, 8, 128}), vf = tensor(CPA_FP8_E4M3, {B, L, 8, 128}),
             sc = tensor(CPA_F32, {B, L});
  EXPECT_CALL(attn_decode_shard(&q, &kf, &vf, &sc, kb, ke, L, 0.1f, &o, &l, ws, big, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_decode_shard(&q, &kf, &vf, nullptr, kb, ke, L, 0.1f, &o, &l, ws, big, nullptr), CPA_E_INVAL,
              false);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, &sc, kb, ke, L, 0.1f, &o, &l, ws, big, nullptr), CPA_E_INVAL, false);
  cpa_tensor sbad = tensor(CPA_F32, {B, L - 1});
  EXPECT_CALL(attn_decode_shard(&q, &kf, &vf, &sbad, kb, ke, L, 0.1f, &o, &l, ws, big, nullptr), CPA_E_INVAL,
              false);
  // mixed dtypes, unsupported head dims, misaligned rows
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vf, nullptr, kb, ke, L, 0.1f, &o, &l, ws, big, nullptr), CPA_E_INVAL,
              false);
  cpa_tensor q96 = tensor(CPA_BF16, {B, 32, 96}), k96 = tensor(CPA_BF16, {B, L, 8, 96}),
             o96 = tensor(CPA_F32, {B, 32, 96});
  EXPECT_CALL(attn_decode_shard(&q96, &k96, &k96, nullptr, kb, ke, L, 0.1f, &o96, &l, ws, big, nullptr),
              CPA_E_UNSUPPORTED, false);
  cpa_tensor kmis = kc;
  kmis.stride[1] = 8 * 128 + 4;  // 2056-byte token stride
  kmis.stride[0] = kmis.stride[1] * L;
  EXPECT_CALL(attn_decode_shard(&q, &kmis, &vc, nullptr, kb, ke, L, 0.1f, &o, &l, ws, big, nullptr), CPA_E_INVAL,
              false);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, nullptr, nullptr, ke, L, 0.1f, &o, &l, ws, big, nullptr),
              CPA_E_INVAL, false);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, nullptr, kb, ke, -1, 0.1f, &o, &l, ws, big, nullptr), CPA_E_INVAL,
              false);
  EXPECT_CALL(attn_decode_shard(&q, &kc, &vc, nullptr, kb, ke, L, 0.f, &o, &l, ws, big, nullptr), CPA_E_INVAL,
              false);
  cpa_tensor q7 = tensor(CPA_BF16, {B, 30, 128}), o7 = tensor(CPA_F32, {B, 30, 128}), l7 = tensor(CPA_F32, {B, 30});
  EXPECT_CALL(attn_decode_shard(&q7, &kc, &vc, nullptr, kb, ke, L, 0.1f, &o7, &l7, ws, big, nullptr), CPA_E_INVAL,
              false);  // 30 query heads on 8 kv heads
  // a GQA group of 40 heads (three head blocks)
  cpa_tensor q40 = tensor(CPA_F32, {B, 40, 64}), k40 = tensor(CPA_F32, {B, L, 1, 64}),
             o40 = tensor(CPA_F32, {B, 40, 64}), l40 = tensor(CPA_F32, {B, 40});
  EXPECT_CALL(attn_decode_shard(&q40, &k40, &k40, nullptr, kb, ke, L, 0.1f, &o40, &l40, ws, big, nullptr), CPA_OK,
              true);
  // MLA
  cpa_tensor qm = tensor(CPA_BF16, {B, 64, 576}), lat = tensor(CPA_BF16, {B, L, 1, 576}),
             om = tensor(CPA_F32, {B, 64, 512}), lm = tensor(CPA_F32, {B, 64});
  EXPECT_CALL(attn_decode_shard(&qm, &lat, nullptr, nullptr, kb, ke, L, 0.05f, &om, &lm, ws, big, nullptr), CPA_OK,
              true);
  cpa_tensor qm32 = tensor(CPA_BF16, {B, 32, 576}), om32 = tensor(CPA_F32, {B, 32, 512});
  EXPECT_CALL(attn_decode_shard(&qm32, &lat, nullptr, nullptr, kb, ke, L, 0.05f, &om32, &l, ws, big, nullptr),
              CPA_E_UNSUPPORTED, false);
  cpa_tensor latf = tensor(CPA_FP8_E4M3, {B, L, 1, 576});
  EXPECT_CALL(attn_decode_shard(&qm, &latf, nullptr, &sc, kb, ke, L, 0.05f, &om, &lm, ws, big, nullptr), CPA_OK,
              true);
  // the allocation-free variant: small shapes run, large ones are refused
  EXPECT_CALL(attn_decode_shard_noalloc(&qm, &lat, nullptr, nullptr, kb, ke, L, 0.05f, &om, &lm, nullptr), CPA_OK,
              true);
  const int BB = 200, LL = 2048;  // 2 splits x 200 x 64 x 512 x 4 B = 52 MB of states
  cpa_tensor qbig = tensor(CPA_BF16, {BB, 64, 576}), latbig = tensor(CPA_BF16, {BB, LL, 1, 576}),
             obig = tensor(CPA_F32, {BB, 64, 512}), lbig = tensor(CPA_F32, {BB, 64});
  EXPECT_CALL(attn_decode_shard_noalloc(&qbig, &latbig, nullptr, nullptr, kb, ke, LL, 0.05f, &obig, &lbig, nullptr),
              CPA_E_CAPACITY, false);
  // multi-query rows
  cpa_tensor qq = tensor(CPA_BF16, {B, 3, 64, 576}), oq = tensor(CPA_F32, {B, 3, 64, 512}),
             lq = tensor(CPA_F32, {B, 3, 64});
  EXPECT_CALL(attn_decode_shard_mq(&qq, &lat, nullptr, nullptr, kb, ke, L, 0.05f, &oq, &lq, ws, big, nullptr), CPA_OK,
              true);
  cpa_tensor qq0 = tensor(CPA_BF16, {B, 65, 64, 576}), oq0 = tensor(CPA_F32, {B, 65, 64, 512}),
             lq0 = tensor(CPA_F32, {B, 65, 64});
  EXPECT_CALL(attn_decode_shard_mq(&qq0, &lat, nullptr, nullptr, kb, ke, L, 0.05f, &oq0, &lq0, ws, big, nullptr),
              CPA_E_INVAL, false);  // Q > 64
  check_decode_paged(B, L, kb, ke, ws, big);
}

static void check_sparse_topk_cachewrite() {
  const int N = 5, B = 5, L = 3000, K = 2048;
  cpa_tensor q = tensor(CPA_BF16, {N, 64, 576}), cache = tensor(CPA_BF16, {B, L, 1, 576}),
             o = tensor(CPA_F32, {N, 64, 512}), l = tensor(CPA_F32, {N, 64});
  const int32_t* idx = static_cast<const int32_t*>(dev());
  const size_t need = attn_sparse_mla_workspace_size(N, K);
  void* ws = dev(1 << 12);
  EXPECT_CALL(attn_sparse_mla(&q, &cache, nullptr, nullptr, idx, K, K, nullptr, 0.05f, &o, &l, ws, need, nullptr), CPA_OK,
              true);
  EXPECT_CALL(attn_sparse_mla(&q, &cache, nullptr, nullptr, idx, K - 1, K, nullptr, 0.05f, &o, &l, ws, need, nullptr),
              CPA_E_INVAL, false);  // stride < k
  EXPECT_CALL(attn_sparse_mla(&q, &cache, nullptr, nullptr, nullptr, K, K, nullptr, 0.05f, &o, &l, ws, need, nullptr),
              CPA_E_INVAL, false);

  cpa_tensor cache8 = tensor(CPA_FP8_E4M3, {B, L, 1, 576}), scale8 = tensor(CPA_F32, {B, L});
  EXPECT_CALL(attn_sparse_mla(&q, &cache8, &scale8, nullptr, idx, K, K, nullptr, 0.05f, &o, &l, ws, need, nullptr),
              CPA_OK, true);
  EXPECT_CALL(attn_sparse_mla(&q, &cache8, nullptr, nullptr, idx, K, K, nullptr, 0.05f, &o, &l, ws, need, nullptr),
              CPA_E_INVAL, false);  // FP8 without its scales
  EXPECT_CALL(attn_sparse_mla(&q, &cache, &scale8, nullptr, idx, K, K, nullptr, 0.05f, &o, &l, ws, need, nullptr),
              CPA_E_INVAL, false);  // scales with a bf16 cache

  float* sc = static_cast<float*>(dev());
  int32_t* i32 = static_cast<int32_t*>(dev(1 << 8));
  float* f32 = static_cast<float*>(dev(1 << 9));
  EXPECT_CALL(attn_topk_local(sc, 16384, 64, 16384, nullptr, 2048, 3, 8, f32, i32, i32, i32, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_topk_local(sc, 16384, 64, 16384, nullptr, 2048, 3, 1 << 20, f32, i32, i32, i32, nullptr),
              CPA_E_INVAL, false);  // global ids past 2^31
  EXPECT_CALL(attn_topk_local(sc, 16384, -1, 16384, nullptr, 2048, 0, 1, f32, i32, i32, i32, nullptr), CPA_E_INVAL,
              false);
  EXPECT_CALL(attn_topk_local(reinterpret_cast<float*>(dev(2)), 16384, 64, 16384, nullptr, 2048, 0, 1, f32, i32, i32,
                              i32, nullptr),
              CPA_E_INVAL, false);  // misaligned scores
  EXPECT_CALL(attn_topk_merge(8, 64, 2048, f32, i32, i32, nullptr, 2048, i32, i32, i32, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_topk_merge(65, 64, 2048, f32, i32, i32, nullptr, 2048, i32, i32, i32, nullptr), CPA_E_INVAL,
              false);  // P > 64

  cpa_tensor src = tensor(CPA_BF16, {100, 576}), dst = tensor(CPA_BF16, {4, 200, 576});
  const int64_t* slot = static_cast<const int64_t*>(dev());
  EXPECT_CALL(attn_cache_write_round_robin(8, 3, 2, &src, slot, i32, &dst, nullptr), CPA_OK, true);
  EXPECT_CALL(attn_cache_write_round_robin(8, 8, 2, &src, slot, i32, &dst, nullptr), CPA_E_INVAL, false);
  cpa_tensor dst8 = tensor(CPA_FP8_E4M3, {4, 200, 576});
  EXPECT_CALL(attn_cache_write_round_robin(8, 3, 2, &src, slot, i32, &dst8, nullptr), CPA_E_INVAL, false);
}

int main() {
  check_prefill_planners();
  check_decode_planners();
  check_merge();
  check_prefill();
  check_decode();
  check_sparse_topk_cachewrite();
  if (g_fail) {
    std::fprintf(stderr, "%d host checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed (%d launches reached)\n", cpa::g_launches);
  return 0;
}
