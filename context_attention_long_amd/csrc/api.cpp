// C ABI of libcpattn: argument validation on the host, then kernel dispatch.
// Every check here runs before any launch, so a rejected call touches no
// device memory. The kernels assume what these checks establish (shapes,
// strides, segment bounds).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "internal.h"

namespace cpa {

namespace {
thread_local std::string g_err;
}

void clear_error() { g_err.clear(); }

cpa_status fail(cpa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace cpa

namespace {

using cpa::fail;

int elem_size(int32_t dt) { return dt == CPA_F32 ? 4 : dt == CPA_BF16 ? 2 : dt == CPA_FP8_E4M3 ? 1 : 0; }

const char* dt_name(int32_t dt) {
  return dt == CPA_F32 ? "f32" : dt == CPA_BF16 ? "bf16" : dt == CPA_FP8_E4M3 ? "fp8_e4m3" : "?";
}

// Checks a tensor: non-null, dtype in `dtypes` (bitmask of 1 << dtype), rank,
// non-negative shape, unit last stride; base and row strides aligned to
// `align` bytes (16 for tensors moved with 16-byte vector accesses; 0 means
// the element size, for tensors accessed element by element).
cpa_status check_tensor(const cpa_tensor* t, const char* name, unsigned dtypes, int ndim, int align = 16) {
  if (t == nullptr) return fail(CPA_E_INVAL, "%s: descriptor is NULL", name);
  if (t->ndim != ndim) return fail(CPA_E_INVAL, "%s: ndim %d, expected %d", name, t->ndim, ndim);
  if (t->dtype < 0 || t->dtype > 2 || !(dtypes & (1u << t->dtype)))
    return fail(CPA_E_UNSUPPORTED, "%s: dtype %s not supported here", name, dt_name(t->dtype));
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(CPA_E_INVAL, "%s: negative shape", name);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) numel *= t->shape[i];
  if (numel == 0) return CPA_OK;
  if (t->data == nullptr) return fail(CPA_E_INVAL, "%s: data is NULL", name);
  if (t->stride[ndim - 1] != 1) return fail(CPA_E_INVAL, "%s: last dimension must be contiguous", name);
  const int es = elem_size(t->dtype);
  const int al = align > 0 ? align : es;
  if (((uintptr_t)t->data) % al) return fail(CPA_E_INVAL, "%s: data must be %d-byte aligned", name, al);
  for (int i = 0; i < ndim - 1; ++i) {
    if (t->stride[i] < 0) return fail(CPA_E_INVAL, "%s: negative stride", name);
    if (t->shape[i] > 1 && (t->stride[i] * es) % al)
      return fail(CPA_E_INVAL, "%s: stride of dim %d must be a multiple of %d bytes", name, i, al);
  }
  return CPA_OK;
}

#define CPA_TRY(x)                      \
  do {                                  \
    cpa_status st_ = (x);               \
    if (st_ != CPA_OK) return st_;      \
  } while (0)

cpa_status hip_status(int err, const char* what) {
  if (err != hipSuccess)
    return fail(CPA_E_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
  return CPA_OK;
}

int num_cus() {
  static int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 256;
    return cus;
  }();
  return n;
}

constexpr float kLog2e = 1.4426950408889634f;

// ---- decode split plan: how many workgroups share one request's shard ----
struct DecodePlan {
  bool mla;
  int nsplit;
  int head_blocks;  // GQA: workgroups per (row, kv head, split), one per 16 query heads
};

int mla_nsplit(int64_t B, int64_t max_len) {
  if (B <= 0) return 1;
  const int64_t slots = num_cus();                 // one 8-wavefront workgroup per CU
  int64_t ns = (slots + B - 1) / B;                // fill the machine once
  const int64_t by_len = (max_len + 255) / 256;    // at least 256 tokens per split
  if (ns > by_len) ns = by_len;
  if (ns < 1) ns = 1;
  if (ns > 64) ns = 64;
  return (int)ns;
}

// GQA: units = rows x kv heads x query-head blocks; one 4-wavefront
// workgroup per CU (with 8 requests x 8 kv heads x 16384 tokens, bf16
// streamed at 6.0 TB/s with one per CU against 5.4 with two, FP8 at 4.9
// against 4.1), and at least 128 tokens per split.
int gqa_nsplit(int64_t units, int64_t max_len) {
  if (units <= 0) return 1;
  int64_t ns = ((int64_t)num_cus() + units - 1) / units;
  const int64_t by_len = (max_len + 127) / 128;
  if (ns > by_len) ns = by_len;
  if (ns < 1) ns = 1;
  if (ns > 256) ns = 256;
  return (int)ns;
}

size_t decode_ws_bytes(int64_t B, int64_t Hq, int64_t Dv, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t o = (size_t)nsplit * B * Hq * Dv * sizeof(float);
  const size_t o_al = (o + 255) / 256 * 256;
  return o_al + (size_t)nsplit * B * Hq * sizeof(float);
}

}  // namespace

extern "C" const char* cpa_last_error(void) { return cpa::g_err.c_str(); }

extern "C" int32_t cpa_abi_version(void) { return 102; }

// --------------------------------------------------------------------- merge

extern "C" cpa_status attn_merge_states(int32_t n_states, const cpa_tensor* o_parts,
                                        const cpa_tensor* lse_parts, const cpa_tensor* out,
                                        const cpa_tensor* lse_out, void* stream) {
  cpa::clear_error();
  if (n_states < 1) return fail(CPA_E_INVAL, "merge: n_states = %d < 1", n_states);
  CPA_TRY(check_tensor(o_parts, "merge o_parts", 1u << CPA_F32, 4));
  CPA_TRY(check_tensor(lse_parts, "merge lse_parts", 1u << CPA_F32, 3, 0));
  if (out == nullptr) return fail(CPA_E_INVAL, "merge out: descriptor is NULL");
  // f32 rows are stored 16 bytes at a time, bf16 rows 8 bytes at a time
  CPA_TRY(check_tensor(out, "merge out", (1u << CPA_F32) | (1u << CPA_BF16), 3, out->dtype == CPA_BF16 ? 8 : 16));
  const int64_t S = o_parts->shape[0], N = o_parts->shape[1], H = o_parts->shape[2],
                Dv = o_parts->shape[3];
  if (S != n_states) return fail(CPA_E_INVAL, "merge: o_parts has %lld states, n_states = %d", (long long)S, n_states);
  if (lse_parts->shape[0] != S || lse_parts->shape[1] != N || lse_parts->shape[2] != H)
    return fail(CPA_E_INVAL, "merge: lse_parts shape does not match o_parts [S, N, H]");
  if (out->shape[0] != N || out->shape[1] != H || out->shape[2] != Dv)
    return fail(CPA_E_INVAL, "merge: out shape must be [N, H, Dv]");
  if (Dv % 4) return fail(CPA_E_UNSUPPORTED, "merge: Dv = %lld must be a multiple of 4", (long long)Dv);
  if (N > INT32_MAX || H > INT32_MAX || Dv > INT32_MAX) return fail(CPA_E_INVAL, "merge: dims too large");
  bool has_lse_out = lse_out != nullptr && lse_out->data != nullptr;
  if (has_lse_out) {
    CPA_TRY(check_tensor(lse_out, "merge lse_out", 1u << CPA_F32, 2, 0));
    if (lse_out->shape[0] != N || lse_out->shape[1] != H)
      return fail(CPA_E_INVAL, "merge: lse_out must be f32 [N, H]");
  }
  // lse_parts need not be 16-byte strided: it is read element-wise
  cpa::MergeArgs a{};
  a.o = static_cast<const float*>(o_parts->data);
  a.lse = static_cast<const float*>(lse_parts->data);
  a.out = out->data;
  a.lse_out = has_lse_out ? static_cast<float*>(lse_out->data) : nullptr;
  a.o_s = o_parts->stride[0];
  a.o_n = o_parts->stride[1];
  a.o_h = o_parts->stride[2];
  a.l_s = lse_parts->stride[0];
  a.l_n = lse_parts->stride[1];
  a.l_h = lse_parts->stride[2];
  a.out_n = out->stride[0];
  a.out_h = out->stride[1];
  a.lo_n = has_lse_out ? lse_out->stride[0] : 0;
  a.lo_h = has_lse_out ? lse_out->stride[1] : 0;
  a.S = (int32_t)S;
  a.N = (int32_t)N;
  a.H = (int32_t)H;
  a.Dv = (int32_t)Dv;
  a.out_bf16 = out->dtype == CPA_BF16;
  if (N * H == 0) return CPA_OK;
  return hip_status(cpa::launch_merge(a, stream), "merge launch");
}

// -------------------------------------------------------------------- decode

// Paged cache (attn_decode_shard_paged): the block table, its row stride,
// log2 of the page size and the pool's page count.
struct Paging {
  const int32_t* table;
  int64_t stride;
  int32_t shift, n_pages;
};

// Splits of a paged decode: at least `ns`, and enough that a split of the
// longest range touches at most kPageCap pages (a split of n tokens touches
// at most (n - 1) / page + 2 pages).
int paged_nsplit(int ns, int64_t max_len, int shift) {
  const int64_t per = ((int64_t)(cpa::kPageCap - 2)) << shift;  // tokens per split that always fit
  const int64_t need = (max_len + per - 1) / per;
  return (int)std::max<int64_t>(ns, need);
}

namespace {

// rows = query rows of the launch (requests x query rows per request)
cpa_status decode_plan(int64_t rows, int64_t Hq, const cpa_tensor* kcache, const cpa_tensor* vcache,
                       int64_t max_len, DecodePlan* p) {
  const int64_t Hkv = kcache->shape[2];
  p->mla = vcache == nullptr;
  p->head_blocks = 1;
  if (p->mla) {
    p->nsplit = mla_nsplit(rows, max_len);
  } else {
    p->head_blocks = cpa::gqa_head_blocks((int)(Hq / Hkv));
    p->nsplit = gqa_nsplit(rows * Hkv * p->head_blocks, max_len);
  }
  return CPA_OK;
}

// Shared decode path. q is the [B, Hq, Dqk] view of query row 0 of every
// request; a request has Q query rows, q_q elements apart. o_part / lse_part
// are [B * Q, Hq, Dv] / [B * Q, Hq] (row b * Q + k) and kv_end has B * Q
// entries; kv_begin has B.
cpa_status decode_impl(const cpa_tensor* q, int64_t Q, int64_t q_q, const cpa_tensor* kcache,
                       const cpa_tensor* vcache, const cpa_tensor* kv_scale, const int32_t* kv_begin,
                       const int32_t* kv_end, int64_t max_shard_len, float softmax_scale, const cpa_tensor* o_part,
                       const cpa_tensor* lse_part, void* workspace, size_t ws_bytes, void* stream,
                       bool lib_scratch = false, const Paging* pg = nullptr) {
  CPA_TRY(check_tensor(q, "decode q", (1u << CPA_F32) | (1u << CPA_BF16), 3));
  CPA_TRY(check_tensor(kcache, "decode kcache", (1u << CPA_F32) | (1u << CPA_BF16) | (1u << CPA_FP8_E4M3), 4));
  CPA_TRY(check_tensor(o_part, "decode o_part", 1u << CPA_F32, 3));
  CPA_TRY(check_tensor(lse_part, "decode lse_part", 1u << CPA_F32, 2, 0));
  const int64_t B = q->shape[0], Hq = q->shape[1], Dqk = q->shape[2];
  const int64_t Lmax = kcache->shape[1], Hkv = kcache->shape[2];
  if (kcache->shape[0] != B || kcache->shape[3] != Dqk)
    return fail(CPA_E_INVAL, "decode: kcache must be [B, Lmax, Hkv, Dqk] matching q");
  if (Hkv < 1 || Hq % Hkv) return fail(CPA_E_INVAL, "decode: Hq = %lld not a multiple of Hkv = %lld", (long long)Hq, (long long)Hkv);
  if (Lmax > INT32_MAX || B * Q > INT32_MAX) return fail(CPA_E_INVAL, "decode: sizes too large");
  const int64_t R = B * Q;  // output rows
  if (max_shard_len < 0) return fail(CPA_E_INVAL, "decode: max_shard_len < 0");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(CPA_E_INVAL, "decode: softmax_scale must be finite and > 0");
  if (B > 0 && (kv_begin == nullptr || kv_end == nullptr)) return fail(CPA_E_INVAL, "decode: kv_begin/kv_end NULL");
  const bool fp8 = kcache->dtype == CPA_FP8_E4M3;
  int64_t Dv;
  if (vcache == nullptr) {
    // MLA: value = first 512 dims of the 576-dim latent
    if (Hkv != 1 || Dqk != 576) return fail(CPA_E_UNSUPPORTED, "decode: MLA needs Hkv = 1 and Dqk = 576");
    if (Hq != 64) return fail(CPA_E_UNSUPPORTED, "decode: MLA kernel is built for 64 query heads, got %lld", (long long)Hq);
    if (q->dtype != CPA_BF16) return fail(CPA_E_UNSUPPORTED, "decode: MLA needs a bf16 query");
    if (kcache->dtype == CPA_F32) return fail(CPA_E_UNSUPPORTED, "decode: MLA cache must be bf16 or fp8");
    // the kernel addresses a 32-token tile with 32-bit per-thread offsets
    if (kcache->stride[1] > (int64_t)1 << 26) return fail(CPA_E_INVAL, "decode: kcache token stride too large");
    Dv = 512;
  } else {
    CPA_TRY(check_tensor(vcache, "decode vcache", (1u << CPA_F32) | (1u << CPA_BF16) | (1u << CPA_FP8_E4M3), 4));
    if (vcache->dtype != kcache->dtype) return fail(CPA_E_INVAL, "decode: vcache dtype differs from kcache");
    if (vcache->shape[0] != B || vcache->shape[1] != Lmax || vcache->shape[2] != Hkv)
      return fail(CPA_E_INVAL, "decode: vcache must be [B, Lmax, Hkv, Dv]");
    Dv = vcache->shape[3];
    if (Dv != Dqk) return fail(CPA_E_UNSUPPORTED, "decode: GQA needs Dv == Dqk");
    if (Dqk != 64 && Dqk != 128 && Dqk != 256)
      return fail(CPA_E_UNSUPPORTED, "decode: GQA head dim must be 64, 128 or 256, got %lld", (long long)Dqk);
    // the kernel streams 16-byte pieces of K/V rows straight into LDS and
    // addresses a 16-token tile with 32-bit per-lane offsets
    const int64_t esz = fp8 ? 1 : (kcache->dtype == CPA_BF16 ? 2 : 4);
    for (const cpa_tensor* t : {kcache, vcache}) {
      if (((uintptr_t)t->data) % 16 || (t->stride[0] * esz) % 16 || (t->stride[1] * esz) % 16 ||
          (t->stride[2] * esz) % 16)
        return fail(CPA_E_INVAL, "decode: GQA K/V rows must start on 16-byte boundaries (pointer and strides)");
      if (t->stride[1] * esz > (int64_t)1 << 26) return fail(CPA_E_INVAL, "decode: K/V token stride too large");
    }
  }
  if (fp8) {
    if (kv_scale == nullptr || kv_scale->data == nullptr) return fail(CPA_E_INVAL, "decode: FP8 cache needs kv_scale");
    CPA_TRY(check_tensor(kv_scale, "decode kv_scale", 1u << CPA_F32, 2, 0));
    if (kv_scale->shape[0] != B || kv_scale->shape[1] != Lmax)
      return fail(CPA_E_INVAL, "decode: kv_scale must be f32 [B, Lmax]");
    // the kernel addresses a 32-token tile's scales with 32-bit offsets
    if (kv_scale->stride[1] > (int64_t)1 << 26) return fail(CPA_E_INVAL, "decode: kv_scale token stride too large");
  } else if (kv_scale != nullptr && kv_scale->data != nullptr) {
    return fail(CPA_E_INVAL, "decode: kv_scale is only for an FP8 cache");
  }
  if (o_part->shape[0] != R || o_part->shape[1] != Hq || o_part->shape[2] != Dv)
    return fail(CPA_E_INVAL, "decode: o_part must be [B, (Q,) Hq, Dv]");
  if (lse_part->shape[0] != R || lse_part->shape[1] != Hq)
    return fail(CPA_E_INVAL, "decode: lse_part must be [B, (Q,) Hq]");
  if (B == 0 || Hq == 0) return CPA_OK;

  DecodePlan p{};
  CPA_TRY(decode_plan(R, Hq, kcache, vcache, max_shard_len, &p));
  if (pg != nullptr) {
    p.nsplit = paged_nsplit(p.nsplit, max_shard_len, pg->shift);
    if (p.nsplit > (p.mla ? 64 : 256))
      return fail(CPA_E_UNSUPPORTED,
                  "decode_paged: %lld tokens per shard need more than %d pages per split at page size %d",
                  (long long)max_shard_len, cpa::kPageCap, 1 << pg->shift);
  }
  // workgroups: (row, split) for MLA, (request, kv head, head block, split)
  // for GQA, times the Q rows, rounded up to whole groups of 8 units
  const int64_t units = p.mla ? B * p.nsplit : B * Hkv * p.head_blocks * p.nsplit;
  const int64_t n_wg = (units + 7) / 8 * 8 * Q;
  if (n_wg > INT32_MAX) return fail(CPA_E_INVAL, "decode: %lld workgroups exceed the grid limit", (long long)n_wg);
  const size_t need = decode_ws_bytes(R, Hq, Dv, p.nsplit);
  if (lib_scratch && need > ws_bytes)
    return fail(CPA_E_CAPACITY,
                "decode_noalloc: this shape needs %zu bytes of split scratch, the library holds %zu per device; "
                "use attn_decode_shard with a workspace",
                need, ws_bytes);
  if (ws_bytes < need || (need > 0 && workspace == nullptr))
    return fail(CPA_E_CAPACITY, "decode: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (need > 0 && ((uintptr_t)workspace) % 256) return fail(CPA_E_INVAL, "decode: workspace must be 256-byte aligned");

  // partial-state destination: the caller's buffers directly, or the split
  // scratch [nsplit, B * Q, Hq, Dv] + [nsplit, B * Q, Hq] followed by a merge
  float* po;
  float* pl;
  int64_t po_s, po_b, po_h, pl_s, pl_b, pl_h;
  if (p.nsplit == 1) {
    po = static_cast<float*>(o_part->data);
    pl = static_cast<float*>(lse_part->data);
    po_s = 0, po_b = o_part->stride[0], po_h = o_part->stride[1];
    pl_s = 0, pl_b = lse_part->stride[0], pl_h = lse_part->stride[1];
  } else {
    po = static_cast<float*>(workspace);
    const size_t o_bytes = (size_t)p.nsplit * R * Hq * Dv * sizeof(float);
    pl = reinterpret_cast<float*>(static_cast<char*>(workspace) + (o_bytes + 255) / 256 * 256);
    po_h = Dv, po_b = Hq * Dv, po_s = R * Hq * Dv;
    pl_h = 1, pl_b = Hq, pl_s = R * Hq;
  }

  int err;
  if (p.mla) {
    cpa::DecodeMlaArgs a{};
    a.q = static_cast<const uint16_t*>(q->data);
    a.cache = kcache->data;
    a.kv_scale = fp8 ? static_cast<const float*>(kv_scale->data) : nullptr;
    a.kv_begin = kv_begin;
    a.kv_end = kv_end;
    a.o = po;
    a.lse = pl;
    a.q_b = q->stride[0];
    a.q_h = q->stride[1];
    a.c_b = kcache->stride[0];
    a.c_t = kcache->stride[1];
    a.s_b = fp8 ? kv_scale->stride[0] : 0;
    a.s_t = fp8 ? kv_scale->stride[1] : 0;
    a.o_s = po_s, a.o_b = po_b, a.o_h = po_h;
    a.l_s = pl_s, a.l_b = pl_b, a.l_h = pl_h;
    a.B = (int32_t)B;
    a.H = (int32_t)Hq;
    a.Lmax = (int32_t)Lmax;
    a.nsplit = p.nsplit;
    a.fp8 = fp8;
    a.scale_log2 = softmax_scale * kLog2e;
    a.Q = (int32_t)Q;
    a.q_q = q_q;
    if (pg != nullptr) {
      a.block_table = pg->table;
      a.bt_b = pg->stride;
      a.page_shift = pg->shift;
      a.n_pages = pg->n_pages;
    }
    err = cpa::launch_decode_mla(a, stream);
  } else {
    cpa::DecodeGqaArgs a{};
    a.q = q->data;
    a.k = kcache->data;
    a.v = vcache->data;
    a.kv_begin = kv_begin;
    a.kv_end = kv_end;
    a.o = po;
    a.lse = pl;
    a.q_b = q->stride[0];
    a.q_h = q->stride[1];
    a.k_b = kcache->stride[0], a.k_t = kcache->stride[1], a.k_h = kcache->stride[2];
    a.v_b = vcache->stride[0], a.v_t = vcache->stride[1], a.v_h = vcache->stride[2];
    a.o_s = po_s, a.o_b = po_b, a.o_h = po_h;
    a.l_s = pl_s, a.l_b = pl_b, a.l_h = pl_h;
    a.B = (int32_t)B;
    a.Hq = (int32_t)Hq;
    a.Hkv = (int32_t)Hkv;
    a.D = (int32_t)Dqk;
    a.Lmax = (int32_t)Lmax;
    a.nsplit = p.nsplit;
    a.q_bf16 = q->dtype == CPA_BF16;
    a.kv_dtype = kcache->dtype;
    a.kv_scale = fp8 ? static_cast<const float*>(kv_scale->data) : nullptr;
    a.s_b = fp8 ? kv_scale->stride[0] : 0;
    a.s_t = fp8 ? kv_scale->stride[1] : 0;
    a.scale_log2 = softmax_scale * kLog2e;
    a.Q = (int32_t)Q;
    a.q_q = q_q;
    if (pg != nullptr) {
      a.block_table = pg->table;
      a.bt_b = pg->stride;
      a.page_shift = pg->shift;
      a.n_pages = pg->n_pages;
    }
    err = cpa::launch_decode_gqa(a, stream);
  }
  CPA_TRY(hip_status(err, "decode launch"));
  if (p.nsplit > 1) {
    cpa::MergeArgs m{};
    m.o = po;
    m.lse = pl;
    m.out = o_part->data;
    m.lse_out = static_cast<float*>(lse_part->data);
    m.o_s = po_s, m.o_n = po_b, m.o_h = po_h;
    m.l_s = pl_s, m.l_n = pl_b, m.l_h = pl_h;
    m.out_n = o_part->stride[0], m.out_h = o_part->stride[1];
    m.lo_n = lse_part->stride[0], m.lo_h = lse_part->stride[1];
    m.S = p.nsplit;
    m.N = (int32_t)R;
    m.H = (int32_t)Hq;
    m.Dv = (int32_t)Dv;
    m.out_bf16 = 0;
    CPA_TRY(hip_status(cpa::launch_merge(m, stream), "decode split merge launch"));
  }
  return CPA_OK;
}

}  // namespace

extern "C" size_t attn_decode_workspace_size(int64_t batch, int32_t n_heads_q, int32_t head_dim_v,
                                             int64_t max_shard_len) {
  // MLA is recognised by its value width; GQA uses the general split rule
  // (the GQA rule picks fewer splits for more kv heads, so Hkv = 1 bounds it)
  const int ns = head_dim_v == 512 ? mla_nsplit(batch, max_shard_len) : gqa_nsplit(batch, max_shard_len);
  return decode_ws_bytes(batch, n_heads_q, head_dim_v, ns);
}

extern "C" cpa_status attn_decode_shard(const cpa_tensor* q, const cpa_tensor* kcache,
                                        const cpa_tensor* vcache, const cpa_tensor* kv_scale,
                                        const int32_t* kv_begin, const int32_t* kv_end,
                                        int64_t max_shard_len, float softmax_scale,
                                        const cpa_tensor* o_part, const cpa_tensor* lse_part,
                                        void* workspace, size_t ws_bytes, void* stream) {
  cpa::clear_error();
  return decode_impl(q, 1, 0, kcache, vcache, kv_scale, kv_begin, kv_end, max_shard_len, softmax_scale, o_part,
                     lse_part, workspace, ws_bytes, stream);
}

extern "C" cpa_status attn_decode_shard_noalloc(const cpa_tensor* q, const cpa_tensor* kcache,
                                                const cpa_tensor* vcache, const cpa_tensor* kv_scale,
                                                const int32_t* kv_begin, const int32_t* kv_end,
                                                int64_t max_shard_len, float softmax_scale,
                                                const cpa_tensor* o_part, const cpa_tensor* lse_part,
                                                void* stream) {
  cpa::clear_error();
  void* scratch = nullptr;
  CPA_TRY(hip_status(cpa::noalloc_scratch(&scratch), "decode_noalloc: scratch lookup"));
  return decode_impl(q, 1, 0, kcache, vcache, kv_scale, kv_begin, kv_end, max_shard_len, softmax_scale, o_part,
                     lse_part, scratch, cpa::kNoAllocScratchBytes, stream, true);
}

extern "C" size_t attn_decode_paged_workspace_size(int64_t batch, int32_t n_heads_q, int32_t head_dim_v,
                                                   int64_t max_shard_len, int32_t page_size) {
  if (page_size < 1 || (page_size & (page_size - 1)) || page_size > (1 << 20)) return 0;
  const int shift = __builtin_ctz((unsigned)page_size);
  const int ns = head_dim_v == 512 ? mla_nsplit(batch, max_shard_len) : gqa_nsplit(batch, max_shard_len);
  return decode_ws_bytes(batch, n_heads_q, head_dim_v, paged_nsplit(ns, max_shard_len, shift));
}

extern "C" cpa_status attn_decode_shard_paged(const cpa_tensor* q, const cpa_tensor* kpool, const cpa_tensor* vpool,
                                              const cpa_tensor* kv_scale, const int32_t* block_table,
                                              int64_t bt_stride, int64_t n_blocks, int32_t page_size,
                                              const int32_t* kv_begin, const int32_t* kv_end,
                                              int64_t max_shard_len, float softmax_scale,
                                              const cpa_tensor* o_part, const cpa_tensor* lse_part,
                                              void* workspace, size_t ws_bytes, void* stream) {
  cpa::clear_error();
  const unsigned kv_types = (1u << CPA_F32) | (1u << CPA_BF16) | (1u << CPA_FP8_E4M3);
  CPA_TRY(check_tensor(q, "decode_paged q", (1u << CPA_F32) | (1u << CPA_BF16), 3));
  CPA_TRY(check_tensor(kpool, "decode_paged kpool", kv_types, 3));
  if (page_size < 1 || (page_size & (page_size - 1)) || page_size > (1 << 20))
    return fail(CPA_E_INVAL, "decode_paged: page_size %d must be a power of two in [1, 2^20]", page_size);
  const int64_t B = q->shape[0], rows = kpool->shape[0];
  if (rows % page_size) return fail(CPA_E_INVAL, "decode_paged: kpool rows %lld not a multiple of page_size", (long long)rows);
  const int64_t n_pages = rows / page_size;
  if (n_pages > INT32_MAX) return fail(CPA_E_INVAL, "decode_paged: too many pages");
  if (n_blocks < 1 || n_blocks * (int64_t)page_size > INT32_MAX)
    return fail(CPA_E_INVAL, "decode_paged: n_blocks must be >= 1 with n_blocks * page_size < 2^31");
  if (bt_stride < n_blocks) return fail(CPA_E_INVAL, "decode_paged: block table row stride < n_blocks");
  if (B > 0 && block_table == nullptr) return fail(CPA_E_INVAL, "decode_paged: block_table is NULL");
  // [B, Lmax = n_blocks * page_size, Hkv, D] views whose request stride is 0:
  // every request reads the pool, through its own table row
  auto view4 = [&](const cpa_tensor* t) {
    cpa_tensor v = *t;
    v.ndim = 4;
    v.shape[0] = B, v.shape[1] = n_blocks * page_size, v.shape[2] = t->shape[1], v.shape[3] = t->shape[2];
    v.stride[0] = 0, v.stride[1] = t->stride[0], v.stride[2] = t->stride[1], v.stride[3] = t->stride[2];
    return v;
  };
  const cpa_tensor kv = view4(kpool);
  cpa_tensor vv{};
  if (vpool != nullptr) {
    CPA_TRY(check_tensor(vpool, "decode_paged vpool", kv_types, 3));
    if (vpool->shape[0] != rows) return fail(CPA_E_INVAL, "decode_paged: vpool rows differ from kpool");
    vv = view4(vpool);
  }
  cpa_tensor sv{};
  const bool has_scale = kv_scale != nullptr && kv_scale->data != nullptr;
  if (has_scale) {
    CPA_TRY(check_tensor(kv_scale, "decode_paged kv_scale", 1u << CPA_F32, 1, 0));
    if (kv_scale->shape[0] != rows) return fail(CPA_E_INVAL, "decode_paged: kv_scale must be f32 [pool rows]");
    sv = *kv_scale;
    sv.ndim = 2;
    sv.shape[0] = B, sv.shape[1] = n_blocks * page_size;
    sv.stride[0] = 0, sv.stride[1] = kv_scale->stride[0];
  }
  const Paging pg{block_table, bt_stride, __builtin_ctz((unsigned)page_size), (int32_t)n_pages};
  return decode_impl(q, 1, 0, &kv, vpool != nullptr ? &vv : nullptr, has_scale ? &sv : nullptr, kv_begin, kv_end,
                     max_shard_len, softmax_scale, o_part, lse_part, workspace, ws_bytes, stream, false, &pg);
}

extern "C" cpa_status attn_decode_shard_mq(const cpa_tensor* q, const cpa_tensor* kcache,
                                           const cpa_tensor* vcache, const cpa_tensor* kv_scale,
                                           const int32_t* kv_begin, const int32_t* kv_end,
                                           int64_t max_shard_len, float softmax_scale,
                                           const cpa_tensor* o_part, const cpa_tensor* lse_part,
                                           void* workspace, size_t ws_bytes, void* stream) {
  cpa::clear_error();
  CPA_TRY(check_tensor(q, "decode_mq q", (1u << CPA_F32) | (1u << CPA_BF16), 4));
  CPA_TRY(check_tensor(o_part, "decode_mq o_part", 1u << CPA_F32, 4));
  CPA_TRY(check_tensor(lse_part, "decode_mq lse_part", 1u << CPA_F32, 3, 0));
  const int64_t B = q->shape[0], Q = q->shape[1];
  if (Q < 1 || Q > 64) return fail(CPA_E_INVAL, "decode_mq: Q = %lld query rows per request, must be in [1, 64]", (long long)Q);
  if (o_part->shape[0] != B || o_part->shape[1] != Q || lse_part->shape[0] != B || lse_part->shape[1] != Q)
    return fail(CPA_E_INVAL, "decode_mq: o_part / lse_part must be [B, Q, ...] matching q");
  // (request, query row) of the outputs collapse into one row index b * Q + k
  const int64_t o_row = Q > 1 ? o_part->stride[1] : o_part->stride[0];
  const int64_t l_row = Q > 1 ? lse_part->stride[1] : lse_part->stride[0];
  if (B > 1 && Q > 1 && (o_part->stride[0] != Q * o_row || lse_part->stride[0] != Q * l_row))
    return fail(CPA_E_INVAL, "decode_mq: o_part / lse_part must have stride[0] == Q * stride[1]");
  cpa_tensor q3 = *q, o3 = *o_part, l2 = *lse_part;
  q3.ndim = 3;
  q3.shape[1] = q->shape[2], q3.shape[2] = q->shape[3];
  q3.stride[1] = q->stride[2], q3.stride[2] = q->stride[3];
  o3.ndim = 3;
  o3.shape[0] = B * Q, o3.shape[1] = o_part->shape[2], o3.shape[2] = o_part->shape[3];
  o3.stride[0] = o_row, o3.stride[1] = o_part->stride[2], o3.stride[2] = o_part->stride[3];
  o3.stride[3] = 0;
  l2.ndim = 2;
  l2.shape[0] = B * Q, l2.shape[1] = lse_part->shape[2];
  l2.stride[0] = l_row, l2.stride[1] = lse_part->stride[2];
  // query rows of one request may sit at any (aligned) stride from each other
  return decode_impl(&q3, Q, Q > 1 ? q->stride[1] : 0, kcache, vcache, kv_scale, kv_begin, kv_end, max_shard_len, softmax_scale,
                     &o3, &l2, workspace, ws_bytes, stream);
}

// ----------------------------------------------------------- sparse (top-k)

extern "C" size_t attn_sparse_mla_workspace_size(int64_t n_queries, int32_t k) {
  return decode_ws_bytes(n_queries, 64, 512, mla_nsplit(n_queries, k));
}

extern "C" cpa_status attn_sparse_mla(const cpa_tensor* q, const cpa_tensor* cache, const cpa_tensor* kv_scale,
                                      const int32_t* req, const int32_t* idx, int64_t idx_stride, int32_t k,
                                      const int32_t* n_idx, float softmax_scale, const cpa_tensor* out,
                                      const cpa_tensor* lse, void* workspace, size_t ws_bytes, void* stream) {
  cpa::clear_error();
  CPA_TRY(check_tensor(q, "sparse q", 1u << CPA_BF16, 3));
  CPA_TRY(check_tensor(cache, "sparse cache", (1u << CPA_BF16) | (1u << CPA_FP8_E4M3), 4));
  CPA_TRY(check_tensor(out, "sparse out", 1u << CPA_F32, 3));
  CPA_TRY(check_tensor(lse, "sparse lse", 1u << CPA_F32, 2, 0));
  const int64_t N = q->shape[0], B = cache->shape[0], Lmax = cache->shape[1];
  if (q->shape[1] != 64 || q->shape[2] != 576)
    return fail(CPA_E_UNSUPPORTED, "sparse: q must be [N, 64, 576] (the MLA kernel's shape)");
  if (cache->shape[2] != 1 || cache->shape[3] != 576) return fail(CPA_E_INVAL, "sparse: cache must be [B, Lmax, 1, 576]");
  if (out->shape[0] != N || out->shape[1] != 64 || out->shape[2] != 512)
    return fail(CPA_E_INVAL, "sparse: out must be [N, 64, 512]");
  if (lse->shape[0] != N || lse->shape[1] != 64) return fail(CPA_E_INVAL, "sparse: lse must be [N, 64]");
  if (k < 0 || idx_stride < k) return fail(CPA_E_INVAL, "sparse: k = %d, idx_stride = %lld", k, (long long)idx_stride);
  if (N > INT32_MAX || B > INT32_MAX || Lmax > INT32_MAX) return fail(CPA_E_INVAL, "sparse: sizes too large");
  if (N > 0 && k > 0 && idx == nullptr) return fail(CPA_E_INVAL, "sparse: idx is NULL");
  if (req == nullptr && N > B && Lmax > 0) return fail(CPA_E_INVAL, "sparse: without req, query n uses request n < B");
  if ((uintptr_t)idx % 4) return fail(CPA_E_INVAL, "sparse: idx must be 4-byte aligned");
  const bool fp8 = cache->dtype == CPA_FP8_E4M3;
  const int64_t esz = fp8 ? 1 : 2;
  // rows are addressed with 32-bit byte offsets from the request's base
  if (Lmax > 0 && (Lmax - 1) * cache->stride[1] * esz + esz * 576 > (int64_t)UINT32_MAX)
    return fail(CPA_E_INVAL, "sparse: a request's cache spans more than 4 GiB");
  if (fp8) {
    if (kv_scale == nullptr || kv_scale->data == nullptr) return fail(CPA_E_INVAL, "sparse: FP8 cache needs kv_scale");
    CPA_TRY(check_tensor(kv_scale, "sparse kv_scale", 1u << CPA_F32, 2, 0));
    if (kv_scale->shape[0] != B || kv_scale->shape[1] != Lmax)
      return fail(CPA_E_INVAL, "sparse: kv_scale must be f32 [B, Lmax]");
    if (Lmax > 0 && (Lmax - 1) * kv_scale->stride[1] * 4 + 4 > (int64_t)UINT32_MAX)
      return fail(CPA_E_INVAL, "sparse: a request's scales span more than 4 GiB");
    if (cache->stride[1] % 16 || cache->stride[0] % 16)
      return fail(CPA_E_INVAL, "sparse: FP8 rows must start on 16-byte boundaries");
  } else if (kv_scale != nullptr && kv_scale->data != nullptr) {
    return fail(CPA_E_INVAL, "sparse: kv_scale is only for an FP8 cache");
  }
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(CPA_E_INVAL, "sparse: softmax_scale must be finite and > 0");
  if (N == 0) return CPA_OK;
  const int ns = mla_nsplit(N, k);
  if (N * ns > INT32_MAX) return fail(CPA_E_INVAL, "sparse: too many workgroups");
  const size_t need = decode_ws_bytes(N, 64, 512, ns);
  if (ws_bytes < need || (need > 0 && workspace == nullptr))
    return fail(CPA_E_CAPACITY, "sparse: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (need > 0 && ((uintptr_t)workspace) % 256) return fail(CPA_E_INVAL, "sparse: workspace must be 256-byte aligned");

  cpa::SparseMlaArgs a{};
  float* po;
  float* pl;
  if (ns == 1) {
    po = static_cast<float*>(out->data);
    pl = static_cast<float*>(lse->data);
    a.o_s = 0, a.o_n = out->stride[0], a.o_h = out->stride[1];
    a.l_s = 0, a.l_n = lse->stride[0], a.l_h = lse->stride[1];
  } else {
    po = static_cast<float*>(workspace);
    const size_t o_bytes = (size_t)ns * N * 64 * 512 * sizeof(float);
    pl = reinterpret_cast<float*>(static_cast<char*>(workspace) + (o_bytes + 255) / 256 * 256);
    a.o_s = N * 64 * 512, a.o_n = 64 * 512, a.o_h = 512;
    a.l_s = N * 64, a.l_n = 64, a.l_h = 1;
  }
  a.q = static_cast<const uint16_t*>(q->data);
  a.cache = cache->data;
  a.kv_scale = fp8 ? static_cast<const float*>(kv_scale->data) : nullptr;
  a.s_b = fp8 ? kv_scale->stride[0] : 0;
  a.s_t = fp8 ? kv_scale->stride[1] : 0;
  a.fp8 = fp8;
  a.req = req;
  a.idx = idx;
  a.n_idx = n_idx;
  a.o = po;
  a.lse = pl;
  a.q_n = q->stride[0], a.q_h = q->stride[1];
  a.c_b = cache->stride[0], a.c_t = cache->stride[1];
  a.i_n = idx_stride;
  a.N = (int32_t)N, a.B = (int32_t)B, a.K = k, a.Lmax = (int32_t)Lmax, a.nsplit = ns;
  // one query per request reads its rows once; several share them through L2
  a.reuse = req != nullptr;
  a.scale_log2 = softmax_scale * kLog2e;
  CPA_TRY(hip_status(cpa::launch_sparse_mla(a, stream), "sparse launch"));
  if (ns > 1) {
    cpa::MergeArgs m{};
    m.o = po;
    m.lse = pl;
    m.out = out->data;
    m.lse_out = static_cast<float*>(lse->data);
    m.o_s = a.o_s, m.o_n = a.o_n, m.o_h = a.o_h;
    m.l_s = a.l_s, m.l_n = a.l_n, m.l_h = a.l_h;
    m.out_n = out->stride[0], m.out_h = out->stride[1];
    m.lo_n = lse->stride[0], m.lo_h = lse->stride[1];
    m.S = ns;
    m.N = (int32_t)N;
    m.H = 64;
    m.Dv = 512;
    m.out_bf16 = 0;
    CPA_TRY(hip_status(cpa::launch_merge(m, stream), "sparse split merge launch"));
  }
  return CPA_OK;
}

// ------------------------------------------------------ distributed top-k

extern "C" cpa_status attn_topk_local(const float* scores, int64_t score_stride, int32_t n_rows, int32_t L,
                                      const int32_t* n_valid, int32_t k, int64_t id_base, int64_t id_stride,
                                      float* out_score, int32_t* out_id, int32_t* out_row, int32_t* out_count,
                                      void* stream) {
  cpa::clear_error();
  if (n_rows < 0 || L < 0 || k < 0) return fail(CPA_E_INVAL, "topk_local: negative n_rows, L or k");
  if (score_stride < L) return fail(CPA_E_INVAL, "topk_local: score_stride %lld < L", (long long)score_stride);
  if (n_rows == 0) return CPA_OK;
  if (L > 0 && scores == nullptr) return fail(CPA_E_INVAL, "topk_local: scores is NULL");
  if (out_count == nullptr || (k > 0 && (!out_score || !out_id || !out_row)))
    return fail(CPA_E_INVAL, "topk_local: NULL output");
  if (((uintptr_t)scores | (uintptr_t)out_score | (uintptr_t)out_id | (uintptr_t)out_row | (uintptr_t)out_count |
       (uintptr_t)n_valid) % 4)
    return fail(CPA_E_INVAL, "topk_local: arrays must be 4-byte aligned");
  // global ids of rows 0 .. L-1 must be int32 values >= 0
  const int64_t last = L > 0 ? id_base + (int64_t)(L - 1) * id_stride : id_base;
  if (id_base < 0 || last < 0 || id_base > INT32_MAX || last > INT32_MAX)
    return fail(CPA_E_INVAL, "topk_local: global ids outside [0, 2^31)");
  if (L > 1 && id_stride == 0) return fail(CPA_E_INVAL, "topk_local: id_stride 0 gives equal ids");
  cpa::TopkLocalArgs a{};
  a.scores = scores, a.n_valid = n_valid, a.out_score = out_score, a.out_id = out_id, a.out_row = out_row;
  a.out_count = out_count;
  a.s_n = score_stride, a.id_base = id_base, a.id_stride = id_stride;
  a.N = n_rows, a.L = L, a.k = k;
  return hip_status(cpa::launch_topk_local(a, stream), "topk_local launch");
}

extern "C" cpa_status attn_topk_merge(int32_t P, int32_t n_rows, int32_t k_in, const float* cand_score,
                                      const int32_t* cand_id, const int32_t* cand_row, const int32_t* cand_count,
                                      int32_t k, int32_t* out_id, int32_t* owner_row, int32_t* owner_count,
                                      void* stream) {
  cpa::clear_error();
  if (P < 1 || P > 64 || n_rows < 0 || k_in < 0 || k < 0)
    return fail(CPA_E_INVAL, "topk_merge: bad P (1..64), n_rows, k_in or k");
  if ((int64_t)P * k_in > INT32_MAX) return fail(CPA_E_INVAL, "topk_merge: P * k_in too large");
  if (n_rows == 0) return CPA_OK;
  if (k_in > 0 && (!cand_score || !cand_id || !cand_row)) return fail(CPA_E_INVAL, "topk_merge: NULL candidates");
  if (owner_count == nullptr || (k > 0 && (!out_id || !owner_row))) return fail(CPA_E_INVAL, "topk_merge: NULL output");
  if (((uintptr_t)cand_score | (uintptr_t)cand_id | (uintptr_t)cand_row | (uintptr_t)cand_count | (uintptr_t)out_id |
       (uintptr_t)owner_row | (uintptr_t)owner_count) % 4)
    return fail(CPA_E_INVAL, "topk_merge: arrays must be 4-byte aligned");
  cpa::TopkMergeArgs a{};
  a.cand_score = cand_score, a.cand_id = cand_id, a.cand_row = cand_row, a.cand_count = cand_count;
  a.out_id = out_id, a.owner_row = owner_row, a.owner_count = owner_count;
  a.P = P, a.N = n_rows, a.k_in = k_in, a.k = k;
  return hip_status(cpa::launch_topk_merge(a, stream), "topk_merge launch");
}

// ------------------------------------------------------------------- prefill

namespace {

// Every segment must stay inside q / out / lse rows and the packed K/V rows;
// segments must not share q rows (they would race on the same outputs).
cpa_status check_segments(const cpa_segment* seg, int32_t n_seg, int64_t n_local, int64_t T_kv) {
  if (n_seg < 0) return fail(CPA_E_INVAL, "prefill: n_seg < 0");
  if (n_seg > 0 && seg == nullptr) return fail(CPA_E_INVAL, "prefill: segments are NULL");
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (int32_t i = 0; i < n_seg; ++i) {
    const cpa_segment& s = seg[i];
    if (s.q_len < 0 || s.q_row0 < 0 || s.pos0 < 0 || s.kv_row0 < 0)
      return fail(CPA_E_INVAL, "prefill: segment %d has a negative field", i);
    if (s.q_len == 0) continue;
    if (s.q_len > 1 && s.pos_stride < 1) return fail(CPA_E_INVAL, "prefill: segment %d has pos_stride < 1", i);
    if ((int64_t)s.q_row0 + s.q_len > n_local)
      return fail(CPA_E_INVAL, "prefill: segment %d rows [%d, %lld) exceed n_local = %lld", i, s.q_row0,
                  (long long)s.q_row0 + s.q_len, (long long)n_local);
    const int64_t last = (int64_t)s.pos0 + (int64_t)(s.q_len - 1) * (s.q_len > 1 ? s.pos_stride : 0);
    if (last > INT32_MAX) return fail(CPA_E_INVAL, "prefill: segment %d positions exceed int32", i);
    if (s.kv_row0 + last + 1 > T_kv)
      return fail(CPA_E_INVAL, "prefill: segment %d reads K/V rows up to %lld but T_kv = %lld", i,
                  (long long)(s.kv_row0 + last + 1), (long long)T_kv);
    spans.emplace_back(s.q_row0, (int64_t)s.q_row0 + s.q_len);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return fail(CPA_E_INVAL, "prefill: segments overlap in q rows");
  return CPA_OK;
}

}  // namespace

extern "C" cpa_status attn_prefill_shard(const cpa_tensor* q, const cpa_tensor* k, const cpa_tensor* v,
                                         const cpa_segment* seg, int32_t n_seg, float softmax_scale,
                                         const cpa_tensor* out, const cpa_tensor* lse, void* stream) {
  cpa::clear_error();
  CPA_TRY(check_tensor(q, "prefill q", 1u << CPA_BF16, 3));
  CPA_TRY(check_tensor(k, "prefill k", 1u << CPA_BF16, 3));
  CPA_TRY(check_tensor(out, "prefill out", (1u << CPA_BF16) | (1u << CPA_F32), 3));
  CPA_TRY(check_tensor(lse, "prefill lse", 1u << CPA_F32, 2, 0));
  const int64_t n_local = q->shape[0], Hq = q->shape[1], Dqk = q->shape[2];
  const int64_t T_kv = k->shape[0], Hkv = k->shape[1];
  if (k->shape[2] != Dqk) return fail(CPA_E_INVAL, "prefill: k head dim differs from q");
  if (Hkv < 1 || Hq % Hkv) return fail(CPA_E_INVAL, "prefill: Hq = %lld not a multiple of Hkv = %lld", (long long)Hq, (long long)Hkv);
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(CPA_E_INVAL, "prefill: softmax_scale must be finite and > 0");
  if (n_local > INT32_MAX || T_kv > ((int64_t)1 << 40)) return fail(CPA_E_INVAL, "prefill: sizes too large");
  int64_t Dv;
  if (v == nullptr) {
    if (Hkv != 1 || Dqk != 576) return fail(CPA_E_UNSUPPORTED, "prefill: MLA (v = NULL) needs Hkv = 1 and Dqk = 576");
    Dv = 512;
  } else {
    CPA_TRY(check_tensor(v, "prefill v", 1u << CPA_BF16, 3));
    if (v->shape[0] != T_kv || v->shape[1] != Hkv) return fail(CPA_E_INVAL, "prefill: v must be [T_kv, Hkv, Dv]");
    Dv = v->shape[2];
  }
  if (out->shape[0] != n_local || out->shape[1] != Hq || out->shape[2] != Dv)
    return fail(CPA_E_INVAL, "prefill: out must be [n_local, Hq, Dv]");
  if (lse->shape[0] != n_local || lse->shape[1] != Hq) return fail(CPA_E_INVAL, "prefill: lse must be [n_local, Hq]");
  CPA_TRY(check_segments(seg, n_seg, n_local, T_kv));
  if (n_local == 0 || n_seg == 0) return CPA_OK;
  if (v != nullptr) {
    if (Dqk != 128 || Dv != 128) return fail(CPA_E_UNSUPPORTED, "prefill: GQA kernel is built for head dim 128");
    const int64_t G = Hq / Hkv;
    if (G > 128 || (128 % G) != 0) return fail(CPA_E_UNSUPPORTED, "prefill: Hq / Hkv = %lld must divide 128", (long long)G);
    // the kernel addresses a 64-key tile with 32-bit per-lane byte offsets
    if (k->stride[0] >= ((int64_t)1 << 24) || v->stride[0] >= ((int64_t)1 << 24))
      return fail(CPA_E_INVAL, "prefill: k / v token stride too large");
    cpa::PrefillGqaArgs a{};
    a.q = static_cast<const uint16_t*>(q->data);
    a.k = static_cast<const uint16_t*>(k->data);
    a.v = static_cast<const uint16_t*>(v->data);
    a.out = out->data;
    a.lse = static_cast<float*>(lse->data);
    a.q_n = q->stride[0], a.q_h = q->stride[1];
    a.k_t = k->stride[0], a.k_h = k->stride[1];
    a.v_t = v->stride[0], a.v_h = v->stride[1];
    a.o_n = out->stride[0], a.o_h = out->stride[1];
    a.l_n = lse->stride[0], a.l_h = lse->stride[1];
    a.Hkv = (int32_t)Hkv;
    a.G = (int32_t)G;
    a.out_bf16 = out->dtype == CPA_BF16;
    a.scale_log2 = softmax_scale * kLog2e;
    return hip_status(cpa::launch_prefill_gqa(a, seg, n_seg, stream), "prefill launch");
  }
  if (Hq != 64) return fail(CPA_E_UNSUPPORTED, "prefill: MLA kernel is built for 64 query heads, got %lld", (long long)Hq);
  // the kernel addresses a 32-token tile with 32-bit per-thread byte offsets
  if (k->stride[0] > ((int64_t)1 << 26)) return fail(CPA_E_INVAL, "prefill: latent token stride too large");
  cpa::PrefillMlaArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.lat = static_cast<const uint16_t*>(k->data);
  a.out = out->data;
  a.lse = static_cast<float*>(lse->data);
  a.q_n = q->stride[0], a.q_h = q->stride[1];
  a.k_t = k->stride[0];
  a.o_n = out->stride[0], a.o_h = out->stride[1];
  a.l_n = lse->stride[0], a.l_h = lse->stride[1];
  a.out_bf16 = out->dtype == CPA_BF16;
  a.scale_log2 = softmax_scale * kLog2e;
  return hip_status(cpa::launch_prefill_mla(a, seg, n_seg, stream), "prefill launch");
}

// ------------------------------------------------------ round-robin cache write

extern "C" cpa_status attn_cache_write_round_robin(int32_t C, int32_t rank, int32_t n_repl, const cpa_tensor* src,
                                                   const int64_t* slot, const int32_t* req, const cpa_tensor* dst,
                                                   void* stream) {
  cpa::clear_error();
  if (C < 1 || rank < 0 || rank >= C) return fail(CPA_E_INVAL, "cache write: bad C = %d or rank = %d", C, rank);
  if (n_repl < 0) return fail(CPA_E_INVAL, "cache write: n_repl < 0");
  const unsigned any = (1u << CPA_F32) | (1u << CPA_BF16) | (1u << CPA_FP8_E4M3);
  CPA_TRY(check_tensor(src, "cache write src", any, 2, 4));
  CPA_TRY(check_tensor(dst, "cache write dst", any, 3, 4));
  if (src->dtype != dst->dtype) return fail(CPA_E_INVAL, "cache write: src and dst dtypes differ");
  if (src->shape[1] != dst->shape[2]) return fail(CPA_E_INVAL, "cache write: src rows and dst rows differ in width");
  const int64_t es = elem_size(src->dtype);
  const int64_t row_bytes = src->shape[1] * es;
  if (row_bytes % 4) return fail(CPA_E_INVAL, "cache write: row of %lld bytes is not a multiple of 4", (long long)row_bytes);
  const int64_t n = src->shape[0];
  if (n == 0 || dst->shape[0] == 0 || dst->shape[1] == 0) return CPA_OK;
  if (slot == nullptr || req == nullptr) return fail(CPA_E_INVAL, "cache write: slot / req is NULL");
  if (((uintptr_t)slot) % 8 || ((uintptr_t)req) % 4) return fail(CPA_E_INVAL, "cache write: slot / req misaligned");
  if (dst->shape[0] > INT32_MAX) return fail(CPA_E_INVAL, "cache write: too many requests");
  cpa::CacheWriteArgs a{};
  a.src = static_cast<const char*>(src->data);
  a.slot = slot;
  a.req = req;
  a.dst = static_cast<char*>(dst->data);
  a.n = n;
  a.src_row = src->stride[0] * es;
  a.dst_b = dst->stride[0] * es;
  a.dst_row = dst->stride[1] * es;
  a.row_bytes = row_bytes;
  a.C = C;
  a.rank = rank;
  a.n_repl = n_repl;
  a.B = (int32_t)dst->shape[0];
  a.Lmax = dst->shape[1];
  a.vec16 = row_bytes % 16 == 0 && a.src_row % 16 == 0 && a.dst_b % 16 == 0 && a.dst_row % 16 == 0 &&
            ((uintptr_t)src->data) % 16 == 0 && ((uintptr_t)dst->data) % 16 == 0;
  return hip_status(cpa::launch_cache_write_rr(a, stream), "cache write launch");
}
