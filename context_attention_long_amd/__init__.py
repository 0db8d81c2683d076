"""Python binding of libcpattn (context-parallel attention shards, gfx950).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the current stream. The library is built
in-tree (``python -m context_attention_long_amd.build``); if it is missing,
every call raises: there is no fallback.

Names follow the C ABI in ``include/cpattn.h``:
``cp_plan_zigzag``, ``cp_plan_interleave``, ``cp_decode_shards``,
``attn_prefill_shard``, ``attn_decode_shard``, ``attn_merge_states``.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcpattn.so")

CPA_OK, CPA_E_INVAL, CPA_E_UNSUPPORTED, CPA_E_CAPACITY, CPA_E_HIP = range(5)
CPA_F32, CPA_BF16, CPA_FP8_E4M3 = 0, 1, 2
CPA_LAYOUT_CONTIGUOUS, CPA_LAYOUT_ROUND_ROBIN = 0, 1

_STATUS = {1: "CPA_E_INVAL", 2: "CPA_E_UNSUPPORTED", 3: "CPA_E_CAPACITY", 4: "CPA_E_HIP"}


class CpaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class CpaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class CpaSegment(ctypes.Structure):
    _fields_ = [("req", ctypes.c_int32), ("q_row0", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("pos0", ctypes.c_int32), ("pos_stride", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("kv_row0", ctypes.c_int64)]


class CpaPlan(ctypes.Structure):
    _fields_ = [("tok_index", ctypes.POINTER(ctypes.c_int64)), ("pos_id", ctypes.POINTER(ctypes.c_int32)),
                ("req_id", ctypes.POINTER(ctypes.c_int32)), ("cap_local", ctypes.c_int64),
                ("seg", ctypes.POINTER(CpaSegment)), ("cap_seg", ctypes.c_int64),
                ("n_local", ctypes.c_int64), ("n_seg", ctypes.c_int64), ("n_padded", ctypes.c_int64)]


SEGMENT_DTYPE = np.dtype([("req", np.int32), ("q_row0", np.int32), ("q_len", np.int32), ("pos0", np.int32),
                          ("pos_stride", np.int32), ("reserved", np.int32), ("kv_row0", np.int64)])
assert SEGMENT_DTYPE.itemsize == ctypes.sizeof(CpaSegment) == 32

# exported symbols of include/cpattn.h
SYMBOLS = ("cpa_last_error", "cpa_abi_version", "cp_plan_zigzag", "cp_plan_interleave", "cp_decode_shards",
           "attn_prefill_shard", "attn_decode_workspace_size", "attn_decode_shard", "attn_merge_states",
           "cp_round_robin_slot", "cp_plan_round_robin", "attn_cache_write_round_robin",
           "attn_decode_shard_mq", "cp_plan_multi_query", "attn_sparse_mla_workspace_size", "attn_sparse_mla",
           "attn_topk_local", "attn_topk_merge", "attn_decode_shard_noalloc", "attn_decode_paged_workspace_size",
           "attn_decode_shard_paged")

_lib_handle = None


def lib():
    """Load libcpattn.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m context_attention_long_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.cpa_last_error.restype = ctypes.c_char_p
        L.cpa_abi_version.restype = ctypes.c_int32
        for name in ("cp_plan_zigzag", "cp_plan_interleave"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int32),
                          P(CpaPlan)]
        L.cp_decode_shards.restype = ctypes.c_int
        L.cp_decode_shards.argtypes = [ctypes.c_int64, ctypes.c_int32, P(ctypes.c_int64), P(ctypes.c_int64)]
        L.attn_prefill_shard.restype = ctypes.c_int
        L.attn_prefill_shard.argtypes = [P(CpaTensor), P(CpaTensor), P(CpaTensor), P(CpaSegment), ctypes.c_int32,
                                         ctypes.c_float, P(CpaTensor), P(CpaTensor), ctypes.c_void_p]
        L.attn_decode_workspace_size.restype = ctypes.c_size_t
        L.attn_decode_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
        L.attn_decode_shard.restype = ctypes.c_int
        L.attn_decode_shard.argtypes = [P(CpaTensor), P(CpaTensor), P(CpaTensor), P(CpaTensor), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, P(CpaTensor),
                                        P(CpaTensor), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.attn_decode_shard_noalloc.restype = ctypes.c_int
        L.attn_decode_shard_noalloc.argtypes = [P(CpaTensor), P(CpaTensor), P(CpaTensor), P(CpaTensor),
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                                P(CpaTensor), P(CpaTensor), ctypes.c_void_p]
        L.attn_decode_shard_mq.restype = ctypes.c_int
        L.attn_decode_shard_mq.argtypes = L.attn_decode_shard.argtypes
        L.attn_decode_paged_workspace_size.restype = ctypes.c_size_t
        L.attn_decode_paged_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.c_int64, ctypes.c_int32]
        L.attn_decode_shard_paged.restype = ctypes.c_int
        L.attn_decode_shard_paged.argtypes = [P(CpaTensor), P(CpaTensor), P(CpaTensor), P(CpaTensor),
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                              P(CpaTensor), P(CpaTensor), ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p]
        L.cp_plan_multi_query.restype = ctypes.c_int
        L.cp_plan_multi_query.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          P(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          P(ctypes.c_int32), P(ctypes.c_int32), P(ctypes.c_int64)]
        L.attn_sparse_mla_workspace_size.restype = ctypes.c_size_t
        L.attn_sparse_mla_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.attn_sparse_mla.restype = ctypes.c_int
        L.attn_sparse_mla.argtypes = [P(CpaTensor), P(CpaTensor), P(CpaTensor), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, P(CpaTensor),
                                      P(CpaTensor), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        vp = ctypes.c_void_p
        L.attn_topk_local.restype = ctypes.c_int
        L.attn_topk_local.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int32,
                                      ctypes.c_int64, ctypes.c_int64, vp, vp, vp, vp, vp]
        L.attn_topk_merge.restype = ctypes.c_int
        L.attn_topk_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_int32,
                                      vp, vp, vp, vp]
        L.cp_round_robin_slot.restype = ctypes.c_int
        L.cp_round_robin_slot.argtypes = [ctypes.c_int64, ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int64)]
        L.cp_plan_round_robin.restype = ctypes.c_int
        L.cp_plan_round_robin.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int64),
                                          ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int32),
                                          P(ctypes.c_int64)]
        L.attn_cache_write_round_robin.restype = ctypes.c_int
        L.attn_cache_write_round_robin.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(CpaTensor),
                                                   ctypes.c_void_p, ctypes.c_void_p, P(CpaTensor), ctypes.c_void_p]
        L.attn_merge_states.restype = ctypes.c_int
        L.attn_merge_states.argtypes = [ctypes.c_int32, P(CpaTensor), P(CpaTensor), P(CpaTensor), P(CpaTensor),
                                        ctypes.c_void_p]
        _lib_handle = L
    return _lib_handle


def _check(status):
    if status != CPA_OK:
        raise CpaError(status, lib().cpa_last_error().decode())


def _i32(a):
    return (ctypes.c_int32 * len(a))(*[int(x) for x in a])


# ------------------------------------------------------------------ planners

class Plan:
    """Host plan of one rank: numpy arrays tok_index, pos_id, req_id and a
    structured ``segments`` array (SEGMENT_DTYPE), plus n_padded."""

    def __init__(self, tok_index, pos_id, req_id, segments, n_padded):
        self.tok_index, self.pos_id, self.req_id = tok_index, pos_id, req_id
        self.segments, self.n_padded = segments, n_padded

    @property
    def n_local(self):
        return len(self.tok_index)

    @property
    def n_seg(self):
        return len(self.segments)


def _plan(fn_name, C, rank, new_len, prefix_len):
    f = getattr(lib(), fn_name)
    n = len(new_len)
    nl = _i32(new_len)
    pl = _i32(prefix_len) if prefix_len is not None else None
    out = CpaPlan()
    st = f(C, rank, n, nl, pl, ctypes.byref(out))
    if st not in (CPA_OK, CPA_E_CAPACITY):
        _check(st)
    tok = np.empty(out.n_local, np.int64)
    pos = np.empty(out.n_local, np.int32)
    req = np.empty(out.n_local, np.int32)
    seg = np.zeros(out.n_seg, SEGMENT_DTYPE)
    out.tok_index = tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out.pos_id = pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    out.req_id = req.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    out.cap_local = out.n_local
    out.seg = seg.ctypes.data_as(ctypes.POINTER(CpaSegment))
    out.cap_seg = out.n_seg
    _check(f(C, rank, n, nl, pl, ctypes.byref(out)))
    return Plan(tok, pos, req, seg, int(out.n_padded))


def cp_plan_zigzag(C, rank, new_len, prefix_len=None):
    return _plan("cp_plan_zigzag", C, rank, new_len, prefix_len)


def cp_plan_interleave(C, rank, new_len, prefix_len=None):
    return _plan("cp_plan_interleave", C, rank, new_len, prefix_len)


def cp_decode_shards(L, C):
    b = (ctypes.c_int64 * C)()
    e = (ctypes.c_int64 * C)()
    _check(lib().cp_decode_shards(int(L), int(C), b, e))
    return list(zip(list(b), list(e)))


def cp_round_robin_slot(slot, C):
    """(rank, row) of a slot in round-robin decode storage."""
    r = ctypes.c_int32()
    row = ctypes.c_int64()
    _check(lib().cp_round_robin_slot(int(slot), int(C), ctypes.byref(r), ctypes.byref(row)))
    return r.value, row.value


def cp_plan_round_robin(C, rank, ctx_len, n_repl=0, repl_rank=0):
    """Per-request decode range of `rank` in its round-robin local cache:
    (kv_begin int32 array, kv_end int32 array, rows a local cache needs)."""
    n = len(ctx_len)
    cl = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in ctx_len])
    beg = np.zeros(n, np.int32)
    end = np.zeros(n, np.int32)
    mx = ctypes.c_int64()
    _check(lib().cp_plan_round_robin(int(C), int(rank), n, cl, int(n_repl), int(repl_rank),
                                     beg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     end.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(mx)))
    return beg, end, mx.value


def cp_plan_multi_query(layout, C, rank, ctx_len, Q, n_repl=0, repl_rank=0):
    """Per-row decode ranges of `rank` for Q query rows per request (the last
    Q slots of each request): (kv_begin int32 [n_req], kv_end int32
    [n_req * Q], rows a local cache needs). layout: CPA_LAYOUT_CONTIGUOUS or
    CPA_LAYOUT_ROUND_ROBIN."""
    n = len(ctx_len)
    cl = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in ctx_len])
    beg = np.zeros(n, np.int32)
    end = np.zeros(max(n * int(Q), 0), np.int32)
    mx = ctypes.c_int64()
    _check(lib().cp_plan_multi_query(int(layout), int(C), int(rank), n, cl, int(Q), int(n_repl), int(repl_rank),
                                     beg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     end.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(mx)))
    return beg, end, mx.value


# ------------------------------------------------------------------ tensors

def _torch():
    import torch
    return torch


def tensor_desc(t, dtype=None):
    """cpa_tensor for a torch tensor (dtype override for raw FP8 bytes)."""
    torch = _torch()
    if dtype is None:
        dtype = {torch.float32: CPA_F32, torch.bfloat16: CPA_BF16, torch.uint8: CPA_FP8_E4M3}.get(t.dtype)
        if dtype is None and hasattr(torch, "float8_e4m3fn") and t.dtype == torch.float8_e4m3fn:
            dtype = CPA_FP8_E4M3
        if dtype is None:
            raise TypeError(f"unsupported dtype {t.dtype}")
    d = CpaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = dtype
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(d):
    return ctypes.byref(d) if d is not None else None


# ------------------------------------------------------------------ attention

def attn_prefill_shard(q, k, v, segments, softmax_scale, out=None, lse=None, out_dtype=None, stream=None):
    """Causal attention of local queries q [n_local, Hq, Dqk] against packed
    k [T_kv, Hkv, Dqk] / v [T_kv, Hkv, Dv] (v=None: MLA, value = k[..., :512]).
    ``segments``: host structured array (SEGMENT_DTYPE). Returns (out, lse)."""
    torch = _torch()
    n_local, Hq = q.shape[0], q.shape[1]
    Dv = v.shape[-1] if v is not None else 512
    if out is None:
        out = torch.empty((n_local, Hq, Dv), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((n_local, Hq), dtype=torch.float32, device=q.device)
    seg = np.ascontiguousarray(segments, dtype=SEGMENT_DTYPE)
    dq, dk, do, dl = tensor_desc(q), tensor_desc(k), tensor_desc(out), tensor_desc(lse)
    dv = tensor_desc(v) if v is not None else None
    _check(lib().attn_prefill_shard(ctypes.byref(dq), ctypes.byref(dk), _ptr(dv),
                                    seg.ctypes.data_as(ctypes.POINTER(CpaSegment)), len(seg),
                                    float(softmax_scale), ctypes.byref(do), ctypes.byref(dl), _stream(stream)))
    return out, lse


def attn_decode_workspace_size(batch, n_heads_q, head_dim_v, max_shard_len):
    return int(lib().attn_decode_workspace_size(int(batch), int(n_heads_q), int(head_dim_v), int(max_shard_len)))


def attn_decode_shard(q, kcache, vcache, kv_begin, kv_end, max_shard_len, softmax_scale, kv_scale=None,
                      o_part=None, lse_part=None, workspace=None, stream=None, kcache_dtype=None):
    """Split-KV decode of one shard. q [B, Hq, Dqk]; kcache [B, Lmax, Hkv, Dqk]
    (torch.uint8 = FP8 E4M3 bytes, then kv_scale [B, Lmax] f32, one scale per
    token for its key and value); vcache [B, Lmax, Hkv, Dv] of the same dtype,
    or None (MLA); kv_begin / kv_end int32 device tensors [B]. Returns
    (o_part, lse_part)."""
    torch = _torch()
    B, Hq = q.shape[0], q.shape[1]
    Dv = vcache.shape[-1] if vcache is not None else 512
    if o_part is None:
        o_part = torch.empty((B, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_size(B, Hq, Dv, max_shard_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    dq, dk = tensor_desc(q), tensor_desc(kcache, kcache_dtype)
    dv = tensor_desc(vcache) if vcache is not None else None
    ds = tensor_desc(kv_scale) if kv_scale is not None else None
    do, dl = tensor_desc(o_part), tensor_desc(lse_part)
    for t in (kv_begin, kv_end):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise TypeError("kv_begin / kv_end must be contiguous int32 tensors on the query's device")
    _check(lib().attn_decode_shard(ctypes.byref(dq), ctypes.byref(dk), _ptr(dv), _ptr(ds),
                                   ctypes.c_void_p(kv_begin.data_ptr()), ctypes.c_void_p(kv_end.data_ptr()),
                                   int(max_shard_len), float(softmax_scale), ctypes.byref(do), ctypes.byref(dl),
                                   ctypes.c_void_p(ws_ptr), ws_bytes, _stream(stream)))
    return o_part, lse_part


def attn_decode_paged_workspace_size(batch, n_heads_q, head_dim_v, max_shard_len, page_size):
    return int(lib().attn_decode_paged_workspace_size(int(batch), int(n_heads_q), int(head_dim_v),
                                                      int(max_shard_len), int(page_size)))


def attn_decode_shard_paged(q, kpool, vpool, block_table, page_size, kv_begin, kv_end, max_shard_len,
                            softmax_scale, kv_scale=None, o_part=None, lse_part=None, workspace=None, stream=None,
                            kpool_dtype=None):
    """Split-KV decode over a paged cache. q [B, Hq, Dqk]; kpool [n_pages *
    page_size, Hkv, Dqk] (torch.uint8 = FP8 E4M3 bytes, then kv_scale [rows]
    f32); vpool the same with Dv, or None (MLA); block_table int32 device
    tensor [B, n_blocks] (logical block -> physical page); kv_begin / kv_end
    int32 device tensors [B] of logical positions. Returns (o_part, lse_part)."""
    torch = _torch()
    B, Hq = q.shape[0], q.shape[1]
    Dv = vpool.shape[-1] if vpool is not None else 512
    if o_part is None:
        o_part = torch.empty((B, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_paged_workspace_size(B, Hq, Dv, max_shard_len, page_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    dq, dk = tensor_desc(q), tensor_desc(kpool, kpool_dtype)
    dv = tensor_desc(vpool) if vpool is not None else None
    ds = tensor_desc(kv_scale) if kv_scale is not None else None
    do, dl = tensor_desc(o_part), tensor_desc(lse_part)
    for t in (kv_begin, kv_end):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise TypeError("kv_begin / kv_end must be contiguous int32 tensors on the query's device")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1 \
            or block_table.device != q.device:
        raise TypeError("block_table must be an int32 [B, n_blocks] tensor (rows contiguous) on the query's device")
    _check(lib().attn_decode_shard_paged(ctypes.byref(dq), ctypes.byref(dk), _ptr(dv), _ptr(ds),
                                         ctypes.c_void_p(block_table.data_ptr()), int(block_table.stride(0)),
                                         int(block_table.shape[1]), int(page_size),
                                         ctypes.c_void_p(kv_begin.data_ptr()), ctypes.c_void_p(kv_end.data_ptr()),
                                         int(max_shard_len), float(softmax_scale), ctypes.byref(do),
                                         ctypes.byref(dl), ctypes.c_void_p(ws_ptr), ws_bytes, _stream(stream)))
    return o_part, lse_part


def attn_decode_shard_noalloc(q, kcache, vcache, kv_begin, kv_end, max_shard_len, softmax_scale, o_part, lse_part,
                              kv_scale=None, stream=None, kcache_dtype=None):
    """attn_decode_shard without a workspace: the split states live in the
    library's per-device scratch array, so the call allocates nothing (the
    caller passes o_part [B, Hq, Dv] and lse_part [B, Hq]). Calls that
    overlap on one GPU race on that array."""
    torch = _torch()
    dq, dk = tensor_desc(q), tensor_desc(kcache, kcache_dtype)
    dv = tensor_desc(vcache) if vcache is not None else None
    ds = tensor_desc(kv_scale) if kv_scale is not None else None
    do, dl = tensor_desc(o_part), tensor_desc(lse_part)
    for t in (kv_begin, kv_end):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise TypeError("kv_begin / kv_end must be contiguous int32 tensors on the query's device")
    _check(lib().attn_decode_shard_noalloc(ctypes.byref(dq), ctypes.byref(dk), _ptr(dv), _ptr(ds),
                                           ctypes.c_void_p(kv_begin.data_ptr()), ctypes.c_void_p(kv_end.data_ptr()),
                                           int(max_shard_len), float(softmax_scale), ctypes.byref(do),
                                           ctypes.byref(dl), _stream(stream)))
    return o_part, lse_part


def attn_decode_shard_mq(q, kcache, vcache, kv_begin, kv_end, max_shard_len, softmax_scale, kv_scale=None,
                         o_part=None, lse_part=None, workspace=None, stream=None, kcache_dtype=None):
    """Multi-query split-KV decode of one shard. q [B, Q, Hq, Dqk]; kv_begin
    int32 [B], kv_end int32 [B * Q] (device); the rest as attn_decode_shard.
    Returns (o_part [B, Q, Hq, Dv], lse_part [B, Q, Hq])."""
    torch = _torch()
    B, Q, Hq = q.shape[0], q.shape[1], q.shape[2]
    Dv = vcache.shape[-1] if vcache is not None else 512
    if o_part is None:
        o_part = torch.empty((B, Q, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Q, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_size(B * Q, Hq, Dv, max_shard_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    dq, dk = tensor_desc(q), tensor_desc(kcache, kcache_dtype)
    dv = tensor_desc(vcache) if vcache is not None else None
    ds = tensor_desc(kv_scale) if kv_scale is not None else None
    do, dl = tensor_desc(o_part), tensor_desc(lse_part)
    for t, n in ((kv_begin, B), (kv_end, B * Q)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise TypeError("kv_begin / kv_end must be contiguous int32 tensors on the query's device")
        if t.numel() != n:
            raise ValueError("kv_begin needs B entries and kv_end B * Q")
    _check(lib().attn_decode_shard_mq(ctypes.byref(dq), ctypes.byref(dk), _ptr(dv), _ptr(ds),
                                      ctypes.c_void_p(kv_begin.data_ptr()), ctypes.c_void_p(kv_end.data_ptr()),
                                      int(max_shard_len), float(softmax_scale), ctypes.byref(do), ctypes.byref(dl),
                                      ctypes.c_void_p(ws_ptr), ws_bytes, _stream(stream)))
    return o_part, lse_part


def attn_sparse_mla_workspace_size(n_queries, k):
    return int(lib().attn_sparse_mla_workspace_size(int(n_queries), int(k)))


def attn_sparse_mla(q, cache, idx, softmax_scale, n_idx=None, req=None, out=None, lse=None, workspace=None,
                    stream=None, kv_scale=None, cache_dtype=None):
    """Sparse MLA attention: query n of q [N, 64, 576] bf16 attends the rows
    idx[n, :n_idx[n]] of request req[n] of cache [B, Lmax, 1, 576] (bf16, or
    torch.uint8 FP8 E4M3 bytes with kv_scale [B, Lmax] f32). idx: int32
    device tensor [N, k] (last dim contiguous); n_idx / req: int32 device
    tensors [N] or None. Returns (out [N, 64, 512] f32, lse [N, 64] f32)."""
    torch = _torch()
    N = q.shape[0]
    if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != N or (idx.shape[1] > 1 and idx.stride(1) != 1):
        raise TypeError("idx must be an int32 tensor [N, k] with a contiguous last dim")
    for t in (n_idx, req):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != N):
            raise TypeError("n_idx / req must be contiguous int32 tensors [N]")
    k = idx.shape[1]
    if out is None:
        out = torch.empty((N, 64, 512), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((N, 64), dtype=torch.float32, device=q.device)
    need = attn_sparse_mla_workspace_size(N, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    dq, dc, do, dl = tensor_desc(q), tensor_desc(cache, cache_dtype), tensor_desc(out), tensor_desc(lse)
    ds = tensor_desc(kv_scale) if kv_scale is not None else None
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None
    _check(lib().attn_sparse_mla(ctypes.byref(dq), ctypes.byref(dc), _ptr(ds), ptr(req), ptr(idx),
                                 int(idx.stride(0)) if N > 0 else int(k), int(k), ptr(n_idx), float(softmax_scale),
                                 ctypes.byref(do), ctypes.byref(dl), ctypes.c_void_p(ws_ptr), ws_bytes,
                                 _stream(stream)))
    return out, lse


def _dptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def attn_topk_local(scores, k, id_base, id_stride, n_valid=None, stream=None):
    """Local top-k of each row of scores [N, L] f32 (device, last dim
    contiguous): entry j has global id id_base + j * id_stride. Returns
    (score [N, k] f32, id [N, k] int32, row [N, k] int32, count [N] int32)."""
    torch = _torch()
    N, L = scores.shape
    if scores.dtype != torch.float32 or (L > 1 and scores.stride(1) != 1):
        raise TypeError("scores must be float32 [N, L] with a contiguous last dim")
    if n_valid is not None and (n_valid.dtype != torch.int32 or not n_valid.is_contiguous() or n_valid.numel() != N):
        raise TypeError("n_valid must be a contiguous int32 tensor [N]")
    dev = scores.device
    kk = max(int(k), 0)  # a negative k reaches the library, which rejects it
    osc = torch.empty((N, kk), dtype=torch.float32, device=dev)
    oid = torch.empty((N, kk), dtype=torch.int32, device=dev)
    orow = torch.empty((N, kk), dtype=torch.int32, device=dev)
    cnt = torch.empty((N,), dtype=torch.int32, device=dev)
    _check(lib().attn_topk_local(_dptr(scores), int(scores.stride(0)) if N > 0 else int(L), int(N), int(L),
                                 _dptr(n_valid), int(k), int(id_base), int(id_stride), _dptr(osc), _dptr(oid),
                                 _dptr(orow), _dptr(cnt), _stream(stream)))
    return osc, oid, orow, cnt


def attn_topk_merge(cand_score, cand_id, cand_row, k, cand_count=None, stream=None):
    """Exact global top k of P ranks' lists: cand_* [P, N, k_in] (f32 /
    int32 / int32, contiguous), cand_count [P, N] int32 or None. Returns
    (out_id [N, k], owner_row [P, N, k], owner_count [P, N]) int32."""
    torch = _torch()
    P, N, k_in = cand_score.shape
    for t, dt in ((cand_score, torch.float32), (cand_id, torch.int32), (cand_row, torch.int32)):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != (P, N, k_in):
            raise TypeError("cand_score / cand_id / cand_row must be contiguous [P, N, k_in] f32 / int32 / int32")
    if cand_count is not None and (cand_count.dtype != torch.int32 or not cand_count.is_contiguous()
                                   or tuple(cand_count.shape) != (P, N)):
        raise TypeError("cand_count must be a contiguous int32 tensor [P, N]")
    dev = cand_score.device
    kk = max(int(k), 0)
    oid = torch.empty((N, kk), dtype=torch.int32, device=dev)
    orow = torch.empty((P, N, kk), dtype=torch.int32, device=dev)
    ocnt = torch.empty((P, N), dtype=torch.int32, device=dev)
    _check(lib().attn_topk_merge(int(P), int(N), int(k_in), _dptr(cand_score), _dptr(cand_id), _dptr(cand_row),
                                 _dptr(cand_count), int(k), _dptr(oid), _dptr(orow), _dptr(ocnt), _stream(stream)))
    return oid, orow, ocnt


def attn_merge_states(o_parts, lse_parts, out=None, lse_out=None, out_dtype=None, stream=None):
    """Exact LSE merge: o_parts [S, N, H, Dv] f32, lse_parts [S, N, H] f32.
    Returns (out [N, H, Dv], lse_out [N, H])."""
    torch = _torch()
    S, N, H, Dv = o_parts.shape
    if out is None:
        out = torch.empty((N, H, Dv), dtype=out_dtype or torch.float32, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty((N, H), dtype=torch.float32, device=o_parts.device)
    do, dl, dout, dlo = tensor_desc(o_parts), tensor_desc(lse_parts), tensor_desc(out), tensor_desc(lse_out)
    _check(lib().attn_merge_states(S, ctypes.byref(do), ctypes.byref(dl), ctypes.byref(dout), ctypes.byref(dlo),
                                   _stream(stream)))
    return out, lse_out


def attn_cache_write_round_robin(C, rank, src, slot, req, dst, n_repl=0, stream=None, dtype=None):
    """Write rows of src [n, W] into rank `rank`'s round-robin local cache
    dst [B, Lmax_local, W] (row n_repl + slot // C of request req) where
    slot % C == rank. slot: int64 device tensor [n]; req: int32 device [n].
    dtype overrides the cpa dtype (raw FP8 bytes as torch.uint8)."""
    torch = _torch()
    if slot.dtype != torch.int64 or req.dtype != torch.int32 or not slot.is_contiguous() or not req.is_contiguous():
        raise TypeError("slot must be a contiguous int64 tensor and req a contiguous int32 tensor")
    if slot.numel() != src.shape[0] or req.numel() != src.shape[0]:
        raise ValueError("slot and req need one entry per source row")
    ds, dd = tensor_desc(src, dtype), tensor_desc(dst, dtype)
    _check(lib().attn_cache_write_round_robin(int(C), int(rank), int(n_repl), ctypes.byref(ds),
                                              ctypes.c_void_p(slot.data_ptr()), ctypes.c_void_p(req.data_ptr()),
                                              ctypes.byref(dd), _stream(stream)))
    return dst
