"""Attention over a rank's shard and the exact partial-softmax merge (oracle).

Float64 throughout. Inputs are float64 arrays (or any array plus a ``decode``
callable that turns a slice of stored bits into float64, see ``formats``).

Definitions written out here:

* Causal attention -- *Long Context* 1.1: a token's output compares its query
  with the keys of all tokens up to and including it, turns the scores into
  probabilities with a softmax and sums the values with those weights.
  Scores are ``scale * q . k``; the softmax scale is an explicit argument.
* Log-sum-exp -- *Long Context* 3.3: besides its output each shard reports
  the natural log of its sum of exponentiated scores, ``lse = log sum_t
  exp(s_t)``. Written with the usual max shift ``m + log sum exp(s - m)``,
  which is the same number. An empty key set has output 0 and lse = -inf.
* GQA -- vLLM DCP post, 5.4: kv heads are broadcast to groups of query heads;
  reading taken: query head h uses kv head ``h // (Hq / Hkv)``.
* MLA -- *Long Context* 1.3 and vLLM DCP post, 5.3: one latent vector per
  token is read by all heads; the vLLM GLM-5.3 post, footnote 1, counts QK
  over 576 dims and PV over 512. Reading taken: keys are the 576-dim latent
  and values are its first 512 dims (``v=None, dv=512``).
* Merge -- *Long Context* 3.3: ``lse = logsumexp_c lse_c``,
  ``scale_c = exp(lse_c - lse)``, ``O = sum_c scale_c * O_c``; exact apart
  from the order of additions (3.3; DeepSeek-V4 notes, section 5).
* Paged cache -- DeepSeek-V4 notes, 1 and 9.1: a request's cache is read
  through a block table of fixed-size logical blocks mapped to physical pages
  (``paged_rows``, ``decode_shard_paged``).
* Merge in statistics form -- DeepSeek-V4 notes, section 5: per shard
  ``m_p = max s``, ``l_p = sum exp(s - m_p)``, ``u_p = sum exp(s - m_p) v``;
  globally ``m = max m_p``, ``Z = sum e^(m_p - m) l_p``,
  ``o = sum e^(m_p - m) u_p / Z``.

Rows are independent; ``prefill_shard`` computes several rows with one
matrix product only to keep numpy fast, with the causal limit of each row
applied as an explicit mask. Nothing is tiled over keys and there is no
running (online) softmax here.

Pins (``tests/test_oracle_attention.py``): the two-GPU example of
*Long Context* 3.2/3.3 (exp-scores 4, 2, 1, 1) to exact rationals; torch's
float64 ``scaled_dot_product_attention(is_causal=True)`` for C = 1; union of
all ranks' outputs equals unsharded attention; merged split-KV equals
unsharded attention; single-key and equal-score closed forms; the two merge
forms agree. Paged decode (``tests/test_oracle_paged.py``): a hand-written
row mapping; shuffled pages equal the contiguous cache (GQA, MLA FP8 with
per-row scales); unreferenced pages unread; shared prefix pages; invalid
entries read page 0; page size 1 and one page per request.
"""

import numpy as np

_NEG_INF = -np.inf


def _f64(x, decode=None):
    return decode(x) if decode is not None else np.asarray(x, dtype=np.float64)


def attend(q, keys, values, scale):
    """One query against a key set. q [D], keys [n, D], values [n, Dv].
    Returns (o [Dv], lse)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1]), _NEG_INF
    s = scale * (keys @ q)
    m = np.max(s)
    e = np.exp(s - m)
    ell = np.sum(e)
    return (e @ values) / ell, m + np.log(ell)


def _group(Hq, Hkv):
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq // Hkv


def prefill_shard(q, k, segments, scale, v=None, dv=None, rows=None, decode=None,
                  max_elems=1 << 25):
    """Causal attention for a rank's local query rows against their true
    causal history (cached prefix included).

    q        [n_local, Hq, Dqk]   local queries in plan order
    k        [T_kv, Hkv, Dqk]     packed full keys, request j at rows kv_row0_j ..
    v        [T_kv, Hkv, Dv]      packed values, or None for MLA (v = k[..., :dv])
    segments list of (req, q_row0, q_len, pos0, pos_stride, kv_row0)
    rows     optional list of local rows to compute (others are not computed)

    Returns (O, LSE): O [len(rows), Hq, Dv], LSE [len(rows), Hq] in the order
    of ``rows`` (all local rows, ascending, when rows is None).
    """
    n_local, Hq, Dqk = q.shape
    Hkv = k.shape[1]
    G = _group(Hq, Hkv)
    if v is None:
        if dv is None:
            raise ValueError("MLA needs dv")
        Dv = dv
    else:
        Dv = v.shape[-1]
    # local row -> (kv_row0, position)
    where = {}
    for (_req, r0, n, pos0, stride, kv0) in segments:
        for i in range(n):
            where[r0 + i] = (kv0, pos0 + i * stride)
    if rows is None:
        rows = sorted(where)
    rows = list(rows)
    O = np.full((len(rows), Hq, Dv), np.nan)
    L = np.full((len(rows), Hq), np.nan)
    # batch rows that share a request (same kv_row0) to use matrix products
    by_req = {}
    for out_i, r in enumerate(rows):
        kv0, p = where[r]
        by_req.setdefault(kv0, []).append((out_i, r, p))
    for kv0, items in by_req.items():
        items.sort(key=lambda t: t[2])
        pmax = items[-1][2]
        chunk = max(1, max_elems // max(1, Hq * (pmax + 1)))
        for c0 in range(0, len(items), chunk):
            part = items[c0:c0 + chunk]
            p_hi = part[-1][2]
            keys = _f64(k[kv0:kv0 + p_hi + 1], decode)  # [n_keys, Hkv, Dqk]
            vals = keys[..., :Dv] if v is None else _f64(v[kv0:kv0 + p_hi + 1], decode)
            qr = _f64(q[[t[1] for t in part]], decode)  # [R, Hq, Dqk]
            pos = np.array([t[2] for t in part])
            # key index t is visible to a row at position p iff t <= p
            visible = np.arange(p_hi + 1)[None, :] <= pos[:, None]  # [R, n_keys]
            for hk in range(Hkv):
                R = len(part)
                qh = qr[:, hk * G:(hk + 1) * G, :].reshape(R * G, Dqk)
                kh = np.ascontiguousarray(keys[:, hk, :])  # [n_keys, D]
                s = (scale * (qh @ kh.T)).reshape(R, G, p_hi + 1)
                s = np.where(visible[:, None, :], s, _NEG_INF)
                m = np.max(s, axis=-1, keepdims=True)
                e = np.exp(s - m)
                ell = np.sum(e, axis=-1, keepdims=True)
                vh = np.ascontiguousarray(vals[:, hk, :])
                o = (e.reshape(R * G, p_hi + 1) @ vh).reshape(R, G, Dv) / ell
                lse = (m + np.log(ell))[..., 0]
                for j, t in enumerate(part):
                    O[t[0], hk * G:(hk + 1) * G] = o[j]
                    L[t[0], hk * G:(hk + 1) * G] = lse[j]
    return O, L


def decode_shard(q, kcache, begin, end, scale, vcache=None, dv=None, decode=None,
                 kv_scale=None, batch=None):
    """Split-KV decode on one shard: for request b and query head h, attention
    of the single query q[b, h] over cache rows [begin_b, end_b).

    q       [B, Hq, Dqk]
    kcache  [B, Lmax, Hkv, Dqk]   (decode turns a slice into float64 values,
                                   e.g. fp8 codes times the per-token scale)
    vcache  [B, Lmax, Hkv, Dv] or None for MLA (v = k[..., :dv])
    kv_scale [B, Lmax] per-token scale or None: every entry of token t's
            cache row -- its key and, for a GQA cache, its value -- is
            decode(code) * kv_scale[b, t] (FP8 cache)
    Returns O [B, Hq, Dv] (0 for an empty range), LSE [B, Hq] (-inf if empty).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Dqk = q.shape
    Hkv = kcache.shape[2]
    G = _group(Hq, Hkv)
    Dv = dv if vcache is None else vcache.shape[-1]
    O = np.zeros((B, Hq, Dv))
    L = np.full((B, Hq), _NEG_INF)
    for b in (range(B) if batch is None else batch):
        s0, s1 = int(begin[b]), int(end[b])
        if s1 <= s0:
            continue
        keys = _f64(kcache[b, s0:s1], decode)  # [n, Hkv, Dqk]
        vals = keys[..., :Dv] if vcache is None else _f64(vcache[b, s0:s1], decode)
        if kv_scale is not None:
            tok_scale = np.asarray(kv_scale[b, s0:s1], np.float32).astype(np.float64)[:, None, None]
            keys = keys * tok_scale
            vals = vals * tok_scale
        for h in range(Hq):
            o, lse = attend(q[b, h], keys[:, h // G, :], vals[:, h // G, :], scale)
            O[b, h] = o
            L[b, h] = lse
    return O, L


def paged_rows(block_table, page_size, n_pages, positions):
    """Pool rows of a request's logical cache positions under a page table.

    DeepSeek-V4 notes, 1 (vLLM maps fixed-size logical blocks of a request's
    cache into physical pages) and 9.1 (decode keeps the cache paged and reads
    it through the table). Reading taken: logical position t lies in logical
    block t // page_size at offset t % page_size; the block's table entry names
    the physical page, and the row is page * page_size + offset. A table entry
    outside [0, n_pages) is read as page 0 (the library's contract for an
    invalid entry: an in-bounds read, not a fault; the pages say nothing).
    """
    t = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(block_table, dtype=np.int64)[t // page_size]
    pages = np.where((pages >= 0) & (pages < n_pages), pages, 0)
    return pages * page_size + t % page_size


def decode_shard_paged(q, kpool, block_table, page_size, begin, end, scale, vpool=None, dv=None,
                       decode=None, kv_scale=None, batch=None):
    """Split-KV decode over a paged cache: ``decode_shard`` of each request on
    the pool rows its block table names (``paged_rows``).

    q           [B, Hq, Dqk]
    kpool       [n_pages * page_size, Hkv, Dqk]   rows of all pages
    vpool       same shape with Dv, or None for MLA (v = k[..., :dv])
    kv_scale    [n_pages * page_size] per-row scale, or None
    block_table [B, n_blocks]: logical block j of request b -> physical page
    begin, end  [B] logical positions, end <= n_blocks * page_size
    Returns O [B, Hq, Dv], LSE [B, Hq] as ``decode_shard``.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    n_pages = kpool.shape[0] // page_size
    Dv = dv if vpool is None else vpool.shape[-1]
    O = np.zeros((B, Hq, Dv))
    L = np.full((B, Hq), _NEG_INF)
    for b in (range(B) if batch is None else batch):
        s0, s1 = int(begin[b]), int(end[b])
        if s1 <= s0:
            continue
        rows = paged_rows(block_table[b], page_size, n_pages, np.arange(s0, s1))
        kc = kpool[rows][None]
        vc = None if vpool is None else vpool[rows][None]
        sc = None if kv_scale is None else np.asarray(kv_scale)[rows][None]
        o, lse = decode_shard(q[b:b + 1], kc, [0], [s1 - s0], scale, vcache=vc, dv=dv, decode=decode, kv_scale=sc)
        O[b], L[b] = o[0], lse[0]
    return O, L


def decode_shard_mq(q, kcache, begin, end, scale, vcache=None, dv=None, decode=None,
                    kv_scale=None, batch=None):
    """Multi-query decode on one shard: request b has Q query rows, and row k
    attends cache rows [begin_b, end[b*Q + k]) exactly as decode_shard
    attends a single query (the causal ends come from plan_multi_query).

    q [B, Q, Hq, Dqk]; begin [B]; end [B * Q]; the rest as decode_shard.
    Returns O [B, Q, Hq, Dv], LSE [B, Q, Hq]."""
    q = np.asarray(q, dtype=np.float64)
    B, Q = q.shape[:2]
    end = np.asarray(end).reshape(B, Q)
    outs = [decode_shard(q[:, k], kcache, begin, end[:, k], scale, vcache=vcache, dv=dv, decode=decode,
                         kv_scale=kv_scale, batch=batch) for k in range(Q)]
    return np.stack([o for o, _ in outs], axis=1), np.stack([l for _, l in outs], axis=1)


def sparse_mla(q, cache, idx, scale, n_idx=None, req=None, dv=512, decode=None, kv_scale=None, rows=None):
    """Sparse (top-k index list) MLA attention: query n attends only the
    cache rows its list names -- *Long Context* 2.4: every query of a sparse
    attention model comes with its own list of selected tokens; vLLM GLM-5.3
    post, footnote 1: each query reads its 2,048 selected latent rows (QK over
    576 dims, PV over 512) for all heads.

    q      [N, H, 576]
    cache  [B, Lmax, 1, 576] (decode turns stored bits into float64;
           kv_scale [B, Lmax] multiplies FP8 entries, as in decode_shard)
    idx    [N, K] integer rows of request req[n]'s cache (req=None: n)
    n_idx  [N] or None: only the first n_idx[n] entries of row n count
    Reading taken where the pages are silent: an entry outside [0, Lmax) is
    no selection (padding) and is skipped, and so is every entry of a query
    whose request is outside [0, B); an entry listed twice counts twice (a
    top-k list has none). Returns O [N, H, dv], LSE [N, H]."""
    q = np.asarray(q, dtype=np.float64)
    N, Hq, _ = q.shape
    Lmax = cache.shape[1]
    idx = np.asarray(idx)
    O = np.zeros((N, Hq, dv))
    L = np.full((N, Hq), _NEG_INF)
    for n in (range(N) if rows is None else rows):
        b = n if req is None else int(req[n])
        k = idx.shape[1] if n_idx is None else max(0, min(int(n_idx[n]), idx.shape[1]))
        sel = [int(t) for t in idx[n, :k] if 0 <= int(t) < Lmax] if 0 <= b < cache.shape[0] else []
        if not sel:
            continue
        keys = _f64(cache[b, sel], decode)[:, 0, :]           # [n_sel, 576]
        if kv_scale is not None:
            keys = keys * np.asarray(kv_scale[b, sel], np.float32).astype(np.float64)[:, None]
        for h in range(Hq):
            O[n, h], L[n, h] = attend(q[n, h], keys, keys[:, :dv], scale)
    return O, L


def sparse_mla_cost(k_rows, heads, row_bytes, q_out_bytes_per_head=2176, flops_per_row_head=2176):
    """Per-query work of sparse MLA attention as the vLLM GLM-5.3 post,
    footnote 1, counts it: k_rows selected rows of row_bytes each (cache entry
    plus its index), q_out_bytes_per_head of BF16 query and output per head,
    flops_per_row_head FLOPs per row and head. Returns (flops, bytes)."""
    flops = k_rows * heads * flops_per_row_head
    nbytes = k_rows * row_bytes + heads * q_out_bytes_per_head
    return flops, nbytes


def merge_states(o_parts, lse_parts):
    """Exact LSE merge of S partial states. o_parts [S, ..., Dv],
    lse_parts [S, ...]. A state with lse = -inf carries no mass; if every
    state is empty the result is O = 0, lse = -inf."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    tot = np.sum(np.exp(lse_parts - m_safe), axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(np.isfinite(m), m_safe + np.log(tot), _NEG_INF)
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    w = np.where(np.isfinite(lse)[None], np.exp(lse_parts - lse_safe[None]), 0.0)
    out = np.sum(w[..., None] * o_parts, axis=0)
    return out, lse


def shard_stats(q, keys, values, scale):
    """Per-shard statistics of the DeepSeek-V4 notes, section 5:
    (m_p, l_p, u_p) for one query over one shard's key set."""
    s = scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))
    m = np.max(s)
    e = np.exp(s - m)
    return m, np.sum(e), e @ np.asarray(values, np.float64)


def merge_stats(ms, ls, us):
    """Global combine of the DeepSeek-V4 notes, section 5: returns (o, Z, m)."""
    ms = np.asarray(ms, np.float64)
    m = np.max(ms)
    w = np.exp(ms - m)
    Z = np.sum(w * np.asarray(ls, np.float64))
    o = np.sum(w[:, None] * np.asarray(us, np.float64), axis=0) / Z
    return o, Z, m
