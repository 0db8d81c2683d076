"""Seeded synthetic inputs for the attention shards.

This module is shared by both sides of every parity check (the float64 oracle
and the HIP path) and by the benchmark. It holds none of the method's
arithmetic: it only draws random numbers and rounds them into the formats the
attention path stores (bf16 words, OCP FP8 E4M3 bytes with a per-token fp32
scale). Both sides then decode the same stored bits themselves.

Seeding: a tensor of stream s of seed family k (each workload has its own,
``WORKLOADS[name]["seed"]``) is drawn slab by slab along its first axis;
slab i of ``chunk`` rows comes from ``numpy.random.default_rng([k, s, i])``. The result therefore does not
depend on how many threads draw it. Streams: 0 request lengths, 1 queries,
2 keys / latent cache, 3 values, 4 multi-query decode queries, 5 sparse
queries, 6 and 7 top-k index lists, 8 index scores, 9 sampled rows.

Workload shapes follow the pages' workloads: a GLM-5.3-like 128k-token MLA
context with 64 heads and a 576-dim latent (QK over 576, PV over 512), a
32/8-head GQA model with head dim 128, and an agentic request-length mix that
is bimodal around a ~67k median (about half above 64k with a tail, the rest
short to mid).
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3_MAX = 448.0


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(family, stream, chunk=None):
    key = [int(family), int(stream)] if chunk is None else [int(family), int(stream), int(chunk)]
    return np.random.default_rng(key)


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (round to nearest, ties to even) -> uint16 words."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = np.right_shift(u, 16)
    np.bitwise_and(r, 1, out=r)
    np.add(r, 0x7FFF, out=r)
    np.add(r, u, out=r)
    np.right_shift(r, 16, out=r)
    return r.astype(np.uint16)


def f32_to_e4m3(x):
    """Per-token FP8 quantisation of the last axis: scale = amax / 448 (1 if the
    row is all zero), codes = RNE(x / scale) saturated to +-448, as OCP E4M3FN
    bytes. Returns (codes uint8 [..., D], scale float32 [...])."""
    import torch  # rounding to E4M3 via torch's float8_e4m3fn cast

    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def gqa_kv_to_e4m3(k, v):
    """FP8 form of a GQA cache with one scale per token: the scale covers the
    token's key and value rows over all kv heads (amax / 448), the codes are
    E4M3 bytes. k, v [B, L, Hkv, D] float32 -> (k codes, v codes uint8
    [B, L, Hkv, D], scale float32 [B, L])."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    B, L, Hkv, D = k.shape
    n = Hkv * D
    codes, scale = f32_to_e4m3(np.concatenate([k.reshape(B, L, n), v.reshape(B, L, n)], axis=-1))
    return codes[..., :n].reshape(B, L, Hkv, D), codes[..., n:].reshape(B, L, Hkv, D), scale


def _slabs(n, chunk):
    return [(i, i * chunk, min(n, (i + 1) * chunk)) for i in range(-(-n // chunk))]


def normal(family, stream, shape, std=1.0, chunk=4096, out_fn=None, out_dtype=None):
    """Draw N(0, std^2) float32 of ``shape`` slab by slab and pass each slab
    through ``out_fn`` (e.g. bf16 rounding) into an array of ``out_dtype``."""
    shape = tuple(int(s) for s in shape)
    n0 = shape[0]
    rest = shape[1:]
    out = np.empty(shape, dtype=out_dtype or np.float32)

    def work(sl):
        i, a, b = sl
        g = rng(family, stream, i)
        x = g.standard_normal((b - a,) + rest, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[a:b] = out_fn(x) if out_fn is not None else x

    slabs = _slabs(n0, chunk)
    if len(slabs) == 1:
        work(slabs[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, slabs))
    return out


def bf16_normal_slabs(family, stream, shape, slabs, std=1.0, chunk=4096, out=None):
    """Only the slabs ``slabs`` (``chunk`` rows each along the first axis) of
    bf16_normal(family, stream, shape, std, chunk), drawn alone into ``out``
    (a lazily allocated uint16 array of ``shape`` if None, other rows left
    unset). The rows are identical to those of the full draw."""
    shape = tuple(int(s) for s in shape)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    for i in sorted(set(int(x) for x in slabs)):
        a, b = i * chunk, min(shape[0], (i + 1) * chunk)
        x = rng(family, stream, i).standard_normal((b - a,) + shape[1:], dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[a:b] = f32_to_bf16_bits(x)
    return out


def bf16_normal(family, stream, shape, std=1.0, chunk=4096):
    """N(0, std^2) rounded to bf16; returns uint16 words."""
    return normal(family, stream, shape, std, chunk, f32_to_bf16_bits, np.uint16)


def f32_normal(family, stream, shape, std=1.0, chunk=4096):
    return normal(family, stream, shape, std, chunk)


def latent_cache(family, stream, B, L, D, std, chunk=8192, fp8=False):
    """A [B, L, 1, D] latent cache drawn N(0, std^2) per request slab.
    Returns bf16 words, or (E4M3 codes, per-token scale [B, L]) when fp8."""
    codes = np.empty((B, L, 1, D), dtype=np.uint8 if fp8 else np.uint16)
    scales = np.empty((B, L), dtype=np.float32) if fp8 else None
    jobs = [(b, i, a, e) for b in range(B) for (i, a, e) in _slabs(L, chunk)]

    def work(job):
        b, i, a, e = job
        g = rng(family, stream, b * 100000 + i)
        x = g.standard_normal((e - a, D), dtype=np.float32)
        x *= np.float32(std)
        if fp8:
            c, s = f32_to_e4m3(x)
            codes[b, a:e, 0] = c
            scales[b, a:e] = s
        else:
            codes[b, a:e, 0] = f32_to_bf16_bits(x)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    return (codes, scales) if fp8 else codes


def latent_cache_both(family, stream, B, L, D, std, chunk=8192):
    """One draw of a [B, L, 1, D] latent cache, stored both as bf16 words and
    as E4M3 codes with per-token scales: (bf16, codes, scales [B, L])."""
    bits = np.empty((B, L, 1, D), dtype=np.uint16)
    codes = np.empty((B, L, 1, D), dtype=np.uint8)
    scales = np.empty((B, L), dtype=np.float32)
    jobs = [(b, i, a, e) for b in range(B) for (i, a, e) in _slabs(L, chunk)]

    def work(job):
        b, i, a, e = job
        g = rng(family, stream, b * 100000 + i)
        x = g.standard_normal((e - a, D), dtype=np.float32)
        x *= np.float32(std)
        bits[b, a:e, 0] = f32_to_bf16_bits(x)
        c, s = f32_to_e4m3(x)
        codes[b, a:e, 0] = c
        scales[b, a:e] = s

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    return bits, codes, scales


# ---------------------------------------------------------------- workloads

AGENTIC_MEDIAN = 67 * 1024  # "median of ~67k tokens"; k = 1024
AGENTIC_CAP = 256 * 1024
AGENTIC_SIGMA = 0.65


def agentic_lengths(family=5, n=16):
    """Request lengths for the ragged interleave workload: half lognormal
    around a 67k median (capped at 256k), half uniform in [1k, 64k], shuffled.
    Drawn from default_rng([family, 0])."""
    g = rng(family, 0)
    half = n // 2
    ln = np.rint(g.lognormal(mean=math.log(AGENTIC_MEDIAN), sigma=AGENTIC_SIGMA, size=half))
    ln = np.clip(ln, 1, AGENTIC_CAP).astype(np.int64)
    un = g.integers(1024, 64 * 1024, size=n - half, endpoint=True).astype(np.int64)
    allv = np.concatenate([ln, un])
    return allv[g.permutation(n)].astype(np.int32)


def topk_lists(family, stream, n, L, k, limit=None):
    """Synthetic top-k selections: row i lists min(k, limit_i) distinct cache
    rows drawn uniformly from [0, limit_i) (limit_i = L, or limit[i] for a
    causal query that sees only rows below it), in random order, padded with
    -1. Row i comes from default_rng([family, stream, i]). Returns (idx int32
    [n, k], count int32 [n])."""
    idx = np.full((n, k), -1, np.int32)
    cnt = np.zeros(n, np.int32)
    for i in range(n):
        lim = int(L if limit is None else limit[i])
        g = rng(family, stream, i)
        m = min(k, lim)
        if m == lim:
            sel = g.permutation(lim)
        else:
            sel = g.choice(lim, m, replace=False)
        idx[i, :m] = sel
        cnt[i] = m
    return idx, cnt


# The workloads, by name: sizes, dtypes and scale; "seed" is the family id
# their inputs draw from (the first argument of the generators above).
WORKLOADS = {
    "gqa_decode_f32_4k": dict(
        seed=1, name="split-KV decode + LSE merge, fp32, GQA 8/1 d128, KV 4096, C=4",
        kind="decode", B=1, Hq=8, Hkv=1, Dqk=128, Dv=128, L=4096, C=4, dtype="f32",
        scale=1.0 / math.sqrt(128)),
    "gqa_zigzag_prefill_16k": dict(
        seed=2, name="zigzag prefill shard, GQA 32/8 d128 bf16, 16384-token prompt, C=4 rank 1",
        kind="prefill", strategy="zigzag", Hq=32, Hkv=8, Dqk=128, Dv=128,
        new_len=[16384], prefix_len=[0], C=4, rank=1, dtype="bf16",
        scale=1.0 / math.sqrt(128)),
    "mla_decode_131k": dict(
        seed=3, name="MLA decode over token-sharded latent cache, B64 H64 576/512, 131072 ctx, C=8",
        kind="decode_mla", B=64, Hq=64, Hkv=1, Dqk=576, Dv=512, L=131072, C=8,
        std=0.5, scale=1.0 / math.sqrt(576)),
    "mla_zigzag_prefill_prefix32k": dict(
        seed=4, name="MLA zigzag prefill, H64 576/512, 131072 new after 32768 prefix, C=8 rank 0",
        kind="prefill", strategy="zigzag", Hq=64, Hkv=1, Dqk=576, Dv=512,
        new_len=[131072], prefix_len=[32768], C=8, rank=0, dtype="bf16",
        scale=1.0 / math.sqrt(576)),
    "gqa_interleave_prefill_agentic16": dict(
        seed=5, name="interleave prefill, 16 agentic requests, GQA 32/8 d128 bf16, C=4 rank 2",
        kind="prefill", strategy="interleave", Hq=32, Hkv=8, Dqk=128, Dv=128,
        new_len=None, prefix_len=None, C=4, rank=2, dtype="bf16",
        scale=1.0 / math.sqrt(128)),
}


def workload(name):
    c = dict(WORKLOADS[name])
    if c["kind"] == "prefill" and c["new_len"] is None:  # the ragged agentic batch
        c["new_len"] = [int(x) for x in agentic_lengths(c["seed"], 16)]
        c["prefix_len"] = [0] * 16
    return c


def page_table(family, stream, B, n_blocks, n_pages, shared=0):
    """Seeded block table [B, n_blocks] int32 of distinct physical page ids
    drawn from range(n_pages) (a random permutation), except that the first
    `shared` logical blocks of every request name the same pages as request
    0's (a shared prefix). Needs n_pages >= shared + B * (n_blocks - shared)."""
    need = shared + B * (n_blocks - shared)
    assert n_pages >= need
    perm = rng(family, stream).permutation(n_pages)[:need].astype(np.int32)
    table = np.empty((B, n_blocks), np.int32)
    table[:, :shared] = perm[:shared]
    table[:, shared:] = perm[shared:].reshape(B, n_blocks - shared)
    return table
