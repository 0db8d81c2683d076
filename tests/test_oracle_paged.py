"""Pins of the paged-cache decode in the oracle (CPU only).

``oracle.attention.paged_rows`` / ``decode_shard_paged`` read a request's
cache through its block table (DeepSeek-V4 notes, 1 and 9.1: logical blocks
of fixed size mapped to physical pages). Pinned to: a worked example of the
row mapping written out by hand; decode over pages holding a contiguous cache
in shuffled order equals decode over that contiguous cache (bf16-valued and
FP8 with per-row scales); pages no table names are never read (NaN there
changes nothing); requests sharing prefix pages equal contiguous caches with
equal prefixes; an entry outside the pool reads page 0; page size 1 and one
page per request.
"""

import numpy as np

from oracle import attention as att
from oracle import formats
import synth


def test_rows_worked_example():
    # page size 4, logical blocks 0, 1, 2 in physical pages 2, 0, 5
    rows = att.paged_rows([2, 0, 5], 4, 6, np.arange(12))
    assert rows.tolist() == [8, 9, 10, 11, 0, 1, 2, 3, 20, 21, 22, 23]
    # a range that starts inside a block
    assert att.paged_rows([2, 0, 5], 4, 6, np.arange(3, 7)).tolist() == [11, 0, 1, 2]


def _scatter(cache, table, page_size, n_pages):
    """Pool holding logical block j of request b in page table[b, j]."""
    B, L = cache.shape[:2]
    nb = L // page_size
    pool = np.full((n_pages, page_size) + cache.shape[2:], np.nan)
    blocks = cache.reshape((B, nb, page_size) + cache.shape[2:])
    for b in range(B):
        for j in range(nb):
            pool[table[b, j]] = blocks[b, j]
    return pool.reshape((n_pages * page_size,) + cache.shape[2:])


def test_shuffled_pages_equal_contiguous_gqa():
    rng = np.random.default_rng(3)
    B, L, Hq, Hkv, D, ps = 3, 48, 4, 2, 8, 8
    k = rng.standard_normal((B, L, Hkv, D))
    v = rng.standard_normal((B, L, Hkv, D))
    q = rng.standard_normal((B, Hq, D))
    table = synth.page_table(11, 0, B, L // ps, 40)
    kp, vp = _scatter(k, table, ps, 40), _scatter(v, table, ps, 40)
    beg, end = [0, 5, 17], [48, 30, 18]
    O, LSE = att.decode_shard_paged(q, kp, table, ps, beg, end, 0.3, vpool=vp)
    O2, L2 = att.decode_shard(q, k, beg, end, 0.3, vcache=v)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, L2)


def test_shuffled_pages_equal_contiguous_mla_fp8():
    rng = np.random.default_rng(4)
    B, L, H, D, dv, ps = 2, 64, 3, 24, 16, 16
    x = rng.standard_normal((B, L, 1, D)).astype(np.float32)
    codes, scale = synth.f32_to_e4m3(x)  # scale [B, L, 1]
    q = rng.standard_normal((B, H, D))
    table = synth.page_table(11, 1, B, L // ps, 9)
    cp = _scatter(codes.astype(np.float64), table, ps, 9)
    cp = np.nan_to_num(cp).astype(np.uint8)  # unused pages: code 0
    sp = _scatter(scale[..., 0].astype(np.float64)[..., None], table, ps, 9)[..., 0]
    sp = np.nan_to_num(sp, nan=1.0).astype(np.float32)
    beg, end = [3, 0], [64, 41]
    O, LSE = att.decode_shard_paged(q, cp, table, ps, beg, end, 0.2, dv=dv, decode=formats.e4m3_to_f64,
                                    kv_scale=sp)
    O2, L2 = att.decode_shard(q, codes, beg, end, 0.2, dv=dv, decode=formats.e4m3_to_f64,
                              kv_scale=scale[..., 0])
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, L2)


def test_unreferenced_pages_are_not_read():
    rng = np.random.default_rng(5)
    B, L, H, D, ps = 2, 32, 2, 8, 8
    k = rng.standard_normal((B, L, 1, D))
    q = rng.standard_normal((B, H, D))
    table = synth.page_table(11, 2, B, L // ps, 20)
    kp = _scatter(k, table, ps, 20)  # 12 of 20 pages stay NaN
    assert np.isnan(kp).any()
    O, LSE = att.decode_shard_paged(q, kp, table, ps, [0, 9], [32, 25], 0.5, dv=4)
    assert np.isfinite(O).all() and np.isfinite(LSE).all()


def test_shared_prefix_pages():
    rng = np.random.default_rng(6)
    B, L, H, D, ps, shared = 3, 40, 2, 8, 8, 2
    k = rng.standard_normal((B, L, 1, D))
    k[:, :shared * ps] = k[0, :shared * ps]  # equal prefixes
    q = rng.standard_normal((B, H, D))
    table = synth.page_table(11, 3, B, L // ps, 2 + B * 3, shared=shared)
    assert (table[:, :shared] == table[0, :shared]).all()
    kp = _scatter(k, table, ps, 2 + B * 3)
    O, LSE = att.decode_shard_paged(q, kp, table, ps, [0] * B, [L] * B, 0.4, dv=8)
    O2, L2 = att.decode_shard(q, k, [0] * B, [L] * B, 0.4, dv=8)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, L2)


def test_entry_outside_the_pool_reads_page_zero():
    rng = np.random.default_rng(7)
    ps, n_pages, H, D = 4, 5, 2, 8
    kp = rng.standard_normal((n_pages * ps, 1, D))
    q = rng.standard_normal((1, H, D))
    bad = np.array([[3, -1, 7, 2]], np.int32)
    fixed = np.array([[3, 0, 0, 2]], np.int32)
    O, LSE = att.decode_shard_paged(q, kp, bad, ps, [1], [15], 0.5, dv=8)
    O2, L2 = att.decode_shard_paged(q, kp, fixed, ps, [1], [15], 0.5, dv=8)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, L2)


def test_page_size_one_and_one_page():
    rng = np.random.default_rng(8)
    B, L, H, D = 2, 12, 2, 8
    k = rng.standard_normal((B, L, 1, D))
    q = rng.standard_normal((B, H, D))
    O2, L2 = att.decode_shard(q, k, [2, 0], [12, 7], 0.5, dv=8)
    # page size 1: every token its own page
    t1 = synth.page_table(11, 4, B, L, B * L)
    O, LSE = att.decode_shard_paged(q, _scatter(k, t1, 1, B * L), t1, 1, [2, 0], [12, 7], 0.5, dv=8)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, L2)
    # one page per request (page size L): the pool is the cache, requests swapped
    t2 = np.array([[1], [0]], np.int32)
    O, LSE = att.decode_shard_paged(q, k[::-1].reshape(B * L, 1, D), t2, L, [2, 0], [12, 7], 0.5, dv=8)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, L2)
