"""Pins for the oracle's sparse (top-k index list) MLA attention (CPU only).

A query attends only the cache rows its list names (*Long Context* 2.4; vLLM
GLM-5.3 post, footnote 1, for the per-query work)."""

import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import attention as att
from oracle import formats, plans


def test_printed_cost_of_one_query(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "sparse_mla_cost.json")))
    assert round(g["k_rows"] * g["row_bytes"] / 1e6, 2) == g["rows_mb"]
    for heads, key in ((8, "heads_8"), (64, "heads_64")):
        f, b = att.sparse_mla_cost(g["k_rows"], heads, g["row_bytes"], g["bytes_per_head"], g["flops_per_row_head"])
        e = g[key]
        assert abs(f / 1e6 - e["mflops"]) < 0.5 and round(b / 1e6, 2) == e["mb"]
        assert round(f / b) == e["flop_per_byte"]


def _rand(seed, N, B, L, H=4, D=576):
    rng = np.random.default_rng(seed)
    return rng, rng.standard_normal((N, H, D)), rng.standard_normal((B, L, 1, D))


def test_full_ordered_list_is_dense_decode():
    rng, q, cache = _rand(1, 3, 3, 50)
    ends = [50, 7, 1]
    K = 50
    idx = np.full((3, K), -1)
    for n, e in enumerate(ends):
        idx[n, :e] = np.arange(e)
    o, l = att.sparse_mla(q, cache, idx, 0.05)
    ro, rl = att.decode_shard(q, cache, [0, 0, 0], ends, 0.05, dv=512)
    assert np.allclose(o, ro, atol=1e-13) and np.allclose(l, rl, atol=1e-13)


def _masked_dense(q, keys, sel_mask, scale, dv=512):
    """Textbook masked softmax over all rows, the unlisted ones masked out."""
    s = scale * (keys @ q)
    s = np.where(sel_mask, s, -np.inf)
    if not sel_mask.any():
        return np.zeros(dv), -np.inf
    m = s.max()
    e = np.exp(s - m)
    return (e / e.sum()) @ keys[:, :dv], m + math.log(e.sum())


def test_random_lists_equal_masked_dense_softmax():
    rng, q, cache = _rand(2, 6, 2, 300)
    req = np.array([0, 1, 1, 0, 1, 0])
    K = 64
    idx = np.stack([rng.choice(300, K, replace=False) for _ in range(6)])
    n_idx = np.array([64, 10, 1, 0, 33, 64])
    o, l = att.sparse_mla(q, cache, idx, 0.04, n_idx=n_idx, req=req)
    for n in range(6):
        mask = np.zeros(300, bool)
        mask[idx[n, :n_idx[n]]] = True
        for h in range(q.shape[1]):
            ro, rl = _masked_dense(q[n, h], cache[req[n], :, 0], mask, 0.04)
            assert np.allclose(o[n, h], ro, atol=1e-12)
            assert (np.isneginf(rl) and np.isneginf(l[n, h])) or abs(l[n, h] - rl) < 1e-12


def test_order_and_padding_do_not_matter():
    rng, q, cache = _rand(3, 2, 2, 100)
    idx = np.stack([rng.choice(100, 40, replace=False) for _ in range(2)])
    o, l = att.sparse_mla(q, cache, idx, 0.05)
    perm = np.stack([rng.permutation(r) for r in idx])
    padded = np.concatenate([perm, np.full((2, 5), -1), np.full((2, 3), 100), np.full((2, 2), 7)], axis=1)
    op, lp = att.sparse_mla(q, cache, padded, 0.05, n_idx=[48, 48])   # the trailing 7s lie past n_idx
    assert np.allclose(o, op, atol=1e-12) and np.allclose(l, lp, atol=1e-12)


def test_duplicate_entry_counts_twice():
    rng, q, cache = _rand(4, 1, 1, 10, H=1)
    o, l = att.sparse_mla(q, cache, np.array([[3, 3]]), 0.1)
    s = 0.1 * float(cache[0, 3, 0] @ q[0, 0])
    assert np.allclose(o[0, 0], cache[0, 3, 0, :512]) and abs(l[0, 0] - (s + math.log(2))) < 1e-12


def test_fp8_list_over_all_rows_is_fp8_decode():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((2, 40, 1, 576)) * 0.5).astype(np.float32)
    codes, sc = synth.f32_to_e4m3(x)
    q = rng.standard_normal((2, 4, 576))
    idx = np.tile(np.arange(40), (2, 1))
    o, l = att.sparse_mla(q, codes, idx, 0.05, decode=formats.e4m3_to_f64, kv_scale=sc[..., 0])
    ro, rl = att.decode_shard(q, codes, [0, 0], [40, 40], 0.05, dv=512, decode=formats.e4m3_to_f64,
                              kv_scale=sc[..., 0])
    assert np.allclose(o, ro, atol=1e-13) and np.allclose(l, rl, atol=1e-13)


@pytest.mark.parametrize("C", [2, 3, 8])
def test_owner_local_lists_merge_to_the_full_list(C):
    """Round-robin owners (Long Context 3.1): each rank attends the listed
    entries it stores, at their local rows; the merged states equal the
    unsharded sparse attention (DeepSeek-V4 notes, 5.2: owner-local attention
    plus the LSE combine)."""
    rng, q, cache = _rand(6, 3, 3, 200)
    idx = np.stack([rng.choice(200, 50, replace=False) for _ in range(3)])
    o, l = att.sparse_mla(q, cache, idx, 0.05)
    os_, ls_ = [], []
    for r in range(C):
        own = plans.round_robin_own_tokens(200, C, r)
        local = cache[:, own]
        loc_idx = np.full_like(idx, -1)
        for n in range(3):
            mine = [t // C for t in idx[n] if t % C == r]
            loc_idx[n, :len(mine)] = mine
        po, pl = att.sparse_mla(q, local, loc_idx, 0.05)
        os_.append(po)
        ls_.append(pl)
    mo, ml = att.merge_states(np.stack(os_), np.stack(ls_))
    assert np.allclose(mo, o, atol=1e-12) and np.allclose(ml, l, atol=1e-12)


def test_query_of_an_unknown_request_selects_nothing():
    rng, q, cache = _rand(7, 2, 2, 20)
    idx = np.tile(np.arange(20), (2, 1))
    o, l = att.sparse_mla(q, cache, idx, 0.1, req=[1, 5])
    ro, rl = att.sparse_mla(q[:1], cache[1:], idx[:1], 0.1)
    assert np.allclose(o[0], ro[0]) and np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
