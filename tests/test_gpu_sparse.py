"""GPU parity: sparse (top-k index list) MLA attention against the oracle."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as att
from oracle import formats, plans
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cpa():
    import torch
    import context_attention_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def _inputs(N, B, L, seed, std=0.5):
    rng = np.random.default_rng(seed)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((N, 64, 576)).astype(np.float32))
    cb = synth.f32_to_bf16_bits((rng.standard_normal((B, L, 1, 576)) * std).astype(np.float32))
    return rng, qb, cb


def _run(cpa, qb, cb, idx, scale, n_idx=None, req=None, rows=None):
    o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), H.bf16_tensor(cb), H.i32_tensor(idx), scale,
                               n_idx=H.i32_tensor(n_idx) if n_idx is not None else None,
                               req=H.i32_tensor(req) if req is not None else None)
    _sync()
    ro, rl = att.sparse_mla(formats.bf16_bits_to_f64(qb), cb, idx, scale, n_idx=n_idx, req=req,
                            decode=formats.bf16_bits_to_f64, rows=rows)
    return H.host(o), H.host(l), ro, rl


def test_sparse_ragged_lists_with_padding(cpa):
    """Five queries on three requests; lists of 100 entries with padding
    (-1, Lmax, a huge value) in the middle, counts 0, 1, 33, 100 and 64."""
    N, B, L, K = 5, 3, 300, 100
    rng, qb, cb = _inputs(N, B, L, 11)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    idx[1, 5] = -1
    idx[2, 7] = L
    idx[4, 0] = 2 ** 30
    req = np.array([2, 0, 1, 1, 0], np.int32)
    n_idx = np.array([0, 1, 33, 100, 64], np.int32)
    o, l, ro, rl = _run(cpa, qb, cb, idx, 1 / 24, n_idx=n_idx, req=req)
    H.check_lowp(o, l, ro, rl, "sparse ragged")
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))


@pytest.mark.parametrize("K", [1, 31, 32, 33, 2048])
def test_sparse_decode_shaped(cpa, K):
    """One query per request (no req): tile-exact, ragged and long lists; the
    2,048-entry lists run as several splits plus the merge."""
    N, L = 4, 5000
    rng, qb, cb = _inputs(N, N, L, 100 + K)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    o, l, ro, rl = _run(cpa, qb, cb, idx, 1 / 24)
    H.check_lowp(o, l, ro, rl, f"sparse K={K}")


@pytest.mark.parametrize("fp8", [False, True])
def test_sparse_decode_shaped_8_queries(cpa, fp8):
    """8 queries of 2,048 rows: the queries divide over the 8 XCDs, so the
    splits of a query run on one XCD (their workgroup order differs from the
    4-query case)."""
    N, L, K = 8, 5000, 2048
    if fp8:
        rng, qb, codes, sc = _fp8_inputs(N, N, L, 700)
        idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
        o, l, ro, rl = _run_fp8(cpa, qb, codes, sc, idx, 1 / 24)
    else:
        rng, qb, cb = _inputs(N, N, L, 701)
        idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
        o, l, ro, rl = _run(cpa, qb, cb, idx, 1 / 24)
    H.check_lowp(o, l, ro, rl, f"sparse 8 queries fp8={fp8}")


def test_sparse_whole_tiles_of_padding(cpa):
    """Lists whose first tiles are all padding (the heads have seen no
    selection yet), with padding tiles in the middle and at the end."""
    N, L, K = 3, 900, 300
    rng, qb, cb = _inputs(N, N, L, 17)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    idx[0, :70] = -1
    idx[1, 96:160] = L + 5
    idx[2, 200:] = -7
    o, l, ro, rl = _run(cpa, qb, cb, idx, 1 / 24)
    H.check_lowp(o, l, ro, rl, "sparse padding tiles")


def test_sparse_full_ordered_list_matches_dense_decode(cpa):
    N, L = 2, 777
    rng, qb, cb = _inputs(N, N, L, 5)
    idx = np.tile(np.arange(L, dtype=np.int32), (N, 1))
    o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), H.bf16_tensor(cb), H.i32_tensor(idx), 1 / 24)
    od, ld = cpa.attn_decode_shard(H.bf16_tensor(qb), H.bf16_tensor(cb), None, H.i32_tensor([0, 0]),
                                   H.i32_tensor([L, L]), L, 1 / 24)
    _sync()
    ro, rl = att.decode_shard(formats.bf16_bits_to_f64(qb), cb, [0, 0], [L, L], 1 / 24, dv=512,
                              decode=formats.bf16_bits_to_f64)
    H.check_lowp(H.host(o), H.host(l), ro, rl, "sparse full list")
    H.check_lowp(H.host(od), H.host(ld), ro, rl, "dense decode")


def test_sparse_spiky_scores(cpa):
    """Listed rows that copy a query row give large logits late in the list
    (the running-max rescale)."""
    N, L, K = 2, 1000, 512
    rng, qb, cb = _inputs(N, N, L, 9)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    for n in range(N):
        for j in (200, 401, 511):
            cb[n, idx[n, j], 0, :] = qb[n, 3, :]
    o, l, ro, rl = _run(cpa, qb, cb, idx, 8 / 24)
    H.check_lowp_scaled(o, l, ro, rl, "sparse spiky")


def test_sparse_empty_cases(cpa):
    import torch
    N, B, L = 3, 2, 64
    rng, qb, cb = _inputs(N, B, L, 3)
    # k = 0: no selection anywhere
    idx0 = np.zeros((N, 0), np.int32)
    o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), H.bf16_tensor(cb), torch.zeros((N, 0), dtype=torch.int32,
                               device="cuda"), 1 / 24, req=H.i32_tensor([0, 1, 0]))
    _sync()
    assert np.all(H.host(o) == 0) and np.all(np.isneginf(H.host(l)))
    # a request outside [0, B) and an all-padding list
    idx = np.stack([rng.choice(L, 40, replace=False) for _ in range(N)]).astype(np.int32)
    idx[2, :] = -1
    o, l, ro, rl = _run(cpa, qb, cb, idx, 1 / 24, req=np.array([0, 7, 1], np.int32))
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1])) and np.all(np.isneginf(l[2]))
    H.check_lowp(o, l, ro, rl, "sparse empty cases")


@pytest.mark.parametrize("C", [2, 4])
def test_sparse_owner_local_lists_merge(cpa, C):
    """Round-robin owners: each rank attends the listed entries it stores (at
    their local rows); the merged GPU states equal the oracle's full lists."""
    import torch
    N, L, K = 3, 2000, 600
    rng, qb, cb = _inputs(N, N, L, 20 + C)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    po, pl = [], []
    for r in range(C):
        own = plans.round_robin_own_tokens(L, C, r)
        local = np.ascontiguousarray(cb[:, own])
        loc = np.full_like(idx, -1)
        cnt = np.zeros(N, np.int32)
        for n in range(N):
            mine = [t // C for t in idx[n] if t % C == r]
            loc[n, :len(mine)] = mine
            cnt[n] = len(mine)
        o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), H.bf16_tensor(local), H.i32_tensor(loc), 1 / 24,
                                   n_idx=H.i32_tensor(cnt))
        po.append(o)
        pl.append(l)
    mo, ml = cpa.attn_merge_states(torch.stack(po), torch.stack(pl))
    _sync()
    ro, rl = att.sparse_mla(formats.bf16_bits_to_f64(qb), cb, idx, 1 / 24, decode=formats.bf16_bits_to_f64)
    H.check_lowp(H.host(mo), H.host(ml), ro, rl, f"sparse owner-local C={C}")


def test_sparse_rejects_bad_arguments(cpa):
    import torch
    N, L = 2, 64
    rng, qb, cb = _inputs(N, N, L, 1)
    idx = H.i32_tensor(np.zeros((N, 8), np.int32))
    q, c = H.bf16_tensor(qb), H.bf16_tensor(cb)
    with pytest.raises(cpa.CpaError):   # more queries than requests without req
        cpa.attn_sparse_mla(H.bf16_tensor(np.concatenate([qb, qb])), c, H.i32_tensor(np.zeros((4, 8), np.int32)), 0.1)
    with pytest.raises(cpa.CpaError):   # scale
        cpa.attn_sparse_mla(q, c, idx, float("nan"))
    with pytest.raises(cpa.CpaError):   # short workspace
        cpa.attn_sparse_mla(q, c, H.i32_tensor(np.zeros((N, 2048), np.int32)), 0.1,
                            workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))


def _fp8_inputs(N, B, L, seed, std=0.5):
    rng = np.random.default_rng(seed)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((N, 64, 576)).astype(np.float32))
    codes, sc = synth.f32_to_e4m3((rng.standard_normal((B, L, 1, 576)) * std).astype(np.float32))
    return rng, qb, codes, sc[..., 0]


def _run_fp8(cpa, qb, codes, sc, idx, scale, n_idx=None, req=None):
    o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), H.u8_tensor(codes), H.i32_tensor(idx), scale,
                               n_idx=H.i32_tensor(n_idx) if n_idx is not None else None,
                               req=H.i32_tensor(req) if req is not None else None, kv_scale=H.f32_tensor(sc))
    _sync()
    ro, rl = att.sparse_mla(formats.bf16_bits_to_f64(qb), codes, idx, scale, n_idx=n_idx, req=req,
                            decode=formats.e4m3_to_f64, kv_scale=sc)
    return H.host(o), H.host(l), ro, rl


@pytest.mark.parametrize("K", [1, 33, 2048])
def test_sparse_fp8_decode_shaped(cpa, K):
    """FP8 E4M3 cache with per-token scales: one query per request, tile-exact,
    ragged and long lists (2,048 entries: several splits plus the merge)."""
    N, L = 4, 5000
    rng, qb, codes, sc = _fp8_inputs(N, N, L, 300 + K)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    o, l, ro, rl = _run_fp8(cpa, qb, codes, sc, idx, 1 / 24)
    H.check_lowp(o, l, ro, rl, f"sparse fp8 K={K}")


def test_sparse_fp8_ragged_padding_and_shared_requests(cpa):
    """FP8: five queries on three requests (rows shared through L2), counts
    0, 1, 33, 100 and 64, padding entries (-1, Lmax, a huge value) and a
    first tile that is all padding."""
    N, B, L, K = 5, 3, 300, 100
    rng, qb, codes, sc = _fp8_inputs(N, B, L, 12)
    idx = np.stack([rng.choice(L, K, replace=False) for _ in range(N)]).astype(np.int32)
    idx[1, 5] = -1
    idx[2, 7] = L
    idx[4, 0] = 2 ** 30
    idx[3, :32] = -3
    req = np.array([2, 0, 1, 1, 0], np.int32)
    n_idx = np.array([0, 1, 33, 100, 64], np.int32)
    o, l, ro, rl = _run_fp8(cpa, qb, codes, sc, idx, 1 / 24, n_idx=n_idx, req=req)
    H.check_lowp(o, l, ro, rl, "sparse fp8 ragged")
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))


def test_sparse_fp8_full_list_matches_fp8_decode(cpa):
    """Listing every row of a request in order is the FP8 dense decode."""
    N, L = 2, 777
    rng, qb, codes, sc = _fp8_inputs(N, N, L, 6)
    idx = np.tile(np.arange(L, dtype=np.int32), (N, 1))
    o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), H.u8_tensor(codes), H.i32_tensor(idx), 1 / 24,
                               kv_scale=H.f32_tensor(sc))
    od, ld = cpa.attn_decode_shard(H.bf16_tensor(qb), H.u8_tensor(codes), None, H.i32_tensor([0, 0]),
                                   H.i32_tensor([L, L]), L, 1 / 24, kv_scale=H.f32_tensor(sc))
    _sync()
    ro, rl = att.decode_shard(formats.bf16_bits_to_f64(qb), codes, [0, 0], [L, L], 1 / 24, dv=512,
                              decode=formats.e4m3_to_f64, kv_scale=sc)
    H.check_lowp(H.host(o), H.host(l), ro, rl, "sparse fp8 full list")
    H.check_lowp(H.host(od), H.host(ld), ro, rl, "fp8 dense decode")
