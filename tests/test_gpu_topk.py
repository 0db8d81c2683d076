"""GPU parity: exact distributed top-k (local lists, merge, owner routing)
against the oracle, bit-exact; then the whole split-index sparse path."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as att
from oracle import formats, plans, topk
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


def _scores(rng, N, L, ties=True):
    s = rng.standard_normal((N, L)).astype(np.float32)
    if ties:  # coarse values: many equal scores
        s = np.round(s * 4) / 4
        s = s.astype(np.float32)
    if L > 8:
        s[:, 3] = -0.0
        s[:, 5] = 0.0
        s[0, 7] = np.nan
        s[-1, 1] = -np.inf
    return s


def _i32(x):
    return H.i32_tensor(np.asarray(x, np.int32))


@pytest.mark.parametrize("L,k", [(0, 4), (1, 1), (100, 0), (100, 64), (5000, 2048), (16384, 2048), (3000, 5000), (16385, 700), (40000, 3000)])
def test_local_topk_bit_exact(cpa, L, k):
    rng = np.random.default_rng(L + k)
    N = 6
    s = _scores(rng, N, L)
    n_valid = np.array([L, L // 2, 0, min(L, 1), max(0, L - 7), L], np.int32)
    for base, stride in ((3, 8), (1000, 1)):
        osc, oid, orow, cnt = cpa.attn_topk_local(H.f32_tensor(s), k, base, stride, n_valid=_i32(n_valid))
        _sync()
        osc, oid, orow, cnt = (H.host(t) for t in (osc, oid, orow, cnt))
        for n in range(N):
            rs, ri, rr = topk.local_topk(s[n], n_valid[n], k, base, stride)
            c = len(ri)
            assert cnt[n] == c
            assert np.array_equal(oid[n, :c], ri) and np.array_equal(orow[n, :c], rr)
            assert np.array_equal(osc[n, :c].astype(np.float32).view(np.uint32), rs.astype(np.float32).view(np.uint32))
            assert np.all(oid[n, c:] == -1) and np.all(orow[n, c:] == -1) and np.all(np.isneginf(osc[n, c:]))


def _local_lists(cpa, s_global, C, k, layout="round_robin"):
    """Run the local top-k of every rank on its own entries (GPU) and the
    oracle's; returns the GPU lists stacked [C, N, k] and the oracle lists."""
    import torch
    N, L = s_global.shape
    g_sc, g_id, g_row, g_cnt, ref = [], [], [], [], []
    for r in range(C):
        if layout == "round_robin":
            own = plans.round_robin_own_tokens(L, C, r)
            base, stride = r, C
        else:
            s0, s1 = plans.contiguous_shards(L, C)[r]
            own = list(range(s0, s1))
            base, stride = s0, 1
        loc = np.ascontiguousarray(s_global[:, own]) if own else np.zeros((N, 0), np.float32)
        osc, oid, orow, cnt = cpa.attn_topk_local(H.f32_tensor(loc), k, base, stride)
        g_sc.append(osc), g_id.append(oid), g_row.append(orow), g_cnt.append(cnt)
        ref.append([topk.local_topk(loc[n], len(own), k, base, stride) for n in range(N)])
    return (torch.stack(g_sc), torch.stack(g_id), torch.stack(g_row), torch.stack(g_cnt)), ref


@pytest.mark.parametrize("layout", ["round_robin", "contiguous"])
@pytest.mark.parametrize("L,C,k", [(1000, 4, 64), (37, 8, 5), (20000, 8, 2048), (10, 3, 40), (70000, 4, 5000), (3000, 64, 40)])
def test_merge_bit_exact_and_exact_global(cpa, layout, L, C, k):
    rng = np.random.default_rng(L * C + k)
    N = 5
    s = _scores(rng, N, L)
    (sc, ids, rows, cnt), ref = _local_lists(cpa, s, C, k, layout)
    oid, orow, ocnt = cpa.attn_topk_merge(sc, ids, rows, k, cand_count=cnt)
    _sync()
    oid, orow, ocnt = H.host(oid), H.host(orow), H.host(ocnt)
    for n in range(N):
        want_ids, want_rows = topk.merge_topk([ref[r][n] for r in range(C)], k)
        c = len(want_ids)
        assert np.array_equal(oid[n, :c], want_ids) and np.all(oid[n, c:] == -1)
        for r in range(C):
            cr = len(want_rows[r])
            assert ocnt[r, n] == cr
            assert np.array_equal(orow[r, n, :cr], want_rows[r]) and np.all(orow[r, n, cr:] == -1)
        # exact: the same set as the direct global top k
        assert sorted(want_ids.tolist()) == sorted(topk.global_topk(s[n], k).tolist())


def test_split_index_sparse_attention_end_to_end(cpa):
    """Index scores split round robin over C ranks: local top-k on each rank,
    merge, each owner's sparse attention over its local rows, LSE merge --
    equals sparse attention over the global top k on the whole cache."""
    import torch
    rng = np.random.default_rng(8)
    N, L, C, k = 3, 6000, 4, 512
    s = _scores(rng, N, L, ties=False)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((N, 64, 576)).astype(np.float32))
    cb = synth.f32_to_bf16_bits((rng.standard_normal((N, L, 1, 576)) * 0.5).astype(np.float32))
    (sc, ids, rows, cnt), _ = _local_lists(cpa, s, C, k)
    oid, orow, ocnt = cpa.attn_topk_merge(sc, ids, rows, k, cand_count=cnt)
    po, pl = [], []
    for r in range(C):
        own = plans.round_robin_own_tokens(L, C, r)
        local = H.bf16_tensor(np.ascontiguousarray(cb[:, own]))
        o, l = cpa.attn_sparse_mla(H.bf16_tensor(qb), local, orow[r].contiguous(), 1 / 24, n_idx=ocnt[r].contiguous())
        po.append(o), pl.append(l)
    mo, ml = cpa.attn_merge_states(torch.stack(po), torch.stack(pl))
    _sync()
    gidx = np.stack([topk.global_topk(s[n], k) for n in range(N)]).astype(np.int32)
    ro, rl = att.sparse_mla(formats.bf16_bits_to_f64(qb), cb, gidx, 1 / 24, decode=formats.bf16_bits_to_f64)
    H.check_lowp(H.host(mo), H.host(ml), ro, rl, "split-index sparse attention")


def test_topk_rejects_bad_arguments(cpa):
    import torch
    s = torch.zeros((2, 10), dtype=torch.float32, device="cuda")
    with pytest.raises(cpa.CpaError):   # ids past 2^31
        cpa.attn_topk_local(s, 4, 2 ** 31 - 5, 1)
    with pytest.raises(cpa.CpaError):   # equal ids
        cpa.attn_topk_local(s, 4, 0, 0)
    with pytest.raises(cpa.CpaError):
        cpa.attn_topk_local(s, -1, 0, 1)
