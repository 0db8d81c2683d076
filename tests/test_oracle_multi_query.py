"""Pins for the oracle's multi-query (speculative / MTP) decode (CPU only).

A request's last Q slots are its query rows; row k at slot p = L - Q + k
reads slots 0..p (causal attention, *How GPUs Share a Long Context*, 1.1).
Each rank reads the part of 0..p it stores (contiguous chunks, vLLM DCP
post, section 4; round-robin storage, *Long Context* 3.1), and the merged
states must equal causal attention over the whole request."""

import itertools
import math

import numpy as np
import pytest

from oracle import attention as att
from oracle import plans


def _local_slots(layout, L, C, r, n_repl):
    """Slot held by each local row (None for a replicated row)."""
    if layout == "contiguous":
        s0, s1 = plans.contiguous_shards(L, C)[r]
        return list(range(s0, s1))
    return [None] * n_repl + plans.round_robin_own_tokens(L, C, r)


@pytest.mark.parametrize("layout", ["contiguous", "round_robin"])
def test_q1_reduces_to_single_query_decode(layout):
    ctx = [1, 2, 7, 16, 33]
    for C in (1, 2, 3, 4, 8):
        for r in range(C):
            beg, end = plans.plan_multi_query(layout, C, r, ctx, 1)
            if layout == "round_robin":
                rb, re_ = plans.plan_round_robin(C, r, ctx)
                assert (beg == rb).all() and (end == re_).all()
            else:
                for b, L in enumerate(ctx):
                    s0, s1 = plans.contiguous_shards(L, C)[r]
                    assert beg[b] == 0 and end[b] == s1 - s0


@pytest.mark.parametrize("layout,n_repl", [("contiguous", 0), ("round_robin", 0), ("round_robin", 2)])
def test_each_row_sees_its_causal_prefix_exactly_once(layout, n_repl):
    """Brute force: over all ranks, row k sees every slot 0..p exactly once,
    no slot after p, and the replicated rows exactly once."""
    for C, Q in itertools.product([1, 2, 3, 4], [1, 2, 3, 4, 8]):
        for owner in range(C if layout == "round_robin" else 1):
            for L in range(Q, Q + 13):
                seen = [dict() for _ in range(Q)]
                repl_seen = [0] * Q
                for r in range(C):
                    beg, end = plans.plan_multi_query(layout, C, r, [L], Q, n_repl, owner)
                    held = _local_slots(layout, L, C, r, n_repl)
                    for k in range(Q):
                        for row in range(beg[0], end[k]):
                            if held[row] is None:
                                repl_seen[k] += 1
                            else:
                                seen[k][held[row]] = seen[k].get(held[row], 0) + 1
                for k in range(Q):
                    p = L - Q + k
                    assert seen[k] == {t: 1 for t in range(p + 1)}
                    assert repl_seen[k] == n_repl


def _masked_causal(q, keys, n_repl, L, Q, scale):
    """Textbook masked softmax: row k (slot L - Q + k) over the replicated
    keys plus slots 0..L-1 with the slots after it masked out."""
    s = (q @ keys.T) * scale                                # [Q, n_repl + L]
    slot = np.concatenate([np.full(n_repl, -1), np.arange(L)])
    p = L - Q + np.arange(Q)
    s = np.where(slot[None, :] <= p[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(axis=1, keepdims=True)) @ keys, (m[:, 0] + np.log(e.sum(axis=1)))


def _sharded(layout, q, main, repl, ctx, C, owner, Q, causal=True):
    B, _, Hq, D = q.shape
    n_repl = repl.shape[1]
    os_, ls_ = [], []
    for r in range(C):
        rows = [_local_slots(layout, L, C, r, n_repl) for L in ctx]
        local = np.zeros((B, max(1, max(len(x) for x in rows)), 1, D))
        for b, held in enumerate(rows):
            for i, t in enumerate(held):
                local[b, i, 0] = repl[b, i] if t is None else main[b, t]
        beg, end = plans.plan_multi_query(layout, C, r, ctx, Q, n_repl, owner)
        if not causal:  # planted mistake: every row reads the whole local cache
            end = np.repeat(end.reshape(B, Q)[:, -1:], Q, axis=1).reshape(-1)
        o, l = att.decode_shard_mq(q, local, beg, end, 1.0 / math.sqrt(D), dv=D)
        os_.append(o)
        ls_.append(l)
    return att.merge_states(np.stack(os_), np.stack(ls_))


@pytest.mark.parametrize("layout,n_repl", [("contiguous", 0), ("round_robin", 0), ("round_robin", 3)])
def test_merged_equals_masked_causal_attention(layout, n_repl):
    rng = np.random.default_rng(5)
    B, Hq, D = 3, 2, 8
    for C, Q in itertools.product([1, 2, 4], [1, 2, 4]):
        ctx = [Q + 11, Q, Q + 5]
        q = rng.standard_normal((B, Q, Hq, D))
        main = rng.standard_normal((B, max(ctx), D))
        repl = rng.standard_normal((B, n_repl, D))
        for owner in range(C if layout == "round_robin" else 1):
            o, l = _sharded(layout, q, main, repl, ctx, C, owner, Q)
            for b, L in enumerate(ctx):
                keys = np.concatenate([repl[b], main[b, :L]])
                for h in range(Hq):
                    ro, rl = _masked_causal(q[b, :, h], keys, n_repl, L, Q, 1.0 / math.sqrt(D))
                    assert np.allclose(o[b, :, h], ro, atol=1e-12)
                    assert np.allclose(l[b, :, h], rl, atol=1e-12)


def test_dropping_the_causal_mask_is_detected():
    rng = np.random.default_rng(9)
    B, Q, Hq, D, C = 1, 4, 1, 8, 2
    ctx = [9]
    q = rng.standard_normal((B, Q, Hq, D))
    main = rng.standard_normal((B, 9, D))
    repl = np.zeros((B, 0, D))
    good, _ = _sharded("contiguous", q, main, repl, ctx, C, 0, Q)
    bad, _ = _sharded("contiguous", q, main, repl, ctx, C, 0, Q, causal=False)
    # rows before the last differ, the last row (which sees everything) agrees
    assert np.abs(good[0, :Q - 1] - bad[0, :Q - 1]).max() > 1e-3
    assert np.allclose(good[0, Q - 1], bad[0, Q - 1], atol=1e-12)


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        plans.plan_multi_query("contiguous", 2, 0, [3], 4)           # fewer than Q slots
    with pytest.raises(ValueError):
        plans.plan_multi_query("contiguous", 2, 0, [8], 2, n_repl=1)  # replicated rows on chunks
    with pytest.raises(ValueError):
        plans.plan_multi_query("paged", 2, 0, [8], 2)
    with pytest.raises(ValueError):
        plans.plan_multi_query("round_robin", 2, 2, [8], 2)
