"""Pins for the oracle's exact distributed top-k (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import plans
from oracle import topk


def _rank_lists(scores, C, layout, k, tie_by_local_row=False):
    """Each rank's local list over the entries it stores."""
    L = len(scores)
    lists = []
    for r in range(C):
        if layout == "round_robin":
            own = plans.round_robin_own_tokens(L, C, r)
            base, stride = r, C
        else:
            s0, s1 = plans.contiguous_shards(L, C)[r]
            own = list(range(s0, s1))
            base, stride = s0, 1
        loc = np.asarray(scores)[own]
        if tie_by_local_row:  # planted mistake: ties broken by local row, not global id
            sel = topk.select(loc, np.arange(len(own)), k)
            lists.append((loc[sel], np.asarray(own, np.int64)[sel], sel))
        else:
            lists.append(topk.local_topk(loc, len(own), k, base, stride))
    return lists


@pytest.mark.parametrize("layout", ["round_robin", "contiguous"])
def test_merge_of_local_lists_is_the_global_top_k(layout):
    rng = np.random.default_rng(0)
    for trial in range(300):
        L = int(rng.integers(0, 40))
        C = int(rng.integers(1, 6))
        k = int(rng.integers(0, 12))
        # integer scores give many ties; sprinkle -0.0 / +0.0, NaN and -inf
        s = rng.integers(-3, 4, size=L).astype(np.float64)
        if L > 3:
            s[rng.integers(0, L)] = -0.0
            s[rng.integers(0, L)] = np.nan
            s[rng.integers(0, L)] = -np.inf
        ids, owner_rows = topk.merge_topk(_rank_lists(s, C, layout, k), k)
        want = topk.global_topk(s, k)
        assert sorted(ids.tolist()) == sorted(want.tolist())
        # every owner's rows map back to exactly its selected ids
        for r, rows in enumerate(owner_rows):
            if layout == "round_robin":
                back = [row * C + r for row in rows]
            else:
                back = [plans.contiguous_shards(L, C)[r][0] + row for row in rows]
            assert back == [int(i) for i in ids if int(i) in set(back)]
        assert sum(len(x) for x in owner_rows) == len(ids) == min(k, L)


def test_brute_force_order_on_tiny_inputs():
    """The selection equals the best min(k, n) under (score desc, id asc),
    checked against a pairwise-comparison count."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(0, 10))
        # values with many ties, -0.0 among them (equal to +0.0 as numbers)
        s = rng.choice(np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0]), size=n)
        ids = rng.permutation(50)[:n]
        k = int(rng.integers(0, 12))

        def better(a, b):  # candidate a ranks above candidate b
            return s[a] > s[b] or (s[a] == s[b] and ids[a] < ids[b])
        rank = [sum(better(b, a) for b in range(n)) for a in range(n)]
        want = sorted(a for a in range(n) if rank[a] < k)
        assert topk.select(s, ids, k).tolist() == want


def test_figure11_effect(golden_dir):
    """Two GPUs, round robin, top 3: GPU 0 keeps tokens 0, 4 and 6 from its
    own half, but token 0 loses against token 1, which only GPU 1 scores."""
    g = json.load(open(os.path.join(golden_dir, "topk_figure11.json")))
    s = np.array(g["scores"], np.float64)
    lists = _rank_lists(s, 2, "round_robin", g["k"])
    assert lists[0][1].tolist() == g["gpu0_local"]
    ids, _ = topk.merge_topk(lists, g["k"])
    assert 1 in ids and 0 not in ids
    assert sorted(ids.tolist()) == sorted(topk.global_topk(s, g["k"]).tolist())


def test_closed_forms():
    s = np.array([0.5, 2.0, 2.0, -1.0, 2.0])
    assert topk.select(s, np.arange(5), 99).tolist() == [0, 1, 2, 3, 4]
    assert topk.select(s, np.arange(5), 1).tolist() == [1]            # ties: lowest id
    assert topk.select(s, np.array([9, 8, 7, 6, 5]), 1).tolist() == [4]
    assert topk.select(np.zeros(6), np.arange(6)[::-1], 2).tolist() == [4, 5]   # ids 1 and 0
    assert topk.select(np.array([np.nan, -np.inf]), np.arange(2), 1).tolist() == [1]
    assert topk.select(np.array([-0.0, 0.0]), np.array([1, 0]), 1).tolist() == [1]
    assert topk.select(np.array([0.0, -0.0]), np.array([1, 0]), 1).tolist() == [1]   # -0 = +0: lower id


def test_local_tie_break_by_row_is_detected():
    """Breaking local ties by local row instead of global id loses
    exactness for contiguous shards: the merge then disagrees with the
    global top k on some input, which the test above would catch."""
    rng = np.random.default_rng(2)
    found = False
    for _ in range(500):
        L, C, k = 12, 3, 2
        s = rng.integers(0, 2, size=L).astype(np.float64)
        # reverse the global ids inside each chunk so row order and id order differ
        lists = []
        for r in range(C):
            s0, s1 = plans.contiguous_shards(L, C)[r]
            own = np.arange(s1 - 1, s0 - 1, -1)
            loc = s[own]
            sel = topk.select(loc, np.arange(len(own)), k)
            lists.append((loc[sel], own[sel], sel))
        ids, _ = topk.merge_topk(lists, k)
        if sorted(ids.tolist()) != sorted(topk.global_topk(s, k).tolist()):
            found = True
            break
    assert found
