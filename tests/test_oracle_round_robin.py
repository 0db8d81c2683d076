"""Pins for the oracle's round-robin decode ownership (CPU only).

Round-robin storage (*How GPUs Share a Long Context*, 3.1; DeepSeek-V4 notes,
section 5: owner(j) = j mod P) and the rule that replicated entries add their
probability mass once (DeepSeek-V4 notes, 5.3)."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as att
from oracle import plans


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_printed_slot_example(golden_dir):
    g = _load(golden_dir, "round_robin_slot_c4.json")
    assert plans.round_robin_slot(g["slot"], g["C"]) == (g["gpu"], g["row"])
    # the slot's owner stores it as that row of its local token list
    assert plans.round_robin_own_tokens(g["slot"] + 1, g["C"], g["gpu"])[g["row"]] == g["slot"]


def test_printed_capacity_example(golden_dir):
    e = _load(golden_dir, "round_robin_slot_c4.json")["capacity_example"]
    gib = 1024 ** 3
    full = e["tokens"] * e["bytes_per_token"] / gib
    worst = max(len(plans.round_robin_own_tokens(e["tokens"], e["gpus"], r)) for r in range(e["gpus"]))
    assert round(full, 1) == e["full_gb"]
    assert round(worst * e["bytes_per_token"] / gib, 1) == e["per_gpu_gb"]


@pytest.mark.parametrize("C", [1, 2, 3, 4, 7])
def test_every_slot_stored_exactly_once(C):
    for L in range(0, 30):
        seen = {}
        for r in range(C):
            own = plans.round_robin_own_tokens(L, C, r)
            assert own == sorted(own)
            for row, slot in enumerate(own):
                assert slot not in seen
                seen[slot] = (r, row)
                assert plans.round_robin_slot(slot, C) == (r, row)
        assert sorted(seen) == list(range(L))
        # balanced: local lengths differ by at most one, early ranks take the rest
        lens = [len(plans.round_robin_own_tokens(L, C, r)) for r in range(C)]
        assert max(lens) - min(lens) <= 1 and lens == sorted(lens, reverse=True)


def test_plan_ranges_ragged_and_replicated():
    ctx = [0, 1, 5, 13]
    for C, n_repl, owner in itertools.product([1, 2, 4], [0, 3], [0, 1]):
        if owner >= C:
            continue
        for r in range(C):
            beg, end = plans.plan_round_robin(C, r, ctx, n_repl, owner)
            for b, L in enumerate(ctx):
                n_own = len(plans.round_robin_own_tokens(L, C, r))
                assert end[b] == n_repl + n_own
                assert beg[b] == (0 if r == owner else n_repl)


def _round_robin_states(q, main, repl, ctx, C, owner, include_all=False):
    """Partial states of the C ranks over their local caches (replicated rows
    first), merged."""
    B, Hq, D = q.shape
    n_repl = repl.shape[1]
    Lmax_local = n_repl + max(len(plans.round_robin_own_tokens(L, C, 0)) for L in ctx)
    os_, ls_ = [], []
    for r in range(C):
        local = np.zeros((B, Lmax_local, 1, D))
        local[:, :n_repl, 0] = repl
        for b, L in enumerate(ctx):
            for row, slot in enumerate(plans.round_robin_own_tokens(L, C, r)):
                local[b, n_repl + row, 0] = main[b, slot]
        beg, end = plans.plan_round_robin(C, r, ctx, n_repl, owner)
        if include_all:
            beg = np.zeros_like(beg)
        o, l = att.decode_shard(q, local, beg, end, 1.0 / math.sqrt(D), vcache=None, dv=D)
        os_.append(o)
        ls_.append(l)
    return att.merge_states(np.stack(os_), np.stack(ls_))


def test_merged_round_robin_equals_unsharded_attention():
    rng = np.random.default_rng(11)
    B, Hq, D = 3, 2, 8
    ctx = [13, 1, 6]
    for n_repl, C in itertools.product([0, 1, 3], [1, 2, 3, 4]):
        q = rng.standard_normal((B, Hq, D))
        main = rng.standard_normal((B, max(ctx), D))
        repl = rng.standard_normal((B, n_repl, D))
        for owner in range(C):
            o, l = _round_robin_states(q, main, repl, ctx, C, owner)
            for b, L in enumerate(ctx):
                keys = np.concatenate([repl[b], main[b, :L]])
                for h in range(Hq):
                    ro, rl = att.attend(q[b, h], keys, keys, 1.0 / math.sqrt(D))
                    assert np.allclose(o[b, h], ro, atol=1e-12) and abs(l[b, h] - rl) < 1e-12


def test_replicated_mass_counted_once_is_what_the_check_detects():
    """With C > 1 ranks all including the replicated rows, the merged LSE
    exceeds the true one (the replicated mass is counted C times): the parity
    check above would fail for that mistake."""
    rng = np.random.default_rng(3)
    B, Hq, D, C = 1, 1, 8, 4
    ctx = [9]
    q = rng.standard_normal((B, Hq, D))
    main = rng.standard_normal((B, 9, D))
    repl = rng.standard_normal((B, 2, D))
    _, good = _round_robin_states(q, main, repl, ctx, C, 0)
    _, bad = _round_robin_states(q, main, repl, ctx, C, 0, include_all=True)
    assert bad[0, 0] > good[0, 0] + 1e-6
