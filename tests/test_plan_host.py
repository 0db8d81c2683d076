"""The library's host planners are bit-exact against the oracle's plans
(CPU only: the planners are host code)."""

import numpy as np
import pytest

import context_attention_long_amd as cpa
from oracle import plans


def _same(lib_plan, ref):
    assert lib_plan.n_local == ref.n_local
    assert np.array_equal(lib_plan.tok_index, ref.tok_index)
    assert np.array_equal(lib_plan.pos_id, ref.pos_id)
    assert np.array_equal(lib_plan.req_id, ref.req_id)
    assert lib_plan.n_padded == ref.n_padded
    got = [tuple(int(x) for x in (s["req"], s["q_row0"], s["q_len"], s["pos0"], s["pos_stride"], s["kv_row0"]))
           for s in lib_plan.segments]
    assert got == [tuple(int(x) for x in s) for s in ref.segments]
    assert np.all(lib_plan.segments["reserved"] == 0)


@pytest.mark.parametrize("strategy", ["zigzag", "interleave"])
def test_planner_bit_exact_exhaustive_grid(strategy):
    lib_fn = cpa.cp_plan_zigzag if strategy == "zigzag" else cpa.cp_plan_interleave
    ref_fn = plans.plan_zigzag if strategy == "zigzag" else plans.plan_interleave
    rng = np.random.default_rng(123)
    batches = [[L] for L in range(0, 41)]
    for _ in range(60):
        n = int(rng.integers(1, 7))
        batches.append([int(x) for x in rng.integers(0, 41, size=n)])
    for new_len in batches:
        for prefix in (None, [int(x) for x in rng.integers(0, 6, size=len(new_len))]):
            for C in range(1, 17):
                for r in range(C):
                    _same(lib_fn(C, r, new_len, prefix), ref_fn(C, r, new_len, prefix))


def test_planner_workloads_bit_exact():
    from synth import agentic_lengths
    cases = [("zigzag", 4, 1, [16384], None), ("zigzag", 8, 0, [131072], [32768]),
             ("interleave", 4, 2, [int(x) for x in agentic_lengths(5)], None),
             ("interleave", 8, 7, [128000], None)]
    for strategy, C, r, L, P in cases:
        lib_fn = cpa.cp_plan_zigzag if strategy == "zigzag" else cpa.cp_plan_interleave
        ref_fn = plans.plan_zigzag if strategy == "zigzag" else plans.plan_interleave
        _same(lib_fn(C, r, L, P), ref_fn(C, r, L, P))
    p = cpa.cp_plan_interleave(4, 2, [int(x) for x in agentic_lengths(5)])
    assert p.n_local == 182010 and p.n_seg == 16
    assert int(np.sum(p.pos_id.astype(np.int64) + 1)) == 6654242875


def test_decode_shards_bit_exact():
    for L in (0, 1, 7, 4096, 131072, 1001):
        for C in (1, 2, 3, 4, 8, 16):
            assert cpa.cp_decode_shards(L, C) == plans.contiguous_shards(L, C)


def test_round_robin_plan_bit_exact():
    import context_attention_long_amd as cpa
    from oracle import plans
    ctx = [0, 1, 2, 7, 31, 100]
    for C in (1, 2, 3, 4, 8):
        for n_repl in (0, 2):
            for owner in range(min(C, 2)):
                for r in range(C):
                    beg, end, mx = cpa.cp_plan_round_robin(C, r, ctx, n_repl, owner)
                    rb, re = plans.plan_round_robin(C, r, ctx, n_repl, owner)
                    assert np.array_equal(beg, rb) and np.array_equal(end, re)
                    assert mx == max([n_repl] + list(re))
        for slot in range(0, 40):
            assert cpa.cp_round_robin_slot(slot, C) == plans.round_robin_slot(slot, C)


def test_round_robin_plan_rejects_bad_arguments():
    import context_attention_long_amd as cpa
    for args in ((0, 0, [3]), (2, 2, [3]), (2, -1, [3]), (2, 0, [-1])):
        with pytest.raises(cpa.CpaError):
            cpa.cp_plan_round_robin(*args)
    with pytest.raises(cpa.CpaError):
        cpa.cp_plan_round_robin(2, 0, [3], 1, 2)
    with pytest.raises(cpa.CpaError):
        cpa.cp_round_robin_slot(-1, 4)


@pytest.mark.parametrize("layout", ["contiguous", "round_robin"])
def test_multi_query_plan_bit_exact(layout):
    code = cpa.CPA_LAYOUT_CONTIGUOUS if layout == "contiguous" else cpa.CPA_LAYOUT_ROUND_ROBIN
    for Q in (1, 2, 3, 4, 8):
        ctx = [Q, Q + 1, Q + 6, 31 + Q, 100]
        for C in (1, 2, 3, 4, 8):
            for n_repl, owner in ([(0, 0)] if layout == "contiguous" else [(0, 0), (2, 0), (3, 1)]):
                if owner >= C:
                    continue
                for r in range(C):
                    beg, end, mx = cpa.cp_plan_multi_query(code, C, r, ctx, Q, n_repl, owner)
                    rb, re = plans.plan_multi_query(layout, C, r, ctx, Q, n_repl, owner)
                    assert np.array_equal(beg, rb) and np.array_equal(end, re)
                    # the last row sees the whole local request: its end bounds the cache rows
                    assert mx == max([n_repl] + list(re.reshape(len(ctx), Q)[:, -1]))


def test_multi_query_plan_rejects_bad_arguments():
    C_, R_ = cpa.CPA_LAYOUT_CONTIGUOUS, cpa.CPA_LAYOUT_ROUND_ROBIN
    for args in ((C_, 2, 0, [3], 4), (C_, 2, 0, [8], 0), (C_, 2, 0, [8], 2, 1), (C_, 2, 0, [8], 2, 0, 1),
                 (7, 2, 0, [8], 2), (R_, 2, 2, [8], 2), (R_, 2, 0, [8], 2, 1, 2), (R_, 0, 0, [8], 2),
                 (R_, 2, 0, [8], 2, -1)):
        with pytest.raises(cpa.CpaError):
            cpa.cp_plan_multi_query(*args)


def test_named_workloads_draw_the_recorded_inputs(golden_dir):
    """The named synthetic workloads keep their sizes and seed families: the
    ragged interleave batch is the recorded 16-length mix, and every
    workload's first query values come from its own family."""
    import json
    import os

    import synth
    with open(os.path.join(golden_dir, "agentic_lengths_seed5.json")) as f:
        fix = json.load(f)
    w = synth.workload("gqa_interleave_prefill_agentic16")
    assert w["new_len"] == fix["lengths"] and sum(w["new_len"]) == fix["total"] == 728040
    sizes = {"gqa_decode_f32_4k": (1, 8, 1, 128, 4096), "mla_decode_131k": (64, 64, 1, 576, 131072)}
    for name, (B, Hq, Hkv, D, L) in sizes.items():
        c = synth.workload(name)
        assert (c["B"], c["Hq"], c["Hkv"], c["Dqk"], c["L"]) == (B, Hq, Hkv, D, L)
    assert synth.workload("gqa_zigzag_prefill_16k")["new_len"] == [16384]
    assert synth.workload("mla_zigzag_prefill_prefix32k")["prefix_len"] == [32768]
    seeds = [synth.workload(n)["seed"] for n in synth.WORKLOADS]
    assert len(set(seeds)) == len(seeds)
    a = synth.bf16_normal(synth.workload("mla_decode_131k")["seed"], 1, (2, 3, 4))
    b = synth.bf16_normal(synth.workload("gqa_zigzag_prefill_16k")["seed"], 1, (2, 3, 4))
    assert not np.array_equal(a, b)
