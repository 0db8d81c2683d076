"""Pins for the oracle's shard plans (CPU only)."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import plans


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_interleave_printed_example_5_3(golden_dir):
    g = _load(golden_dir, "interleave_5_3_cp4.json")
    for r, want in g["printed"].items():
        p = plans.plan_interleave(g["C"], int(r), g["new_len"])
        assert p.tok_index.tolist() == want["tok_index"]
    # index 5 is the first new token of the second request
    p1 = plans.plan_interleave(g["C"], 1, g["new_len"])
    i = p1.tok_index.tolist().index(5)
    assert p1.req_id[i] == g["printed_index5"]["req"]
    assert p1.pos_id[i] == g["printed_index5"]["pos"]


def test_cp4_16_tokens_worked_examples(golden_dir):
    g = _load(golden_dir, "cp4_16tok.json")
    C, L = g["C"], g["new_len"]
    for r in range(C):
        z = plans.plan_zigzag(C, r, L)
        assert z.tok_index.tolist() == g["zigzag_tok_index"][str(r)]
        assert [s[3] + s[2] for s in z.segments] == g["zigzag_block_read_ends"][str(r)]
        assert all(s[2] == 2 for s in z.segments)  # two tokens per block
        it = plans.plan_interleave(C, r, L)
        assert it.tok_index.tolist() == g["interleave_tok_index"][str(r)]


def test_consecutive_pair_counts_printed():
    # Long Context 2.2: 16-token prompt on 4 GPUs split consecutively:
    # the last GPU reads 58 pairs, the first 10 (diagonal included).
    counts = []
    for (b, e) in plans.contiguous_shards(16, 4):
        pl = plans.Plan(np.arange(b, e), np.arange(b, e, dtype=np.int32), np.zeros(e - b, np.int32))
        counts.append(plans.causal_pairs(pl))
    assert counts[0] == 10 and counts[-1] == 58
    assert counts == [10, 26, 42, 58]


def test_zigzag_balance_every_rank_equal():
    # Long Context 2.3: block b costs b + 1/2 units, every rank totals 2C units,
    # "every pair costs 8 units" for C = 4.
    for C in range(1, 9):
        B = 5
        L = 2 * C * B
        pairs = [plans.causal_pairs(plans.plan_zigzag(C, r, [L])) for r in range(C)]
        assert len(set(pairs)) == 1
        # all ranks together read the whole triangle of an L-token prompt
        assert sum(pairs) == L * (L + 1) // 2
        # exact closed form with prefix P: 2BP + 2C B^2 + B, independent of r
        for P in (0, 3, 17):
            for r in range(C):
                got = plans.causal_pairs(plans.plan_zigzag(C, r, [L], [P]))
                assert got == 2 * B * P + 2 * C * B * B + B


def test_zigzag_units_2C():
    # block b (of size B) reads b blocks before it plus half of itself: (b + 1/2) B^2
    # pairs up to the B/2 diagonal term; rank r totals 2C B^2 + B.
    C, B = 4, 64
    for r in range(C):
        pairs = plans.causal_pairs(plans.plan_zigzag(C, r, [2 * C * B]))
        assert abs(pairs / (B * B) - 2 * C) < 1.0 / B + 1e-12


def test_interleave_skew_about_001_percent():
    # Long Context 2.4: 128,000 tokens on 8 GPUs, the busiest does about 0.01% more work.
    T, C = 128000, 8
    pairs = [plans.causal_pairs(plans.plan_interleave(C, r, [T])) for r in range(C)]
    skew = (max(pairs) - min(pairs)) / min(pairs)
    assert 0.5e-4 < skew < 1.5e-4
    assert pairs == sorted(pairs)  # rank r reads one more token per query than rank r-1


def test_interleave_slice_order_matches_view():
    # Long Context 2.4: tokens.view(-1, C, h)[:, r] when C divides T
    T, C = 48, 4
    toks = np.arange(T)
    for r in range(C):
        want = toks.reshape(-1, C)[:, r]
        assert np.array_equal(plans.plan_interleave(C, r, [T]).tok_index, want)


def test_zigzag_remainder_to_early_blocks():
    blocks = plans.zigzag_blocks(19, 4)
    assert [n for _, n in blocks] == [3, 3, 3, 2, 2, 2, 2, 2]
    assert [s for s, _ in blocks] == [0, 3, 6, 9, 11, 13, 15, 17]
    n_local = [plans.plan_zigzag(4, r, [19]).n_local for r in range(4)]
    assert n_local == [5, 5, 5, 4]
    assert plans.plan_zigzag(4, 0, [19]).n_padded == 5


def _check_plan_consistency(p, new_len, prefix_len):
    cu_new = np.concatenate([[0], np.cumsum(new_len)])
    cu_kv = np.concatenate([[0], np.cumsum(np.array(new_len) + np.array(prefix_len))])
    seen = np.zeros(p.n_local, dtype=int)
    for (req, r0, n, pos0, stride, kv0) in p.segments:
        assert n >= 1
        assert kv0 == cu_kv[req]
        for i in range(n):
            row = r0 + i
            seen[row] += 1
            assert p.req_id[row] == req
            assert p.pos_id[row] == pos0 + i * stride
            # position = prefix + offset of the flattened new token inside its request
            assert p.pos_id[row] == prefix_len[req] + (p.tok_index[row] - cu_new[req])
            assert 0 <= p.tok_index[row] - cu_new[req] < new_len[req]
    assert np.all(seen == 1)


@pytest.mark.parametrize("strategy", ["zigzag", "interleave"])
def test_exhaustive_ownership_small_grid(strategy):
    fn = plans.plan_zigzag if strategy == "zigzag" else plans.plan_interleave
    rng = np.random.default_rng(11)
    cases = [[0], [1], [2], [7], [16], [5, 3], [0, 4, 0], [1, 1, 1, 1, 1]]
    for _ in range(40):
        n = int(rng.integers(1, 6))
        cases.append([int(x) for x in rng.integers(0, 41, size=n)])
    for new_len in cases:
        for prefix_len in ([0] * len(new_len), [int(x) for x in rng.integers(0, 6, size=len(new_len))]):
            T = sum(new_len)
            for C in range(1, 17):
                owners = np.zeros(T, dtype=int)
                sizes = []
                for r in range(C):
                    p = fn(C, r, new_len, prefix_len)
                    _check_plan_consistency(p, new_len, prefix_len)
                    owners[p.tok_index] += 1
                    sizes.append(p.n_local)
                    if strategy == "interleave":
                        assert np.all(np.diff(p.tok_index) == C)
                # every new token owned by exactly one rank; union = all tokens
                assert np.all(owners == 1)
                if strategy == "interleave":
                    assert max(sizes) == -(-T // C) or T == 0
                else:
                    assert fn(C, 0, new_len, prefix_len).n_padded == max(sizes)


def test_contiguous_shards_cover():
    for L, C in itertools.product([0, 1, 5, 16, 4096, 131072, 1001], [1, 2, 3, 4, 8]):
        sh = plans.contiguous_shards(L, C)
        assert sh[0][0] == 0 and sh[-1][1] == L
        assert all(a[1] == b[0] for a, b in zip(sh, sh[1:]))
        lens = [e - b for b, e in sh]
        assert max(lens) - min(lens) <= 1 and lens == sorted(lens, reverse=True)


def test_workload_shapes():
    # zigzag, 16384 tokens, C=4, rank 1: blocks 1 and 6 of 2048 tokens
    p = plans.plan_zigzag(4, 1, [16384])
    assert p.n_local == 4096
    assert [(s[3], s[3] + s[2]) for s in p.segments] == [(2048, 4096), (12288, 14336)]
    # MLA zigzag, 131072 new tokens after a 32768 prefix, C=8, rank 0: blocks 0 and 15
    p = plans.plan_zigzag(8, 0, [131072], [32768])
    assert p.n_local == 16384
    assert [(s[3], s[3] + s[2]) for s in p.segments] == [(32768, 40960), (155648, 163840)]
    assert p.tok_index[0] == 0 and p.tok_index[-1] == 131071
    assert plans.causal_pairs(p) == 1610620928
