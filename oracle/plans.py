"""Shard plans for prefill and decode context parallelism (oracle; test use only).

What a plan says, for one rank of a CP group of size C:

* which of the batch's newly extended tokens are this rank's queries
  (``tok_index``: index into the batch's new tokens, flattened request by
  request), in the rank's local row order;
* each local row's original position inside its request, the cached prefix
  included (``pos_id``), and its request (``req_id``);
* segments: maximal runs of local rows of one request whose positions step by
  a constant (``pos0 + i * pos_stride``). A row at position p reads keys
  0..p of its request (diagonal included), which in the packed key/value
  layout are rows ``kv_row0 .. kv_row0 + p`` where request j starts at
  ``kv_row0 = sum_{j' < j} (prefix_j' + new_j')``.

Zigzag -- SGLang prefill CP, "Zigzag strategy"; *Long Context* 2.3: each
request's new tokens are cut into 2C contiguous blocks, rank r takes blocks r
and 2C-1-r, the split restarts for every request; when the length does not
divide, the early blocks take the remainder. Reading taken: the first
``L mod 2C`` blocks get one extra token each. Rows are request-major, the
early block before the late one. Each non-empty block is one segment with
stride 1; the position where the block's key reads stop (*Long Context*
2.3) is ``pos0 + q_len``. A cached prefix is not split; both blocks read it
(*Long Context* 2.3, last paragraph; the docs' metadata paragraph).

Interleave -- SGLang prefill CP, "Interleave strategy"; *Long Context* 2.4:
rank r owns flattened new-token indices r, r+C, r+2C, ... across the whole
batch, without reset at request boundaries; position ids keep their original
values. Rows ascend in flattened index (the one-line slice of 2.4 fixes this
order). One segment per request that owns a row, stride C.

Contiguous decode shards -- vLLM "Decode Context Parallelism" post, section 4:
GPU c holds a contiguous chunk of token positions. Reading taken for a
length that does not divide: the early shards take the remainder.

``n_padded``: the docs say buffers are padded; the plan reports the largest
local row count over the ranks (zigzag) or ceil(T / C) (interleave).

Pins (``tests/test_oracle_plans.py``): the interleave ownership example of
lengths 5 and 3 printed in the SGLang docs; the pair counts of *Long Context*
2.2 (58 and 10); the 2C-unit balance of 2.3 and its closed form; the 0.01%
interleave skew of 2.4; exhaustive ownership/union checks on small grids.
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Plan:
    tok_index: np.ndarray  # int64 [n_local]
    pos_id: np.ndarray  # int32 [n_local]
    req_id: np.ndarray  # int32 [n_local]
    segments: list = field(default_factory=list)  # (req, q_row0, q_len, pos0, pos_stride, kv_row0)
    n_padded: int = 0

    @property
    def n_local(self):
        return int(self.tok_index.shape[0])

    @property
    def n_seg(self):
        return len(self.segments)


def _lengths(new_len, prefix_len):
    new_len = [int(x) for x in new_len]
    if prefix_len is None:
        prefix_len = [0] * len(new_len)
    prefix_len = [int(x) for x in prefix_len]
    if len(prefix_len) != len(new_len):
        raise ValueError("prefix_len and new_len differ in length")
    if any(x < 0 for x in new_len) or any(x < 0 for x in prefix_len):
        raise ValueError("negative length")
    return new_len, prefix_len


def zigzag_blocks(L, C):
    """The 2C contiguous blocks of an L-token request: list of (start, len).
    Early blocks take the remainder, one extra token each."""
    nb = 2 * C
    base, rem = divmod(L, nb)
    out, start = [], 0
    for b in range(nb):
        n = base + (1 if b < rem else 0)
        out.append((start, n))
        start += n
    return out


def _zigzag_rows(C, rank, new_len, prefix_len):
    tok, pos, req, segs = [], [], [], []
    cu_new = 0
    cu_kv = 0
    for j, (L, P) in enumerate(zip(new_len, prefix_len)):
        blocks = zigzag_blocks(L, C)
        for b in (rank, 2 * C - 1 - rank):
            start, n = blocks[b]
            if n == 0:
                continue
            segs.append((j, len(tok), n, P + start, 1, cu_kv))
            for i in range(n):
                tok.append(cu_new + start + i)
                pos.append(P + start + i)
                req.append(j)
        cu_new += L
        cu_kv += P + L
    return tok, pos, req, segs


def plan_zigzag(C, rank, new_len, prefix_len=None):
    if C < 1 or not (0 <= rank < C):
        raise ValueError("bad C or rank")
    new_len, prefix_len = _lengths(new_len, prefix_len)
    tok, pos, req, segs = _zigzag_rows(C, rank, new_len, prefix_len)
    n_padded = max(len(_zigzag_rows(C, r, new_len, prefix_len)[0]) for r in range(C))
    return Plan(np.array(tok, dtype=np.int64), np.array(pos, dtype=np.int32),
                np.array(req, dtype=np.int32), segs, n_padded)


def plan_interleave(C, rank, new_len, prefix_len=None):
    if C < 1 or not (0 <= rank < C):
        raise ValueError("bad C or rank")
    new_len, prefix_len = _lengths(new_len, prefix_len)
    T = sum(new_len)
    cu_new = np.concatenate([[0], np.cumsum(new_len)]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum(np.array(new_len) + np.array(prefix_len))]).astype(np.int64) \
        if new_len else np.zeros(1, dtype=np.int64)
    g = np.arange(rank, T, C, dtype=np.int64)
    # request of flattened index g: the last j with cu_new[j] <= g
    j = np.searchsorted(cu_new, g, side="right") - 1
    pos = np.array(prefix_len, dtype=np.int64)[j] + (g - cu_new[j]) if len(g) else np.zeros(0, np.int64)
    segs = []
    row = 0
    for jj in range(len(new_len)):
        rows = np.nonzero(j == jj)[0]
        if len(rows) == 0:
            continue
        assert rows[0] == row
        segs.append((jj, int(rows[0]), int(len(rows)), int(pos[rows[0]]), C, int(cu_kv[jj])))
        row += len(rows)
    n_padded = -(-T // C)
    return Plan(g, pos.astype(np.int32), j.astype(np.int32), segs, n_padded)


def contiguous_shards(L, C):
    """Decode CP with contiguous token chunks: shard c covers [begin_c, end_c).
    Early shards take the remainder."""
    if C < 1 or L < 0:
        raise ValueError("bad C or L")
    base, rem = divmod(L, C)
    out, s = [], 0
    for c in range(C):
        n = base + (1 if c < rem else 0)
        out.append((s, s + n))
        s += n
    return out


def causal_pairs(plan):
    """(query, key) pairs a rank's queries read, diagonal included: a query at
    position p reads p + 1 keys (*Long Context* 1.1 and 2.2)."""
    return int(np.sum(plan.pos_id.astype(np.int64) + 1))


# ---------------------------------------------------------------- round robin
#
# Decode CP with round-robin storage -- *Long Context* 3.1: with C GPUs,
# token (slot) p of a request is stored on GPU p mod C, as row p // C of
# that GPU's cache (the page's example: slot 9 with C = 4 is GPU 1, row 2); the
# "DeepSeek-V4 Attention Inference Systems" notes, section 5, write the same
# owner rule as owner(j) = j mod P, and 5.3 adds that entries replicated on
# every rank (a local window, attention sinks) must add their probability
# mass once: only a designated rank includes them.
#
# Local cache layout taken here (the pages leave it open): a rank's cache
# for one request holds the n_repl replicated entries in rows [0, n_repl)
# and its own tokens rank, rank + C, rank + 2C, ... in rows n_repl,
# n_repl + 1, ... (ascending slot), so a new token is appended at the end.
# The rank's decode range is rows [0, n_repl + n_own) on the designated
# rank and [n_repl, n_repl + n_own) on the others.

def round_robin_slot(slot, C):
    """(gpu, row) of a slot: gpu = slot mod C, row = slot // C."""
    if C < 1 or slot < 0:
        raise ValueError("bad slot or C")
    return slot % C, slot // C


def round_robin_own_tokens(L, C, rank):
    """The slots of an L-token request that rank `rank` stores, in local
    row order."""
    if C < 1 or not (0 <= rank < C) or L < 0:
        raise ValueError("bad L, C or rank")
    return list(range(rank, L, C))


def plan_round_robin(C, rank, ctx_len, n_repl=0, repl_rank=0):
    """Decode range of rank `rank` in its local cache, per request:
    (kv_begin [n_req], kv_end [n_req]) as int32 arrays."""
    if C < 1 or not (0 <= rank < C) or n_repl < 0 or not (0 <= repl_rank < C):
        raise ValueError("bad C, rank or replication")
    beg, end = [], []
    for L in ctx_len:
        if L < 0:
            raise ValueError("negative length")
        n_own = len(round_robin_own_tokens(int(L), C, rank))
        beg.append(0 if rank == repl_rank else n_repl)
        end.append(n_repl + n_own)
    return np.array(beg, np.int32), np.array(end, np.int32)


# ------------------------------------------------------- multi-query decode
#
# Speculative / MTP decode under decode CP (*Long Context* section 9 names
# it; the DeepSeek-V4 notes, section 11, sweep the query/spec width 1, 2, 4,
# 8): a request carries Q query rows, its last Q slots, whose keys are
# already in the cache. Attention is causal (*Long Context* 1.1), so row k at
# slot p = L - Q + k reads slots 0..p. The reading taken here (the pages do
# not spell it out): on a rank, row k reads the part of 0..p that the rank
# stores; replicated rows of a round-robin cache are seen by every row.

def plan_multi_query(layout, C, rank, ctx_len, Q, n_repl=0, repl_rank=0):
    """Per-row decode ranges of rank `rank` in its local cache:
    (kv_begin int32 [n_req], kv_end int32 [n_req * Q]).

    layout "contiguous": the local cache holds the rank's chunk of
    contiguous_shards(L, C) from row 0. layout "round_robin": local cache as
    in plan_round_robin. Rows are found by listing the slots the rank stores
    and counting those at or below each query slot."""
    if Q < 1 or C < 1 or not (0 <= rank < C):
        raise ValueError("bad Q, C or rank")
    if layout == "contiguous" and (n_repl or repl_rank):
        raise ValueError("contiguous shards take no replicated rows")
    beg, end = [], []
    for L in ctx_len:
        L = int(L)
        if L < Q:
            raise ValueError("a request stores fewer than Q slots")
        if layout == "contiguous":
            s0, s1 = contiguous_shards(L, C)[rank]
            stored = list(range(s0, s1))     # local row i holds slot s0 + i
            first = 0
        elif layout == "round_robin":
            stored = round_robin_own_tokens(L, C, rank)   # local row n_repl + i
            first = n_repl
            beg_b = 0 if rank == repl_rank else n_repl
        else:
            raise ValueError("unknown layout")
        beg.append(0 if layout == "contiguous" else beg_b)
        for k in range(Q):
            p = L - Q + k
            end.append(first + sum(1 for t in stored if t <= p))
    return np.array(beg, np.int32), np.array(end, np.int32)
