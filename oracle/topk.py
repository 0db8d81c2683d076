"""Exact distributed top-k selection (oracle; test use only).

What is computed -- "DeepSeek-V4 Attention Inference Systems" notes, 5.2:
with the sparse-attention index split across ranks, every rank keeps the
best k of its own entries as (score, global id) pairs, the at most P x k
candidates are merged into the exact global top k, the selected ids go to
the ranks that own them, and each owner attends its share (the partial
states then combine exactly). The union of the local top-k lists contains
the global top k, so the merge is exact. *How GPUs Share a Long Context*,
4.1 (Figure 11): a rank that sees only its own index entries can keep an
entry that loses globally, so the ranks exchange their best candidates.

Order used everywhere (the pages ask for deterministic ties and leave the
rule open; reading taken): higher score first; equal scores (-0 equals +0)
by lower global id; NaN below every number. Every rank must use this same
global-id rule for the union to contain the global top k.

Output order (one of several valid orders, fixed so results compare
exactly): the selected candidates in candidate order -- ascending local row
for a rank's own list, rank-major (then the rank's list order) for the
merge, so each owner's selections are one contiguous run.

Pins (``tests/test_oracle_topk.py``): merge of the local lists = the direct
global top k on brute-force grids with many ties; an example built to show
the Figure 11 effect; closed forms (k >= n, k = 1, all-equal scores); a
planted local tie-break by local row breaks exactness and is detected.
"""

import numpy as np


def order(scores, ids):
    """Candidate positions sorted best first by (score desc, id asc), NaN last."""
    s = np.asarray(scores, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    nan = np.isnan(s)
    key = np.where(nan, 0.0, -s)         # ascending key = descending score
    key = np.where(key == 0, 0.0, key)   # -0 and +0 are equal scores
    return np.lexsort((ids, key, nan))   # NaN after every number


def select(scores, ids, k):
    """Positions (ascending, i.e. candidate order) of the best min(k, n)."""
    best = order(scores, ids)[:max(0, min(int(k), len(ids)))]
    return np.sort(best)


def local_topk(scores, n_valid, k, id_base, id_stride):
    """One rank's list for one query: candidates are local rows
    0..n_valid-1 with global ids id_base + row * id_stride.
    Returns (scores, ids, rows) of the selection in ascending row order."""
    rows = np.arange(int(n_valid))
    s = np.asarray(scores, dtype=np.float64)[:int(n_valid)]
    ids = int(id_base) + rows * int(id_stride)
    sel = select(s, ids, k)
    return s[sel], ids[sel], rows[sel]


def merge_topk(lists, k):
    """Merge the ranks' lists for one query. ``lists[p] = (scores, ids,
    rows)`` of rank p. Returns (ids of the global top k in rank-major
    candidate order, per-rank local rows of the selected entries)."""
    s = np.concatenate([np.asarray(l[0], np.float64) for l in lists]) if lists else np.zeros(0)
    ids = np.concatenate([np.asarray(l[1], np.int64) for l in lists]) if lists else np.zeros(0, np.int64)
    src = np.concatenate([np.full(len(l[1]), p) for p, l in enumerate(lists)]) if lists else np.zeros(0, int)
    rows = np.concatenate([np.asarray(l[2], np.int64) for l in lists]) if lists else np.zeros(0, np.int64)
    sel = select(s, ids, k)
    owner_rows = [rows[sel][src[sel] == p] for p in range(len(lists))]
    return ids[sel], owner_rows


def global_topk(scores, k):
    """Direct top k over all entries of one query (global id = index)."""
    s = np.asarray(scores, dtype=np.float64)
    return select(s, np.arange(len(s)), k)
