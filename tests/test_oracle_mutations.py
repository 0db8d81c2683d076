"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies the oracle, the input generators and the oracle's pin tests
into a scratch directory, plants one mistake in the copied oracle source (a
one-place text edit), and runs those pins there in a child pytest. The case
passes only if the child reports failing tests (exit status 1): a mistake
that every pin lets through would mean the pins do not cover that part of
the oracle. The unmodified copy must pass (exit status 0).

The mistakes are the plausible ones for each part: a mask, index, sign,
bias or pairing written slightly wrong.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PLANS = ["tests/test_oracle_plans.py", "tests/test_oracle_round_robin.py", "tests/test_oracle_multi_query.py"]
ATT = ["tests/test_oracle_attention.py"]
FMT = ["tests/test_oracle_formats.py"]
SPARSE = ["tests/test_oracle_sparse.py"]
TOPK = ["tests/test_oracle_topk.py"]
MQ = ["tests/test_oracle_multi_query.py"]
RR = ["tests/test_oracle_round_robin.py"]
PAGED = ["tests/test_oracle_paged.py"]

# (name, oracle file, text to replace, replacement, pin files to run)
MUTATIONS = [
    ("paged row offset from the block index", "attention.py",
     "return pages * page_size + t % page_size", "return pages * page_size + t // page_size", PAGED),
    ("paged block from the offset", "attention.py",
     "pages = np.asarray(block_table, dtype=np.int64)[t // page_size]",
     "pages = np.asarray(block_table, dtype=np.int64)[(t // page_size) % len(block_table)][::-1]", PAGED),
    ("paged invalid entry read as the last page", "attention.py",
     "pages = np.where((pages >= 0) & (pages < n_pages), pages, 0)",
     "pages = np.where((pages >= 0) & (pages < n_pages), pages, n_pages - 1)", PAGED),
    ("paged scales read at the logical position", "attention.py",
     "sc = None if kv_scale is None else np.asarray(kv_scale)[rows][None]",
     "sc = None if kv_scale is None else np.asarray(kv_scale)[s0:s1][None]", PAGED),
    ("causal mask drops the diagonal", "attention.py",
     "visible = np.arange(p_hi + 1)[None, :] <= pos[:, None]",
     "visible = np.arange(p_hi + 1)[None, :] < pos[:, None]", ATT),
    ("prefill GQA heads taken round robin", "attention.py",
     "qh = qr[:, hk * G:(hk + 1) * G, :].reshape(R * G, Dqk)",
     "qh = qr[:, hk::Hkv, :].reshape(R * G, Dqk)", ATT),
    ("decode GQA heads taken round robin", "attention.py",
     "o, lse = attend(q[b, h], keys[:, h // G, :], vals[:, h // G, :], scale)",
     "o, lse = attend(q[b, h], keys[:, h % Hkv, :], vals[:, h % Hkv, :], scale)", ATT),
    ("softmax scale divides", "attention.py",
     "s = (scale * (qh @ kh.T)).reshape(R, G, p_hi + 1)",
     "s = ((qh @ kh.T) / scale).reshape(R, G, p_hi + 1)", ATT),
    ("decode score without the scale", "attention.py",
     "s = scale * (keys @ q)\n    m = np.max(s)\n    e = np.exp(s - m)\n    ell = np.sum(e)\n    return (e @ values)",
     "s = (keys @ q)\n    m = np.max(s)\n    e = np.exp(s - m)\n    ell = np.sum(e)\n    return (e @ values)", ATT),
    ("no max shift inside the exponential", "attention.py",
     "    m = np.max(s)\n    e = np.exp(s - m)\n    ell = np.sum(e)\n    return (e @ values) / ell, m + np.log(ell)",
     "    m = np.max(s)\n    e = np.exp(s)\n    ell = np.sum(e)\n    return (e @ values) / ell, m + np.log(ell)", ATT),
    ("merge weight sign flipped", "attention.py",
     "np.exp(lse_parts - lse_safe[None])", "np.exp(lse_safe[None] - lse_parts)", ATT),
    ("merge LSE without the log of the total", "attention.py",
     "lse = np.where(np.isfinite(m), m_safe + np.log(tot), _NEG_INF)",
     "lse = np.where(np.isfinite(m), m_safe + tot - 1.0, _NEG_INF)", ATT),
    ("MLA value is the latent's tail", "attention.py",
     "vals = keys[..., :Dv] if v is None else _f64(v[kv0:kv0 + p_hi + 1], decode)",
     "vals = keys[..., -Dv:] if v is None else _f64(v[kv0:kv0 + p_hi + 1], decode)", ATT),
    ("FP8 per-token scale left out", "attention.py",
     "            keys = keys * tok_scale\n", "            keys = keys\n", ATT),
    ("FP8 per-token scale left out of GQA values", "attention.py",
     "            vals = vals * tok_scale\n", "            vals = vals\n", ATT),
    ("sparse list: last cache row treated as padding", "attention.py",
     "if 0 <= int(t) < Lmax]", "if 0 <= int(t) < Lmax - 1]", SPARSE),
    ("sparse list: entries deduplicated", "attention.py",
     "sel = [int(t) for t in idx[n, :k] if 0 <= int(t) < Lmax]",
     "sel = sorted({int(t) for t in idx[n, :k] if 0 <= int(t) < Lmax})", SPARSE),
    ("multi-query row slot off by one", "plans.py",
     "            p = L - Q + k\n", "            p = L - Q + k - 1\n", MQ),
    ("E4M3 exponent bias 8", "formats.py",
     "normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)",
     "normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 8.0)", FMT),
    ("E4M3 subnormal exponent", "formats.py",
     "subnormal = (m / 8.0) * np.exp2(1.0 - 7.0)", "subnormal = (m / 8.0) * np.exp2(0.0 - 7.0)", FMT),
    ("E4M3 NaN code read as a number", "formats.py",
     "val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)", "val = val", FMT),
    ("zigzag pairs block r with r + C", "plans.py",
     "for b in (rank, 2 * C - 1 - rank):", "for b in (rank, rank + C):", PLANS),
    ("zigzag remainder to the late blocks", "plans.py",
     "n = base + (1 if b < rem else 0)\n        out.append((start, n))",
     "n = base + (1 if b >= nb - rem else 0)\n        out.append((start, n))", PLANS),
    ("zigzag positions drop the cached prefix", "plans.py",
     "pos.append(P + start + i)", "pos.append(start + i)", PLANS + ATT),
    ("packed kv row skips the prefix", "plans.py", "cu_kv += P + L", "cu_kv += L", ATT),
    ("interleave starts at rank + 1", "plans.py",
     "g = np.arange(rank, T, C, dtype=np.int64)", "g = np.arange(rank + 1, T, C, dtype=np.int64)", PLANS),
    ("interleave segment stride 1", "plans.py",
     "segs.append((jj, int(rows[0]), int(len(rows)), int(pos[rows[0]]), C, int(cu_kv[jj])))",
     "segs.append((jj, int(rows[0]), int(len(rows)), int(pos[rows[0]]), 1, int(cu_kv[jj])))", PLANS + ATT),
    ("decode shards: remainder to the late shards", "plans.py",
     "n = base + (1 if c < rem else 0)\n        out.append((s, s + n))",
     "n = base + (1 if c >= C - rem else 0)\n        out.append((s, s + n))", PLANS),
    ("round robin: row and rank swapped", "plans.py",
     "return slot % C, slot // C", "return slot // C, slot % C", RR),
    ("round robin: replicated rows counted on every rank", "plans.py",
     "beg.append(0 if rank == repl_rank else n_repl)", "beg.append(0)", RR),
    ("top-k ties: higher id first", "topk.py",
     "return np.lexsort((ids, key, nan))", "return np.lexsort((-ids, key, nan))", TOPK),
    ("top-k: -0 below +0", "topk.py",
     "key = np.where(key == 0, 0.0, key)   # -0 and +0 are equal scores",
     "key = np.where(key == 0, np.copysign(1e-300, key), key)", TOPK),
]


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(dst, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for f in os.listdir(os.path.join(ROOT, "tests")):
        if f in ("__init__.py", "conftest.py", "helpers.py") or (f.startswith("test_oracle_") and f.endswith(".py")
                                                                 and f != os.path.basename(__file__)):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))


def _run_pins(dst, files):
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *files],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-3000:]


def test_unmodified_copy_passes(tmp_path):
    _copy_tree(str(tmp_path))
    files = sorted({f for m in MUTATIONS for f in m[4]})
    rc, out = _run_pins(str(tmp_path), files)
    assert rc == 0, out


@pytest.mark.parametrize("name,fname,old,new,files", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, fname, old, new, files):
    _copy_tree(str(tmp_path))
    path = os.path.join(str(tmp_path), "oracle", fname)
    src = open(path).read()
    assert src.count(old) == 1, f"the text to mutate must occur exactly once in oracle/{fname}"
    open(path, "w").write(src.replace(old, new))
    rc, out = _run_pins(str(tmp_path), files)
    assert rc == 1, f"planted mistake '{name}' was not caught by the pins (pytest exit {rc}):\n{out}"
