"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, checked on outputs the oracle computes one by one (sampled
requests / rows, always including the first and last row of every segment)."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as att
from oracle import formats, plans
from tests import helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


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


def _sample_rows(plan, n_extra, seed):
    rows = set()
    for s in plan.segments:
        r0, n = int(s["q_row0"]), int(s["q_len"])
        rows.update([r0, r0 + n - 1, r0 + n // 2])
    rng = synth.rng(seed, 9)
    rows.update(int(x) for x in rng.integers(0, plan.n_local, size=n_extra))
    return sorted(rows)


@pytest.fixture(scope="module")
def mla_decode_inputs():
    c = synth.workload("mla_decode_131k")
    print("[mla decode] generating inputs", flush=True)
    q = synth.bf16_normal(3, 1, (c["B"], c["Hq"], c["Dqk"]))
    bits, codes, scales = synth.latent_cache_both(3, 2, c["B"], c["L"], c["Dqk"], c["std"])
    return c, q, bits, codes, scales


@pytest.mark.parametrize("fp8", [False, True])
def test_mla_decode_workload(cpa, mla_decode_inputs, fp8):
    """MLA decode: batch 64, 64 heads, 576/512, 131072-token context per
    request, cut into C=8 contiguous shards run as 8 partial launches on one
    device + one merge; bf16 cache, then FP8 E4M3 with per-token scale."""
    import torch
    c, q, bits, codes, scales = mla_decode_inputs
    B, L, C = c["B"], c["L"], c["C"]
    qd = H.bf16_tensor(q)
    cd = H.u8_tensor(codes) if fp8 else H.bf16_tensor(bits)
    sd = H.f32_tensor(scales) if fp8 else None
    shards = plans.contiguous_shards(L, C)
    # NaN-filled outputs and 0xff-filled workspace: anything left unwritten fails
    po = torch.full((C, B, 64, 512), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((C, B, 64), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((cpa.attn_decode_workspace_size(B, 64, 512, L // C),), 255, dtype=torch.uint8, device="cuda")
    for i, (s0, s1) in enumerate(shards):
        cpa.attn_decode_shard(qd, cd, None, H.i32_tensor(np.full(B, s0)), H.i32_tensor(np.full(B, s1)), s1 - s0,
                              c["scale"], kv_scale=sd, o_part=po[i], lse_part=pl[i], workspace=ws)
    mo, ml = cpa.attn_merge_states(po, pl)
    _sync()
    print(f"[mla decode fp8={fp8}] kernels done; oracle", flush=True)
    q64 = formats.bf16_bits_to_f64(q)
    cache, dec = (codes, formats.e4m3_to_f64) if fp8 else (bits, formats.bf16_bits_to_f64)
    sc = scales if fp8 else None
    # every partial and merged state was written (the buffers started as NaN)
    for t in (po, pl, mo, ml):
        assert bool(torch.isfinite(t).all())
    # merged output against unsharded attention over the whole context, on
    # 12 seeded requests (the first and last always among them)
    reqs = sorted({0, B - 1} | {int(x) for x in synth.rng(3, 9).choice(B, size=10, replace=False)})
    ro, rl = att.decode_shard(q64, cache, [0] * B, [L] * B, c["scale"], dv=512, decode=dec, kv_scale=sc, batch=reqs)
    e = H.check_lowp(H.host(mo)[reqs], H.host(ml)[reqs], ro[reqs], rl[reqs], f"MLA decode merged fp8={fp8}")
    print(f"MLA decode fp8={fp8} merged errors on requests {reqs} (O abs, LSE abs, O row-rel):", e)
    # two shards' partial states against the shard oracle
    for si, b in ((5, 11), (0, 50)):
        s0, s1 = shards[si]
        ro, rl = att.decode_shard(q64, cache, [s0] * B, [s1] * B, c["scale"], dv=512, decode=dec, kv_scale=sc,
                                  batch=[b])
        e = H.check_lowp(H.host(po[si])[[b]], H.host(pl[si])[[b]], ro[[b]], rl[[b]], f"MLA decode shard {si}")
        print(f"MLA decode fp8={fp8} shard {si} request {b} errors:", e)


@pytest.mark.parametrize("fp8", [False, True])
def test_mla_decode_paged_workload(cpa, mla_decode_inputs, fp8):
    """The MLA decode workload over a paged cache: the same rows in 64-token
    pages of one pool, placed by a seeded random block table; the 8 shard
    launches must give results bit-identical to the contiguous launches
    (whose parity with the oracle test_mla_decode_workload checks)."""
    import torch
    c, q, bits, codes, scales = mla_decode_inputs
    B, L, C = c["B"], c["L"], c["C"]
    ps = 64
    nb = L // ps
    qd = H.bf16_tensor(q)
    cd = H.u8_tensor(codes) if fp8 else H.bf16_tensor(bits)
    sd = H.f32_tensor(scales) if fp8 else None
    table = H.i32_tensor(synth.page_table(3, 9, B, nb, B * nb))
    dst = table.reshape(-1).long()
    pool = torch.empty((B * nb, ps) + tuple(cd.shape[2:]), dtype=cd.dtype, device=cd.device)
    pool[dst] = cd.reshape((B * nb, ps) + tuple(cd.shape[2:]))
    pool = pool.reshape((B * L,) + tuple(cd.shape[2:]))
    spool = None
    if fp8:
        spool = torch.empty((B * nb, ps), dtype=torch.float32, device=cd.device)
        spool[dst] = sd.reshape(B * nb, ps)
        spool = spool.reshape(-1)
    shards = plans.contiguous_shards(L, C)
    for i, (s0, s1) in enumerate(shards):
        beg, end = H.i32_tensor(np.full(B, s0)), H.i32_tensor(np.full(B, s1))
        o1, l1 = cpa.attn_decode_shard_paged(qd, pool, None, table, ps, beg, end, s1 - s0, c["scale"], kv_scale=spool)
        o2, l2 = cpa.attn_decode_shard(qd, cd, None, beg, end, s1 - s0, c["scale"], kv_scale=sd)
        _sync()
        assert bool(torch.isfinite(o1).all()) and bool(torch.isfinite(l1).all())
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"shard {i}: paged differs from contiguous"
    print(f"MLA decode paged fp8={fp8}: 8 shards bit-identical to the contiguous cache", flush=True)


def test_mla_prefill_zigzag_workload(cpa):
    """MLA zigzag prefill: 64 heads, 576/512, 131072 new tokens after a
    32768-token cached prefix, C=8 (16 blocks of 8192), rank 0's share."""
    import torch
    c = synth.workload("mla_zigzag_prefill_prefix32k")
    plan = cpa.cp_plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    T = sum(c["new_len"]) + sum(c["prefix_len"])
    print("[mla prefill] generating inputs", flush=True)
    qb = synth.bf16_normal(4, 1, (plan.n_local, 64, 576), chunk=256)
    lb = synth.bf16_normal(4, 2, (T, 1, 576))
    o, l = cpa.attn_prefill_shard(H.bf16_tensor(qb), H.bf16_tensor(lb), None, plan.segments, c["scale"])
    _sync()
    rows = _sample_rows(plan, 10, 4)
    ref = plans.plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    lat64 = formats.bf16_bits_to_f64(lb)
    print(f"[mla prefill] kernel done; oracle on {len(rows)} rows", flush=True)
    ro, rl = att.prefill_shard(formats.bf16_bits_to_f64(qb[rows]), lat64, _remap(ref.segments, rows),
                               c["scale"], dv=512, rows=list(range(len(rows))))
    e = H.check_lowp(H.host(o)[rows], H.host(l)[rows], ro, rl, "MLA zigzag workload")
    print("MLA zigzag workload errors (O abs, LSE abs, O row-rel):", e)
    # every row was written (the outputs started as NaN)
    assert bool(torch.isfinite(l).all()) and bool(torch.isfinite(o).all())


def _remap(segments, rows):
    """Segments for a compacted copy of the sampled rows: row i of the copy is
    local row rows[i], one single-row segment each."""
    out = []
    for i, r in enumerate(rows):
        for (req, r0, n, pos0, stride, kv0) in segments:
            if r0 <= r < r0 + n:
                out.append((req, i, 1, pos0 + (r - r0) * stride, 1, kv0))
    return out


def test_interleave_ragged_workload(cpa):
    """Interleave prefill on a ragged batch: 16 agentic-length requests
    (T = 728,040), C=4, rank 2; causal GQA 32/8, d=128, bf16."""
    import torch
    c = synth.workload("gqa_interleave_prefill_agentic16")
    plan = cpa.cp_plan_interleave(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    assert plan.n_local == 182010
    T = sum(c["new_len"])
    print("[interleave] generating inputs", flush=True)
    qb = synth.bf16_normal(5, 1, (plan.n_local, 32, 128))
    kb = synth.bf16_normal(5, 2, (T, 8, 128))
    vb = synth.bf16_normal(5, 3, (T, 8, 128))
    o, l = cpa.attn_prefill_shard(H.bf16_tensor(qb), H.bf16_tensor(kb), H.bf16_tensor(vb), plan.segments, c["scale"])
    _sync()
    rows = _sample_rows(plan, 16, 5)
    ref = plans.plan_interleave(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    segs = _remap(ref.segments, rows)
    print(f"[interleave] kernel done; oracle on {len(rows)} rows", flush=True)
    ro, rl = att.prefill_shard(qb[rows].copy(), kb, segs, c["scale"], v=vb, rows=list(range(len(rows))),
                               decode=formats.bf16_bits_to_f64)
    e = H.check_lowp(H.host(o)[rows], H.host(l)[rows], ro, rl, "interleave workload")
    print("interleave workload errors (O abs, LSE abs, O row-rel):", e)
    assert bool(torch.isfinite(l).all()) and bool(torch.isfinite(o).all())
