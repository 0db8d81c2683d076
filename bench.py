#!/usr/bin/env python3
"""Benchmark of the context-parallel attention shard path on one MI355X.

Headline (the JSON line's ``value``): the zigzag prefill shard -- causal GQA,
32 query heads on 8 kv heads, head dim 128, bf16, a 16384-token prompt split
for C=4 ranks, rank 1's share (blocks 1 and 6) -- in TFLOP/s of algorithmic
work (unmasked causal pairs, diagonal included, 2 * (Dqk + Dv) flops per
pair and head). A step is the rank's whole hot path for that batch: the
zigzag plan (host planner) and the shard attention launch.

Secondary (``decode`` object): split-KV MLA decode, batch 64, 64 heads,
576/512 latent, 131072-token context cut into C=8 contiguous shards, run as 8
partial launches on one device plus the exact merge; bf16 cache and FP8 E4M3
cache with per-token scale, in GB/s of algorithmic bytes (cache bytes read
once, plus queries, partial outputs/LSEs and the merge). ``decode_gqa``: the
same step for a GQA cache at a serving shape (batch 8, 32/8 heads, d=128,
131072 tokens, C=8), bf16 and FP8; ``decode_gqa_f32_4k``: the fp32 GQA decode of
batch 1, 8/1 heads, 4096 tokens, C=4, with the last-level cache flushed.

Also reported: the dominant kernel's roofline (live HIP-event timing on the
launch stream); the same prefill kernel with the 256 MB last-level cache
flushed before each launch (its inputs fit in it); and the float64 CPU oracle
timed on a bounded sample of the same workload on this host. All inputs are
seeded and synthetic.

Warmup: at least --warmup untimed steps per workload, continued until
--warmup-ms of wall time have passed. The GPU's clock takes a few hundred
milliseconds of load to reach its steady state; measured after 3 short steps
the same kernels ran 10-15 % slower than in a sustained loop.
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "split-KV decode GB/s (% HBM peak); zigzag prefill TFLOP/s (% MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic per launch of the dominant kernels, from rocprofv3 --pmc runs of
# this script (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled
# by what the same counter read for a plain device copy of known size. A
# figure is reported only while the kernel sources still hash to the digest
# they were measured at; after any change the field is null until re-measured.
TRAFFIC = {
    # profiles/prefill_gqa_zigzag_16k_c4_rank1.md
    "prefill_gqa_kernel": dict(digest="430ae3ec42fd765b", fetch_kib=67611.6, write_kib=33792.3,
                              fetch_scale=1.99994, write_scale=1.0,
                              fetch_bytes=138464403, write_bytes=34603315),
    # profiles/decode_mla_b64_h64_ctx131072_c8.md
    "decode_mla_kernel<bf16>": dict(digest="d9fc94b6f76ea876", fetch_kib=592268.5, write_kib=32833.4,
                                   fetch_scale=1.99994, write_scale=1.0,
                                   fetch_bytes=1212929499, write_bytes=33621402),
    # profiles/decode_gqa_b8_h32_kv8_ctx131072_c8.md
    "decode_gqa_kernel<bf16>": dict(digest="99ed0efbebf30435", fetch_kib=262291.3, write_kib=520.0,
                                   fetch_scale=1.99994, write_scale=1.0,
                                   fetch_bytes=537156467, write_bytes=532480),
}


def _src_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "context_attention_long_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill_gqa_kernel": ("prefill.hip", "lds_dma.h"),
    "decode_mla_kernel<bf16>": ("decode_mla.hip", "mla_core.h", "mla_ws.h", "lds_dma.h", "wave_ops.h", "paged.h"),
    "decode_gqa_kernel<bf16>": ("decode_gqa.hip", "lds_dma.h", "wave_ops.h", "paged.h"),
}


def traffic(kernel):
    """(HBM bytes per launch, how they were obtained), or (None, None)."""
    t = TRAFFIC.get(kernel)
    if t is None or t["digest"] != _src_digest(KERNEL_SOURCES[kernel]):
        return None, None
    return t["fetch_bytes"] + t["write_bytes"], {k: v for k, v in t.items() if k != "digest"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _warm(torch, step, warmup, min_ms):
    """At least `warmup` untimed steps, continued until `min_ms` of wall time
    have passed: the GPU's clock needs a few hundred milliseconds of load to
    settle, and a few short steps alone leave it below its steady state.
    Returns the number of warmup steps run."""
    n = 0
    t0 = time.perf_counter()
    while n < warmup or (time.perf_counter() - t0) * 1e3 < min_ms:
        step()
        n += 1
        if n % 4 == 0:  # keep the queue short, so elapsed wall time tracks GPU work
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def bench_prefill(cpa, torch, synth, steps, warmup, warmup_ms):
    c = synth.workload("gqa_zigzag_prefill_16k")
    plan = cpa.cp_plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    T = sum(c["new_len"])
    dev = torch.device("cuda:0")
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q = to_dev(synth.bf16_normal(2, 1, (plan.n_local, c["Hq"], c["Dqk"])))
    k = to_dev(synth.bf16_normal(2, 2, (T, c["Hkv"], c["Dqk"])))
    v = to_dev(synth.bf16_normal(2, 3, (T, c["Hkv"], c["Dv"])))
    out = torch.empty((plan.n_local, c["Hq"], c["Dv"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((plan.n_local, c["Hq"]), dtype=torch.float32, device=dev)
    pairs = int(np.sum(plan.pos_id.astype(np.int64) + 1))
    flops = pairs * c["Hq"] * 2 * (c["Dqk"] + c["Dv"])

    def step(ev=None):
        p = cpa.cp_plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
        if ev is not None:
            ev[0].record()
        cpa.attn_prefill_shard(q, k, v, p.segments, c["scale"], out=out, lse=lse)
        if ev is not None:
            ev[1].record()

    nwarm = _warm(torch, step, warmup, warmup_ms)
    evs = _events(torch, steps)
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = [a.elapsed_time(b) for a, b in evs]
    # The same launch with the last-level cache (256 MB Infinity Cache)
    # flushed first, outside the events: the workload's Q, K and V (101 MB)
    # fit in that cache, so the timed steps above may find them there. Two
    # flushes: a 512 MiB write (it leaves the cache full of dirty lines, whose
    # write-back then competes with the kernel's reads) and a 512 MiB read.
    # Each (flush, launch) loop is warmed like the steps above before it is
    # timed: the clock settles to the new mix of work (the first few hundred
    # milliseconds of flushes ran the launch up to 15 % slower).
    scratch = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    cold_reps = min(steps, 20)
    cold = {}
    for kind in ("write", "read"):
        flush = (lambda i: scratch.fill_(float(i))) if kind == "write" else (lambda i: scratch.sum())
        _warm(torch, lambda: (flush(0), step()), warmup, warmup_ms)
        cevs = _events(torch, cold_reps)
        for i in range(cold_reps):
            flush(i)
            step(cevs[i])
        torch.cuda.synchronize()
        cold[kind] = sorted(a.elapsed_time(b) for a, b in cevs)
    del scratch
    return dict(cfg=c, plan=plan, flops=flops, pairs=pairs, wall=wall, kernel_ms=kms, warmup_steps=nwarm,
                inputs=(q, k, v), cold_ms=cold)


def bench_prefill_workload(cpa, torch, synth, name, steps, warmup, warmup_ms):
    """One more prefill shard workload (mla_zigzag_prefill_prefix32k: MLA
    zigzag with a cached prefix; gqa_interleave_prefill_agentic16: interleave
    over the ragged agentic batch), timed per
    launch with HIP events: algorithmic TFLOP/s."""
    c = synth.workload(name)
    k = c["seed"]
    planner = cpa.cp_plan_zigzag if c["strategy"] == "zigzag" else cpa.cp_plan_interleave
    plan = planner(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    T = sum(c["new_len"]) + sum(c["prefix_len"])
    dev = torch.device("cuda:0")
    to_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q = to_dev(synth.bf16_normal(k, 1, (plan.n_local, c["Hq"], c["Dqk"]), chunk=256))
    kk = to_dev(synth.bf16_normal(k, 2, (T, c["Hkv"], c["Dqk"])))
    v = None if c["Hkv"] == 1 else to_dev(synth.bf16_normal(k, 3, (T, c["Hkv"], c["Dv"])))
    out = torch.empty((plan.n_local, c["Hq"], c["Dv"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((plan.n_local, c["Hq"]), dtype=torch.float32, device=dev)
    # causal pairs per head: each local row attends to positions 0..pos (prefix included)
    pairs = int(np.sum(plan.pos_id.astype(np.int64) + 1))
    flops = pairs * c["Hq"] * 2 * (c["Dqk"] + c["Dv"])
    _warm(torch, lambda: cpa.attn_prefill_shard(q, kk, v, plan.segments, c["scale"], out=out, lse=lse),
          warmup, warmup_ms)
    evs = _events(torch, steps)
    for i in range(steps):
        evs[i][0].record()
        cpa.attn_prefill_shard(q, kk, v, plan.segments, c["scale"], out=out, lse=lse)
        evs[i][1].record()
    torch.cuda.synchronize()
    kms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    del q, kk, v, out, lse
    torch.cuda.empty_cache()
    tf = flops / (kms * 1e-3) / 1e12
    return {"workload": c["name"], "local_rows": plan.n_local, "algorithmic_tflop": round(flops / 1e12, 3),
            "kernel_ms": round(kms, 3), "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def bench_decode(cpa, torch, synth, steps, warmup, warmup_ms):
    c = synth.workload("mla_decode_131k")
    B, L, C, H = c["B"], c["L"], c["C"], c["Hq"]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    qb = synth.bf16_normal(3, 1, (B, H, c["Dqk"]))
    bits, codes, scales = synth.latent_cache_both(3, 2, B, L, c["Dqk"], c["std"])
    log(f"[bench] decode inputs generated in {time.perf_counter() - t0:.1f}s")
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)
    cache_bf16 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    del bits
    cache_fp8 = torch.from_numpy(codes).to(dev)
    sc = torch.from_numpy(scales).to(dev)
    del codes
    shards = cpa.cp_decode_shards(L, C)
    begins = [torch.full((B,), s0, dtype=torch.int32, device=dev) for s0, _ in shards]
    ends = [torch.full((B,), s1, dtype=torch.int32, device=dev) for _, s1 in shards]
    max_len = max(s1 - s0 for s0, s1 in shards)
    po = torch.empty((C, B, H, 512), dtype=torch.float32, device=dev)
    pl = torch.empty((C, B, H), dtype=torch.float32, device=dev)
    mo = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    ml = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, cpa.attn_decode_workspace_size(B, H, 512, max_len)), dtype=torch.uint8, device=dev)
    res = {}
    for name, cache, kvs, entry in (("bf16", cache_bf16, None, 576 * 2), ("fp8", cache_fp8, sc, 576 + 4)):
        def step(ev=None):
            for i in range(C):
                if ev is not None:
                    ev[i][0].record()
                cpa.attn_decode_shard(q, cache, None, begins[i], ends[i], max_len, c["scale"], kv_scale=kvs,
                                      o_part=po[i], lse_part=pl[i], workspace=ws)
                if ev is not None:
                    ev[i][1].record()
            cpa.attn_merge_states(po, pl, out=mo, lse_out=ml)

        _warm(torch, step, warmup, warmup_ms)
        # timed steps: events only at the step boundaries (an event between
        # every pair of launches adds its own small gap to the stream)
        sev = _events(torch, 1)[0]
        t0 = time.perf_counter()
        sev[0].record()
        for i in range(steps):
            step()
        sev[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_step_ms = sev[0].elapsed_time(sev[1]) / steps
        # per-launch durations (roofline of the partial-launch kernel): a
        # separate pass with events around every launch
        nl = max(3, steps // 4)
        evs = [_events(torch, C) for _ in range(nl)]
        for i in range(nl):
            step(evs[i])
        torch.cuda.synchronize()
        launch_ms = [a.elapsed_time(b) for ev in evs for a, b in ev]
        kv_bytes = B * L * entry
        q_bytes = C * B * H * 576 * 2
        part_bytes = C * B * H * (512 + 1) * 4
        step_bytes = kv_bytes + q_bytes + 2 * part_bytes + B * H * (512 + 1) * 4
        launch_bytes = kv_bytes / C + B * H * 576 * 2 + B * H * (512 + 1) * 4
        ms = wall / steps * 1e3
        lm = float(np.mean(launch_ms))
        res[name] = dict(ms_per_step=ms, gbs=step_bytes / (ms * 1e-3) / 1e9, algorithmic_bytes=step_bytes,
                         gpu_ms_per_step=gpu_step_ms,
                         launch_ms=lm, launch_gbs=launch_bytes / (lm * 1e-3) / 1e9,
                         launch_bytes=launch_bytes)
    res["sparse_fp8"] = bench_sparse(cpa, torch, synth, c, cache_fp8, steps, warmup, warmup_ms, kv_scale=sc)
    res["paged_fp8"] = bench_paged(cpa, torch, synth, c, q, cache_fp8, sc, steps, warmup, warmup_ms)
    del cache_fp8, sc
    torch.cuda.empty_cache()
    res["paged_bf16"] = bench_paged(cpa, torch, synth, c, q, cache_bf16, None, steps, warmup, warmup_ms)
    res["round_robin_bf16"] = bench_round_robin(cpa, torch, c, q, cache_bf16, steps, warmup, warmup_ms)
    res["multi_query_bf16"] = bench_multi_query(cpa, torch, synth, c, cache_bf16, 4, steps, warmup, warmup_ms)
    res["sparse_bf16"] = bench_sparse(cpa, torch, synth, c, cache_bf16, steps, warmup, warmup_ms)
    res["topk"] = bench_topk(cpa, torch, synth, c, steps, warmup, warmup_ms)
    return res


def bench_topk(cpa, torch, synth, c, steps, warmup, warmup_ms):
    """Exact distributed top-2048 with the index split round robin over C=8
    ranks, for the decode batch (64 query rows, 131072 index scores each):
    a step is the C local top-k launches (16384 scores per row and rank) and
    the merge of the C x 2048 candidates into the global top 2048 with the
    owners' index lists. Algorithmic bytes: scores read once, candidate lists
    written and read once, merged ids and owner lists written."""
    N, L, C, k = c["B"], c["L"], c["C"], SPARSE_K
    dev = torch.device("cuda:0")
    s = synth.f32_normal(3, 8, (N, L))
    loc = [torch.from_numpy(np.ascontiguousarray(s[:, r::C])).to(dev) for r in range(C)]
    Lr = loc[0].shape[1]
    sc = torch.empty((C, N, k), dtype=torch.float32, device=dev)
    ids = torch.empty((C, N, k), dtype=torch.int32, device=dev)
    rows = torch.empty((C, N, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((C, N), dtype=torch.int32, device=dev)
    oid = torch.empty((N, k), dtype=torch.int32, device=dev)
    orow = torch.empty((C, N, k), dtype=torch.int32, device=dev)
    ocnt = torch.empty((C, N), dtype=torch.int32, device=dev)
    lib = cpa.lib()
    st = cpa._stream(None)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def step():
        for r in range(C):
            cpa._check(lib.attn_topk_local(ptr(loc[r]), Lr, N, Lr, None, k, r, C, ptr(sc[r]), ptr(ids[r]),
                                           ptr(rows[r]), ptr(cnt[r]), st))
        cpa._check(lib.attn_topk_merge(C, N, k, ptr(sc), ptr(ids), ptr(rows), ptr(cnt), k, ptr(oid), ptr(orow),
                                       ptr(ocnt), st))

    def local0():
        cpa._check(lib.attn_topk_local(ptr(loc[0]), Lr, N, Lr, None, k, 0, C, ptr(sc[0]), ptr(ids[0]),
                                       ptr(rows[0]), ptr(cnt[0]), st))

    def merge():
        cpa._check(lib.attn_topk_merge(C, N, k, ptr(sc), ptr(ids), ptr(rows), ptr(cnt), k, ptr(oid), ptr(orow),
                                       ptr(ocnt), st))

    _warm(torch, step, warmup, warmup_ms)

    def timed(fn, n):
        sev = _events(torch, 1)[0]
        sev[0].record()
        for _ in range(n):
            fn()
        sev[1].record()
        torch.cuda.synchronize()
        return sev[0].elapsed_time(sev[1]) / n

    ms = timed(step, steps)
    local_ms = timed(local0, steps)
    merge_ms = timed(merge, steps)
    nbytes = N * L * 4 + 2 * C * N * k * 12 + N * k * 4 + C * N * k * 4
    # one rank's share: its local top-k over its 16384 scores per row, then the merge
    rank_bytes = N * Lr * 4 + C * N * k * 12 + N * k * 4 + C * N * k * 4 + N * k * 12
    rank_ms = local_ms + merge_ms
    return dict(k=k, ranks=C, rows=N, step_us=ms * 1e3, step_gbs=nbytes / (ms * 1e-3) / 1e9,
                local_us=local_ms * 1e3, merge_us=merge_ms * 1e3, per_rank_us=rank_ms * 1e3,
                per_rank_gbs=rank_bytes / (rank_ms * 1e-3) / 1e9, algorithmic_bytes=nbytes)


SPARSE_K = 2048


def bench_sparse(cpa, torch, synth, c, cache, steps, warmup, warmup_ms, kv_scale=None):
    """Sparse (top-k index list) MLA attention on the same latent cache:
    (a) decode: one query per request, 2,048 rows drawn from its 131072;
    (b) prefill: 4,096 queries of request 0 at positions 8j (j = 12288 ..
    16383, an interleave rank's share), each with 2,048 rows drawn from the
    rows at or below its position. Algorithmic bytes per query: the listed
    rows (1,152 B) and their 4-byte indices, plus per head the bf16 query
    (1,152 B), the f32 output (2,048 B) and its LSE; FLOPs: 2,176 per row
    and head (QK over 576, PV over 512). With kv_scale the cache is FP8:
    a row is 576 code bytes plus its 4-byte scale."""
    B, L, H = c["B"], c["L"], c["Hq"]
    row_bytes = 1152 if kv_scale is None else 576 + 4
    dev = cache.device
    out = {}
    cases = (("decode", B, None, None), ("prefill", 4096, np.zeros(4096, np.int32),
                                         8 * np.arange(12288, 16384, dtype=np.int64)))
    for name, N, req, pos in cases:
        qb = synth.bf16_normal(3, 5, (N, H, c["Dqk"]))
        q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)
        idx, cnt = synth.topk_lists(3, 6 if name == "decode" else 7, N, L, SPARSE_K,
                                    limit=None if pos is None else pos + 1)
        idx_d = torch.from_numpy(idx).to(dev)
        req_d = torch.from_numpy(req).to(dev) if req is not None else None
        o = torch.empty((N, H, 512), dtype=torch.float32, device=dev)
        l = torch.empty((N, H), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, cpa.attn_sparse_mla_workspace_size(N, SPARSE_K)), dtype=torch.uint8, device=dev)

        def step():
            cpa.attn_sparse_mla(q, cache, idx_d, c["scale"], req=req_d, out=o, lse=l, workspace=ws, kv_scale=kv_scale)

        _warm(torch, step, warmup, warmup_ms)
        n_steps = steps if name == "decode" else max(3, steps // 4)
        sev = _events(torch, 1)[0]
        sev[0].record()
        for _ in range(n_steps):
            step()
        sev[1].record()
        torch.cuda.synchronize()
        ms = sev[0].elapsed_time(sev[1]) / n_steps
        rows = int(cnt.sum())
        nbytes = rows * (row_bytes + 4) + N * H * (1152 + 2048 + 4)
        flops = rows * H * 2176
        out[name] = dict(queries=N, k=SPARSE_K, ms=ms, gbs=nbytes / (ms * 1e-3) / 1e9,
                         tflops=flops / (ms * 1e-3) / 1e12, algorithmic_bytes=nbytes, flops=flops)
        del q, idx_d, o, l, ws
    return out


def bench_multi_query(cpa, torch, synth, c, cache, Q, steps, warmup, warmup_ms):
    """Multi-query (MTP: one verified token + three drafts = 4 query rows)
    decode at the same shape: contiguous shards, every query row causal over
    its request; a step is C partial launches plus the merge of B * Q rows."""
    B, L, C, H = c["B"], c["L"], c["C"], c["Hq"]
    dev = cache.device
    qb = synth.bf16_normal(3, 4, (B, Q, H, c["Dqk"]))
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)
    shards = cpa.cp_decode_shards(L, C)
    plans = [cpa.cp_plan_multi_query(cpa.CPA_LAYOUT_CONTIGUOUS, C, r, [L] * B, Q) for r in range(C)]
    begins = [torch.from_numpy(p[0]).to(dev) for p in plans]
    ends = [torch.from_numpy(p[1]).to(dev) for p in plans]
    max_len = max(p[2] for p in plans)
    po = torch.empty((C, B, Q, H, 512), dtype=torch.float32, device=dev)
    pl = torch.empty((C, B, Q, H), dtype=torch.float32, device=dev)
    mo = torch.empty((B * Q, H, 512), dtype=torch.float32, device=dev)
    ml = torch.empty((B * Q, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, cpa.attn_decode_workspace_size(B * Q, H, 512, max_len)), dtype=torch.uint8, device=dev)

    def step():
        for r, (s0, s1) in enumerate(shards):
            cpa.attn_decode_shard_mq(q, cache[:, s0:s1], None, begins[r], ends[r], max_len, c["scale"],
                                     o_part=po[r], lse_part=pl[r], workspace=ws)
        cpa.attn_merge_states(po.view(C, B * Q, H, 512), pl.view(C, B * Q, H), out=mo, lse_out=ml)

    _warm(torch, step, warmup, warmup_ms)
    sev = _events(torch, 1)[0]
    sev[0].record()
    for _ in range(steps):
        step()
    sev[1].record()
    torch.cuda.synchronize()
    ms = sev[0].elapsed_time(sev[1]) / steps
    rows = B * Q
    step_bytes = B * L * 1152 + C * rows * H * 576 * 2 + 2 * C * rows * H * (512 + 1) * 4 + rows * H * (512 + 1) * 4
    # key reads of the query rows: row k of a request sees L - Q + k + 1 keys
    keys = B * sum(L - Q + k + 1 for k in range(Q))
    flops = keys * H * 2 * (576 + 512)
    return dict(Q=Q, gpu_ms_per_step=ms, gbs=step_bytes / (ms * 1e-3) / 1e9, algorithmic_bytes=step_bytes,
                tflops=flops / (ms * 1e-3) / 1e12, flops=flops)


PAGE_SIZE = 64


def bench_paged(cpa, torch, synth, c, q, cache, kvs, steps, warmup, warmup_ms):
    """The MLA decode step (C partial launches + merge) over a paged cache:
    the same rows as `cache`, in 64-token pages of one pool placed in a
    seeded random order (block table [B, L / 64])."""
    B, L, C, H = c["B"], c["L"], c["C"], c["Hq"]
    dev = cache.device
    ps = PAGE_SIZE
    nb = L // ps
    table = torch.from_numpy(synth.page_table(3, 9, B, nb, B * nb)).to(dev)
    dst = table.reshape(-1).long()
    pool = torch.empty((B * nb, ps) + tuple(cache.shape[2:]), dtype=cache.dtype, device=dev)
    pool[dst] = cache.reshape((B * nb, ps) + tuple(cache.shape[2:]))
    pool = pool.reshape((B * L,) + tuple(cache.shape[2:]))
    spool = None
    if kvs is not None:
        spool = torch.empty((B * nb, ps), dtype=kvs.dtype, device=dev)
        spool[dst] = kvs.reshape(B * nb, ps)
        spool = spool.reshape(-1)
    shards = cpa.cp_decode_shards(L, C)
    begins = [torch.full((B,), s0, dtype=torch.int32, device=dev) for s0, _ in shards]
    ends = [torch.full((B,), s1, dtype=torch.int32, device=dev) for _, s1 in shards]
    max_len = max(s1 - s0 for s0, s1 in shards)
    po = torch.empty((C, B, H, 512), dtype=torch.float32, device=dev)
    pl = torch.empty((C, B, H), dtype=torch.float32, device=dev)
    mo = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    ml = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, cpa.attn_decode_paged_workspace_size(B, H, 512, max_len, ps)), dtype=torch.uint8,
                     device=dev)

    def step():
        for i in range(C):
            cpa.attn_decode_shard_paged(q, pool, None, table, ps, begins[i], ends[i], max_len, c["scale"],
                                        kv_scale=spool, o_part=po[i], lse_part=pl[i], workspace=ws)
        cpa.attn_merge_states(po, pl, out=mo, lse_out=ml)

    _warm(torch, step, warmup, warmup_ms)
    sev = _events(torch, 1)[0]
    sev[0].record()
    for _ in range(steps):
        step()
    sev[1].record()
    torch.cuda.synchronize()
    ms = sev[0].elapsed_time(sev[1]) / steps
    entry = 576 * 2 if kvs is None else 576 + 4
    step_bytes = (B * L * entry + C * B * nb * 4 + C * B * H * 576 * 2 + 2 * C * B * H * (512 + 1) * 4
                  + B * H * (512 + 1) * 4)
    del pool, spool
    torch.cuda.empty_cache()
    return dict(page_size=ps, gpu_ms_per_step=ms, gbs=step_bytes / (ms * 1e-3) / 1e9, algorithmic_bytes=step_bytes)


def bench_round_robin(cpa, torch, c, q, cache, steps, warmup, warmup_ms):
    """Round-robin decode storage at the same shape: slot p of every request
    on rank p mod C as row p // C. The C local caches are written from the
    full cache by the slot-translating cache write (timed once, bytes read +
    written), then a step is C partial launches over them plus the merge."""
    B, L, C, H = c["B"], c["L"], c["C"], c["Hq"]
    dev = cache.device
    full = cache[:, :, 0, :]
    src = full.reshape(B * L, -1)
    slot = torch.arange(L, dtype=torch.int64, device=dev).repeat(B)
    req = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(L)
    plans = [cpa.cp_plan_round_robin(C, r, [L] * B) for r in range(C)]
    rows = max(p[2] for p in plans)
    locals_ = [torch.empty((B, rows, 1, cache.shape[-1]), dtype=cache.dtype, device=dev) for _ in range(C)]
    ev = _events(torch, 1)[0]
    ev[0].record()
    for r in range(C):
        cpa.attn_cache_write_round_robin(C, r, src, slot, req, locals_[r][:, :, 0, :])
    ev[1].record()
    torch.cuda.synchronize()
    write_ms = ev[0].elapsed_time(ev[1])
    write_bytes = 2 * B * L * cache.shape[-1] * cache.element_size() + C * B * L * 12
    begins = [torch.from_numpy(p[0]).to(dev) for p in plans]
    ends = [torch.from_numpy(p[1]).to(dev) for p in plans]
    max_len = max(int((p[1] - p[0]).max()) for p in plans)
    po = torch.empty((C, B, H, 512), dtype=torch.float32, device=dev)
    pl = torch.empty((C, B, H), dtype=torch.float32, device=dev)
    mo = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    ml = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, cpa.attn_decode_workspace_size(B, H, 512, max_len)), dtype=torch.uint8, device=dev)

    def step():
        for r in range(C):
            cpa.attn_decode_shard(q, locals_[r], None, begins[r], ends[r], max_len, c["scale"],
                                  o_part=po[r], lse_part=pl[r], workspace=ws)
        cpa.attn_merge_states(po, pl, out=mo, lse_out=ml)

    _warm(torch, step, warmup, warmup_ms)
    sev = _events(torch, 1)[0]
    sev[0].record()
    for _ in range(steps):
        step()
    sev[1].record()
    torch.cuda.synchronize()
    ms = sev[0].elapsed_time(sev[1]) / steps
    step_bytes = B * L * 1152 + C * B * H * 576 * 2 + 2 * C * B * H * (512 + 1) * 4 + B * H * (512 + 1) * 4
    del locals_
    torch.cuda.empty_cache()
    return dict(gpu_ms_per_step=ms, gbs=step_bytes / (ms * 1e-3) / 1e9, algorithmic_bytes=step_bytes,
                cache_write_ms=write_ms, cache_write_gbs=write_bytes / (write_ms * 1e-3) / 1e9,
                cache_write_bytes=write_bytes)


GQA_SERVING = dict(B=8, Hq=32, Hkv=8, D=128, L=131072, C=8)


def _gqa_step_bytes(B, Hq, Hkv, D, L, C, entry, qsz):
    """Algorithmic bytes of a GQA decode step (C partial launches + merge):
    the cache read once (`entry` bytes per token and kv head, K and V and any
    scale share), the queries of every launch, the partial states written and
    read by the merge, and the merged result."""
    kv = B * L * Hkv * entry
    q = C * B * Hq * D * qsz
    part = C * B * Hq * (D + 1) * 4
    return kv + q + 2 * part + B * Hq * (D + 1) * 4, kv / C + B * Hq * D * qsz + B * Hq * (D + 1) * 4


def _gqa_run(cpa, torch, q, k, v, kvs, L, C, scale, steps, warmup, warmup_ms, flush=None):
    """Time C partial decode launches over the contiguous shards plus the
    merge. Returns (ms per step, mean ms per partial launch)."""
    dev = q.device
    B, Hq, D = q.shape
    shards = cpa.cp_decode_shards(L, C)
    begins = [torch.full((B,), s0, dtype=torch.int32, device=dev) for s0, _ in shards]
    ends = [torch.full((B,), s1, dtype=torch.int32, device=dev) for _, s1 in shards]
    max_len = max(s1 - s0 for s0, s1 in shards)
    po = torch.empty((C, B, Hq, D), dtype=torch.float32, device=dev)
    pl = torch.empty((C, B, Hq), dtype=torch.float32, device=dev)
    mo = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ml = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, cpa.attn_decode_workspace_size(B, Hq, D, max_len)), dtype=torch.uint8, device=dev)

    def step(ev=None):
        for i in range(C):
            if ev is not None:
                ev[i][0].record()
            cpa.attn_decode_shard(q, k, v, begins[i], ends[i], max_len, scale, kv_scale=kvs,
                                  o_part=po[i], lse_part=pl[i], workspace=ws)
            if ev is not None:
                ev[i][1].record()
        cpa.attn_merge_states(po, pl, out=mo, lse_out=ml)

    _warm(torch, step, warmup, warmup_ms)
    if flush is None:
        sev = _events(torch, 1)[0]
        sev[0].record()
        for _ in range(steps):
            step()
        sev[1].record()
        torch.cuda.synchronize()
        ms = sev[0].elapsed_time(sev[1]) / steps
    else:  # every step after a cache flush, timed alone
        sevs = _events(torch, steps)
        for i in range(steps):
            flush(i)
            sevs[i][0].record()
            step()
            sevs[i][1].record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in sevs]))
    nl = max(3, steps // 4)
    evs = [_events(torch, C) for _ in range(nl)]
    for i in range(nl):
        if flush is not None:
            flush(i)
        step(evs[i])
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for ev in evs for a, b in ev]))
    return ms, launch_ms


def bench_gqa_decode(cpa, torch, steps, warmup, warmup_ms):
    """Split-KV GQA decode at a serving shape: batch 8, 32 query heads on 8
    kv heads, head dim 128, a 131072-token context per request cut into C=8
    contiguous shards, run as 8 partial launches plus the merge; bf16 cache,
    and FP8 E4M3 with one scale per token (key and value). Inputs: seeded
    N(0,1) drawn on the device (the 4.3 GB bf16 cache would take a minute
    on the host). GB/s of algorithmic bytes."""
    w = GQA_SERVING
    B, Hq, Hkv, D, L, C = w["B"], w["Hq"], w["Hkv"], w["D"], w["L"], w["C"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260)
    q = torch.randn((B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    k = torch.randn((B, L, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    v = torch.randn((B, L, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    res = {"workload": "GQA split-KV decode: batch 8, 32 q / 8 kv heads, d=128, 131072-token context, "
                       "C=8 contiguous shards as 8 partial launches + merge"}
    ms, lms = _gqa_run(cpa, torch, q, k, v, None, L, C, scale, steps, warmup, warmup_ms)
    sb, lb = _gqa_step_bytes(B, Hq, Hkv, D, L, C, 2 * D * 2, 2)
    res["bf16"] = dict(ms_per_step=ms, gbs=sb / (ms * 1e-3) / 1e9, frac_of_hbm_peak=sb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       algorithmic_bytes=sb, launch_ms=lms, launch_gbs=lb / (lms * 1e-3) / 1e9, launch_bytes=lb)
    # FP8: one scale per token over its key and value rows (amax / 448)
    amax = torch.maximum(k.abs().amax(dim=(2, 3)), v.abs().amax(dim=(2, 3))).float()
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).contiguous()
    kc = (k.float() / sc[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (v.float() / sc[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    del k, v
    torch.cuda.empty_cache()
    ms, lms = _gqa_run(cpa, torch, q, kc, vc, sc, L, C, scale, steps, warmup, warmup_ms)
    sb, lb = _gqa_step_bytes(B, Hq, Hkv, D, L, C, 2 * D + 4 / Hkv, 2)
    res["fp8"] = dict(ms_per_step=ms, gbs=sb / (ms * 1e-3) / 1e9, frac_of_hbm_peak=sb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      algorithmic_bytes=sb, launch_ms=lms, launch_gbs=lb / (lms * 1e-3) / 1e9, launch_bytes=lb)
    del kc, vc, sc
    torch.cuda.empty_cache()
    return res


def bench_decode_gqa_f32_4k(cpa, torch, synth, steps, warmup, warmup_ms):
    """Split-KV decode + LSE merge, fp32: batch 1, 8 query heads on 1 kv head,
    head dim 128, 4096-token context as C=4 contiguous 1024-token shards (4
    partial launches + merge per step), with the last-level cache flushed
    (a 512 MiB write) before every timed step, and cache-hot."""
    c = synth.workload("gqa_decode_f32_4k")
    B, Hq, Hkv, D, L, C = c["B"], c["Hq"], c["Hkv"], c["Dqk"], c["L"], c["C"]
    dev = torch.device("cuda:0")
    q = torch.from_numpy(synth.f32_normal(1, 1, (B, Hq, D))).to(dev)
    k = torch.from_numpy(synth.f32_normal(1, 2, (B, L, Hkv, D), chunk=1)).to(dev)
    v = torch.from_numpy(synth.f32_normal(1, 3, (B, L, Hkv, D), chunk=1)).to(dev)
    scratch = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    sb, lb = _gqa_step_bytes(B, Hq, Hkv, D, L, C, 2 * D * 4, 4)
    out = {"workload": c["name"]}
    for name, flush in (("cache_flushed", lambda i: scratch.fill_(float(i))), ("cache_hot", None)):
        ms, lms = _gqa_run(cpa, torch, q, k, v, None, L, C, c["scale"], steps, warmup, warmup_ms, flush=flush)
        out[name] = dict(ms_per_step=ms, gbs=sb / (ms * 1e-3) / 1e9, frac_of_hbm_peak=sb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         launch_ms=lms, launch_gbs=lb / (lms * 1e-3) / 1e9)
    out["algorithmic_bytes"] = sb
    out["launch_bytes"] = lb
    out["note"] = ("4.2 MB per step: the step is bound by launch and merge latency (5 dependent kernels), "
                   "not by HBM bandwidth")
    del scratch
    torch.cuda.empty_cache()
    return out


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _decode_flops(L, Hq, Dqk, Dv):
    return L * Hq * 2 * (Dqk + Dv)


def _oracle_decode_all_shards(att, q, cache, L, C, scale, **kw):
    """The oracle's C contiguous partial decodes of the range [0, L) and
    their merge (what one step of the GPU path computes)."""
    from oracle import plans
    B = q.shape[0]
    parts = [att.decode_shard(q, cache, [s0] * B, [s1] * B, scale, **kw) for s0, s1 in plans.contiguous_shards(L, C)]
    return att.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


def _oracle_rows(att, q, k, v, plan, c, rows_order, seconds, min_rows, decode):
    """Run the oracle's prefill shard on batches of 4 local rows from
    rows_order until `seconds` have passed and at least `min_rows` are done."""
    pos = plan.pos_id.astype(np.int64)
    done, flops = 0, 0
    t0 = time.perf_counter()
    while done < len(rows_order) and (time.perf_counter() - t0 < seconds or done < min_rows):
        rows = sorted(int(r) for r in rows_order[done:done + 4])
        att.prefill_shard(q, k, plan.segments, c["scale"], v=v, dv=c["Dv"], rows=rows, decode=decode)
        flops += int(np.sum(pos[rows] + 1)) * c["Hq"] * 2 * (c["Dqk"] + c["Dv"])
        done += len(rows)
    return done, flops, time.perf_counter() - t0


def _segment_end_rows(plan):
    rows = []
    for (_req, r0, n, _p0, _st, _kv0) in plan.segments:
        rows += [r0, r0 + n - 1]
    return list(dict.fromkeys(rows))


def cpu_baseline(synth, prefill, seconds, per_workload_seconds=5.0, min_rows=0):
    """The float64 oracle, as it stands, on this host's cores, on bounded
    samples of every workload: the zigzag GQA prefill shard (the headline
    comparison, ``value``), and per workload: the fp32 GQA decode in
    full, one request of the MLA decode (bf16 and FP8, extrapolated to the
    batch), and sampled local rows of the MLA zigzag and ragged interleave
    prefill shards (segment ends first, then random rows; extrapolated to
    the whole shard from the FLOP rate)."""
    from oracle import attention as att
    from oracle import formats, plans
    cores = _cores()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(cores)
    except Exception:  # pragma: no cover
        limiter = None
    per = {}

    # the zigzag GQA prefill shard (headline)
    c = prefill["cfg"]
    ref = plans.plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    T = sum(c["new_len"])
    qb = synth.bf16_normal(2, 1, (ref.n_local, c["Hq"], c["Dqk"]))
    kb = synth.bf16_normal(2, 2, (T, c["Hkv"], c["Dqk"]))
    vb = synth.bf16_normal(2, 3, (T, c["Hkv"], c["Dv"]))
    order = synth.rng(2, 9).permutation(ref.n_local)
    done_rows, flops, dt = _oracle_rows(att, qb, kb, vb, ref, c, order, seconds, 0, formats.bf16_bits_to_f64)
    del qb, kb, vb
    head = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done_rows} of {ref.n_local} local query rows (all 32 heads, random order) of the same "
                      f"zigzag workload in {dt:.1f} s; float64 numpy; the full step would take "
                      f"{prefill['flops'] / (flops / dt):.0f} s"}
    per["gqa_zigzag_prefill_16k"] = dict(rows=done_rows, rows_total=ref.n_local, seconds=round(dt, 2),
                          rows_per_s=round(done_rows / dt, 2), fp64_gflops=round(flops / dt / 1e9, 2),
                          full_step_seconds_extrapolated=round(prefill["flops"] / (flops / dt), 1))

    # the fp32 GQA decode (batch 1, 8/1 heads, 4096 tokens), 4 shards + merge, in full
    c1 = synth.workload("gqa_decode_f32_4k")
    q = synth.f32_normal(1, 1, (c1["B"], c1["Hq"], c1["Dqk"])).astype(np.float64)
    k = synth.f32_normal(1, 2, (c1["B"], c1["L"], c1["Hkv"], c1["Dqk"]), chunk=1).astype(np.float64)
    v = synth.f32_normal(1, 3, (c1["B"], c1["L"], c1["Hkv"], c1["Dv"]), chunk=1).astype(np.float64)
    t0 = time.perf_counter()
    _oracle_decode_all_shards(att, q, k, c1["L"], c1["C"], c1["scale"], vcache=v)
    dt = time.perf_counter() - t0
    fl = _decode_flops(c1["L"], c1["Hq"], c1["Dqk"], c1["Dv"]) * c1["B"]
    per["gqa_decode_f32_4k"] = dict(sample="the whole step (4 shard decodes + merge)", seconds=round(dt, 4),
                          fp64_gflops=round(fl / dt / 1e9, 3),
                          cache_gbs=round(c1["B"] * c1["L"] * c1["Hkv"] * (c1["Dqk"] + c1["Dv"]) * 4 / dt / 1e9, 3))

    # the MLA decode (batch 64, 131072 tokens, C=8): request 0 of the batch (its draw is that of the
    # full cache), 8 shards + merge, bf16 and FP8; extrapolated to 64 requests
    c3 = synth.workload("mla_decode_131k")
    q3 = synth.bf16_normal(3, 1, (c3["B"], c3["Hq"], c3["Dqk"]))[:1]
    bits, codes, scales = synth.latent_cache_both(3, 2, 1, c3["L"], c3["Dqk"], c3["std"])
    fl = _decode_flops(c3["L"], c3["Hq"], c3["Dqk"], c3["Dv"])
    per["mla_decode_131k"] = {}
    for name, cache, kw in (("bf16", bits, dict(decode=formats.bf16_bits_to_f64)),
                            ("fp8", codes, dict(decode=formats.e4m3_to_f64, kv_scale=scales))):
        t0 = time.perf_counter()
        _oracle_decode_all_shards(att, formats.bf16_bits_to_f64(q3), cache, c3["L"], c3["C"], c3["scale"],
                                  dv=c3["Dv"], **kw)
        dt = time.perf_counter() - t0
        per["mla_decode_131k"][name] = dict(sample="request 0 of 64: 64 heads x 131072 tokens, 8 shard decodes + merge",
                                    seconds=round(dt, 2), fp64_gflops=round(fl / dt / 1e9, 2),
                                    full_step_seconds_extrapolated=round(dt * c3["B"], 1))
    del bits, codes, scales

    # the MLA zigzag and the ragged interleave prefill shards: sampled local rows
    for wname in ("mla_zigzag_prefill_prefix32k", "gqa_interleave_prefill_agentic16"):
        ck = synth.workload(wname)
        kcfg = ck["seed"]
        planner = plans.plan_zigzag if ck["strategy"] == "zigzag" else plans.plan_interleave
        pk = planner(ck["C"], ck["rank"], ck["new_len"], ck["prefix_len"])
        Tk = sum(ck["new_len"]) + sum(ck["prefix_len"])
        ends = _segment_end_rows(pk)
        rest = [int(r) for r in synth.rng(kcfg, 9).permutation(pk.n_local) if int(r) not in set(ends)]
        order = ends + rest
        # draw only the query slabs (256 rows) and key/value slabs (4096
        # tokens) the sampled rows read, as the full draw has them
        est = max(min_rows, 64) + len(ends)
        rows_needed = order[:est]
        qk = synth.bf16_normal_slabs(kcfg, 1, (pk.n_local, ck["Hq"], ck["Dqk"]), [r // 256 for r in rows_needed],
                                     chunk=256)
        where = {}
        for (_req, r0, n, p0, st, kv0) in pk.segments:
            for r in range(r0, r0 + n):
                where[r] = (kv0, p0 + (r - r0) * st)
        kv_slabs = set()
        for r in rows_needed:
            kv0, p = where[r]
            kv_slabs.update(range(kv0 // 4096, (kv0 + p) // 4096 + 1))
        kk = synth.bf16_normal_slabs(kcfg, 2, (Tk, ck["Hkv"], ck["Dqk"]), kv_slabs)
        vk = None if ck["Hkv"] == 1 else synth.bf16_normal_slabs(kcfg, 3, (Tk, ck["Hkv"], ck["Dv"]), kv_slabs)
        done_rows, flops, dt = _oracle_rows(att, qk, kk, vk, pk, ck, rows_needed, per_workload_seconds, min_rows,
                                            formats.bf16_bits_to_f64)
        total = int(np.sum(pk.pos_id.astype(np.int64) + 1)) * ck["Hq"] * 2 * (ck["Dqk"] + ck["Dv"])
        per[wname] = dict(
            sample=f"{done_rows} local rows ({min(done_rows, len(ends))} of them segment ends, the rest random) "
                   f"of {pk.n_local}, all heads",
            rows=done_rows, rows_total=pk.n_local, seconds=round(dt, 2), rows_per_s=round(done_rows / dt, 3),
            fp64_gflops=round(flops / dt / 1e9, 2), full_step_seconds_extrapolated=round(total / (flops / dt), 0))
        del qk, kk, vk
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    head["per_workload"] = per
    return head


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="keep warming up (untimed) until this much wall time has passed")
    ap.add_argument("--no-decode", action="store_true", help="skip the secondary MLA decode figures")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-workload-seconds", type=float, default=5.0,
                    help="CPU oracle time per sampled workload (MLA and interleave prefill)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="sample at least this many local rows of the MLA / interleave prefill shards")
    ap.add_argument("--cpu-only", action="store_true", help="only the CPU oracle baselines (no GPU figures)")
    ap.add_argument("--decode-only", action="store_true", help="time only the MLA decode (profiling)")
    ap.add_argument("--gqa-only", action="store_true", help="time only the GQA decode figures (profiling)")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="skip the MLA zigzag (prefix) and ragged interleave prefill figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 2 GiB device-to-device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(shards are evaluated as partial launches on one device). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import synth
    if args.cpu_only:
        from oracle import plans as oplans
        c2 = synth.workload("gqa_zigzag_prefill_16k")
        ref = oplans.plan_zigzag(c2["C"], c2["rank"], c2["new_len"], c2["prefix_len"])
        flops = int(np.sum(ref.pos_id.astype(np.int64) + 1)) * c2["Hq"] * 2 * (c2["Dqk"] + c2["Dv"])
        base = cpu_baseline(synth, {"cfg": c2, "flops": flops}, args.cpu_seconds, args.cpu_workload_seconds,
                            args.cpu_rows)
        print(json.dumps({"cpu_baseline": base}), flush=True)
        return

    import torch
    import context_attention_long_amd as cpa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cpa.lib()

    if args.copy_calibration:
        # a plain copy of known size: 2 GiB read + 2 GiB written (larger than
        # the last-level cache, so it runs from and to HBM)
        src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 2147483648 bytes read, 2147483648 written")
        del src, dst
        torch.cuda.empty_cache()

    if args.decode_only:
        dec = bench_decode(cpa, torch, synth, args.steps, args.warmup, args.warmup_ms)
        print(json.dumps({"decode": dec}), flush=True)
        return
    if args.gqa_only:
        g = bench_gqa_decode(cpa, torch, args.steps, args.warmup, args.warmup_ms)
        c1 = bench_decode_gqa_f32_4k(cpa, torch, synth, args.steps, args.warmup, args.warmup_ms)
        print(json.dumps({"decode_gqa": g, "decode_gqa_f32_4k": c1}), flush=True)
        return

    log("[bench] zigzag prefill shard ...")
    pre = bench_prefill(cpa, torch, synth, args.steps, args.warmup, args.warmup_ms)
    ms = pre["wall"] / args.steps * 1e3
    value = pre["flops"] / (ms * 1e-3) / 1e12
    kms = float(np.mean(pre["kernel_ms"]))
    achieved = pre["flops"] / (kms * 1e-3) / 1e12
    log(f"[bench] prefill: {ms:.3f} ms/step, {value:.1f} TFLOP/s; kernel {kms:.3f} ms -> {achieved:.1f} TFLOP/s")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": pre["warmup_steps"],
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 queries/keys/values)",
        "config": {
            "workload": "zigzag prefill shard: causal GQA 32 q / 8 kv heads, d=128, bf16, 16384-token prompt, "
                        "C=4, rank 1 (blocks 1 and 6), no cached prefix",
            "seq_len": 16384, "cp_size": 4, "rank": 1, "local_rows": pre["plan"].n_local,
            "causal_pairs_per_head": pre["pairs"], "algorithmic_gflop": round(pre["flops"] / 1e9, 3),
        },
        "roofline": {
            "kernel": "prefill_gqa_kernel",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic("prefill_gqa_kernel")[0],
            "traffic_detail": traffic("prefill_gqa_kernel")[1],
            "kernel_ms": round(kms, 4),
        },
        "prefill_cache_flushed": {
            kind: {
                "flush": f"512 MiB {kind} before each launch, outside the events (the last-level cache is 256 MB)",
                "reps": len(v),
                "kernel_ms_median": round(float(np.median(v)), 4),
                "tflops_median": round(pre["flops"] / (float(np.median(v)) * 1e-3) / 1e12, 1),
                "frac_of_mfma_peak": round(pre["flops"] / (float(np.median(v)) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            } for kind, v in pre["cold_ms"].items()
        },
    }
    del pre["inputs"]
    torch.cuda.empty_cache()

    if not args.no_decode:
        log("[bench] split-KV MLA decode (8 partial launches + merge) ...")
        dec = bench_decode(cpa, torch, synth, max(3, args.steps // 2), args.warmup, args.warmup_ms)
        line["decode"] = {
            "workload": "MLA split-KV decode: batch 64, 64 heads, 576/512 latent, 131072-token context, "
                        "C=8 contiguous shards as 8 partial launches + merge",
            "unit": "GB/s",
            "bf16": {k: round(v, 4) if isinstance(v, float) else v for k, v in dec["bf16"].items()},
            "fp8": {k: round(v, 4) if isinstance(v, float) else v for k, v in dec["fp8"].items()},
            "roofline": {
                "kernel": "decode_mla_ws_kernel (bf16 cache)", "bound": "hbm",
                "achieved": round(dec["bf16"]["launch_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dec["bf16"]["launch_gbs"] / PEAK_HBM_GBS, 4),
                "traffic": traffic("decode_mla_kernel<bf16>")[0],
                "traffic_detail": traffic("decode_mla_kernel<bf16>")[1],
            },
            "round_robin_bf16": {k: round(v, 4) if isinstance(v, float) else v for k, v in dec["round_robin_bf16"].items()},
            "paged": {k: {kk: round(vv, 4) if isinstance(vv, float) else vv for kk, vv in dec[k].items()}
                      for k in ("paged_bf16", "paged_fp8")},
            "frac_of_hbm_peak_step": {k: round(dec[k]["gbs"] / PEAK_HBM_GBS, 4)
                                      for k in ("bf16", "fp8", "round_robin_bf16", "paged_bf16", "paged_fp8")},
            "topk_split_index": {k: round(v, 4) if isinstance(v, float) else v for k, v in dec["topk"].items()},
            "sparse_bf16": {k: dict({kk: round(vv, 4) if isinstance(vv, float) else vv for kk, vv in v.items()},
                                    frac_of_hbm_peak=round(v["gbs"] / PEAK_HBM_GBS, 4))
                            for k, v in dec["sparse_bf16"].items()},
            "sparse_fp8": {k: dict({kk: round(vv, 4) if isinstance(vv, float) else vv for kk, vv in v.items()},
                                   frac_of_hbm_peak=round(v["gbs"] / PEAK_HBM_GBS, 4))
                           for k, v in dec["sparse_fp8"].items()},
            "multi_query_bf16": dict(
                {k: round(v, 4) if isinstance(v, float) else v for k, v in dec["multi_query_bf16"].items()},
                workload="4 query rows per request (MTP3), causal among them; same cache and shards",
                frac_of_hbm_peak=round(dec["multi_query_bf16"]["gbs"] / PEAK_HBM_GBS, 4),
                frac_of_bf16_mfma_peak=round(dec["multi_query_bf16"]["tflops"] / PEAK_BF16_TFLOPS, 4)),
        }
        log(f"[bench] decode bf16 {dec['bf16']['gbs']:.0f} GB/s/step, fp8 {dec['fp8']['gbs']:.0f} GB/s/step, "
            f"paged (64-token pages) bf16 {dec['paged_bf16']['gbs']:.0f}, fp8 {dec['paged_fp8']['gbs']:.0f} GB/s/step, "
            f"round-robin bf16 {dec['round_robin_bf16']['gbs']:.0f} GB/s/step "
            f"(cache write {dec['round_robin_bf16']['cache_write_gbs']:.0f} GB/s), "
            f"multi-query Q=4 {dec['multi_query_bf16']['gbs']:.0f} GB/s/step, "
            f"{dec['multi_query_bf16']['tflops']:.0f} TFLOP/s; sparse top-2048 decode "
            f"{dec['sparse_bf16']['decode']['gbs']:.0f} GB/s (FP8 {dec['sparse_fp8']['decode']['gbs']:.0f}), "
            f"prefill {dec['sparse_bf16']['prefill']['gbs']:.0f} GB/s (FP8 {dec['sparse_fp8']['prefill']['gbs']:.0f})")

    if not args.no_decode:
        log("[bench] split-KV GQA decode (serving shape, bf16 and FP8) and the fp32 4096-token GQA decode ...")
        g = bench_gqa_decode(cpa, torch, max(3, args.steps // 2), args.warmup, args.warmup_ms)
        rnd = lambda d: {k: round(v, 4) if isinstance(v, float) else v for k, v in d.items()}
        line["decode_gqa"] = {"workload": g["workload"], "unit": "GB/s", "bf16": rnd(g["bf16"]), "fp8": rnd(g["fp8"]),
                              "roofline": {
                                  "kernel": "decode_gqa_kernel (bf16 cache)", "bound": "hbm",
                                  "achieved": round(g["bf16"]["launch_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(g["bf16"]["launch_gbs"] / PEAK_HBM_GBS, 4),
                                  "traffic": traffic("decode_gqa_kernel<bf16>")[0],
                                  "traffic_detail": traffic("decode_gqa_kernel<bf16>")[1]}}
        c1 = bench_decode_gqa_f32_4k(cpa, torch, synth, max(3, args.steps // 2), args.warmup, args.warmup_ms)
        line["decode_gqa_f32_4k"] = {k: (rnd(v) if isinstance(v, dict) else v) for k, v in c1.items()}
        log(f"[bench] GQA decode bf16 {g['bf16']['gbs']:.0f} GB/s/step, fp8 {g['fp8']['gbs']:.0f} GB/s/step; "
            f"fp32 4096-token decode (cache flushed) {c1['cache_flushed']['gbs']:.1f} GB/s/step")

    if not args.no_extra_prefill:
        for wname, key in (("mla_zigzag_prefill_prefix32k", "prefill_mla_zigzag"),
                           ("gqa_interleave_prefill_agentic16", "prefill_interleave")):
            log(f"[bench] {key} ({wname}) ...")
            line[key] = bench_prefill_workload(cpa, torch, synth, wname, max(2, args.steps // 10), 1, args.warmup_ms)
            log(f"[bench] {key}: {line[key]['kernel_ms']} ms, {line[key]['tflops']} TFLOP/s")

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        line["cpu_baseline"] = cpu_baseline(synth, pre, args.cpu_seconds, args.cpu_workload_seconds, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
