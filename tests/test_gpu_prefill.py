"""GPU parity: prefill shard attention (zigzag / interleave plans from the
library's planner) against the float64 oracle on the same bf16 inputs."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as att
from oracle import formats, plans
from tests import helpers as H

pytestmark = pytest.mark.gpu


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


def _segments_tuples(plan):
    return [tuple(int(x) for x in (s["req"], s["q_row0"], s["q_len"], s["pos0"], s["pos_stride"], s["kv_row0"]))
            for s in plan.segments]


def _run_case(cpa, strategy, C, rank, new_len, prefix, Hq, Hkv, seed, out_f32=False, rows=None, spiky=False):
    import torch
    fn = cpa.cp_plan_zigzag if strategy == "zigzag" else cpa.cp_plan_interleave
    plan = fn(C, rank, new_len, prefix)
    ref_plan = (plans.plan_zigzag if strategy == "zigzag" else plans.plan_interleave)(C, rank, new_len, prefix)
    assert _segments_tuples(plan) == [tuple(s) for s in ref_plan.segments]
    T_kv = int(sum(new_len) + (sum(prefix) if prefix else 0))
    D = 128
    rng = np.random.default_rng(seed)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((max(plan.n_local, 1), Hq, D)).astype(np.float32))[:plan.n_local]
    kx = rng.standard_normal((T_kv, Hkv, D)).astype(np.float32)
    if spiky and T_kv > 0:
        # plant keys equal to a query direction times 4 so some logits are large
        kx[rng.integers(0, T_kv, size=max(1, T_kv // 50))] *= 4.0
    kb = synth.f32_to_bf16_bits(kx)
    vb = synth.f32_to_bf16_bits(rng.standard_normal((T_kv, Hkv, D)).astype(np.float32))
    scale = (8.0 if spiky else 1.0) / math.sqrt(D)
    out_dtype = torch.float32 if out_f32 else torch.bfloat16
    o, l = cpa.attn_prefill_shard(H.bf16_tensor(qb), H.bf16_tensor(kb), H.bf16_tensor(vb), plan.segments, scale,
                                  out_dtype=out_dtype)
    _sync()
    if plan.n_local == 0:
        return
    ro, rl = att.prefill_shard(qb, kb, ref_plan.segments, scale, v=vb, rows=rows, decode=formats.bf16_bits_to_f64)
    go, gl = H.host(o), H.host(l)
    if rows is not None:
        go, gl = go[rows], gl[rows]
    H.check_lowp(go, gl, ro, rl, f"{strategy} C={C} r={rank} L={new_len} P={prefix} Hq={Hq}/{Hkv}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 2), (32, 8)])
def test_prefill_zigzag_small(cpa, Hq, Hkv):
    for rank in range(4):
        _run_case(cpa, "zigzag", 4, rank, [300], [0], Hq, Hkv, 10 + rank)
    _run_case(cpa, "zigzag", 4, 1, [300], [37], Hq, Hkv, 20)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 2)])
def test_prefill_interleave_ragged(cpa, Hq, Hkv):
    new_len, prefix = [100, 3, 250, 0, 64, 1], [0, 5, 130, 2, 0, 0]
    for rank in range(3):
        _run_case(cpa, "interleave", 3, rank, new_len, prefix, Hq, Hkv, 30 + rank)


def test_prefill_zigzag_multi_request_and_edges(cpa):
    # blocks smaller than the tile, empty blocks (L < 2C), single tokens
    _run_case(cpa, "zigzag", 4, 0, [7, 1, 0, 129, 513], [0, 3, 9, 0, 64], 8, 2, 40)
    _run_case(cpa, "zigzag", 4, 3, [7, 1, 0, 129, 513], [0, 3, 9, 0, 64], 8, 2, 41)
    _run_case(cpa, "zigzag", 1, 0, [200], [0], 8, 2, 42, out_f32=True)
    _run_case(cpa, "interleave", 8, 5, [3], [0], 8, 2, 43)  # empty share


def test_prefill_spiky_scores(cpa):
    _run_case(cpa, "zigzag", 2, 0, [700], [50], 8, 2, 50, spiky=True)
    _run_case(cpa, "interleave", 2, 1, [700, 90], [50, 0], 8, 2, 51, spiky=True)


def test_prefill_empty_segments_noop(cpa):
    import torch
    q = torch.zeros((4, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((4, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((4, 8), 7.0, dtype=torch.float32, device="cuda")
    cpa.attn_prefill_shard(q, k, k, np.zeros(0, cpa.SEGMENT_DTYPE), 0.1, out=out, lse=lse)
    _sync()
    assert bool((out == 7).all()) and bool((lse == 7).all())


def test_prefill_rejects_out_of_range_segment(cpa):
    import torch
    q = torch.zeros((4, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((10, 2, 128), dtype=torch.bfloat16, device="cuda")
    seg = np.zeros(1, cpa.SEGMENT_DTYPE)
    seg[0] = (0, 0, 4, 7, 1, 0, 0)  # reads K rows up to 7 + 3 + 1 = 11 > 10
    with pytest.raises(cpa.CpaError) as e:
        cpa.attn_prefill_shard(q, k, k, seg, 0.1)
    assert e.value.status == cpa.CPA_E_INVAL
    seg[0] = (0, 2, 4, 0, 1, 0, 0)  # q rows 2..5 > n_local 4
    with pytest.raises(cpa.CpaError):
        cpa.attn_prefill_shard(q, k, k, seg, 0.1)


def _sample_rows(plan, n_extra, seed):
    rows = set()
    for s in plan.segments:
        r0, n = int(s["q_row0"]), int(s["q_len"])
        rows.update([r0, r0 + n - 1, r0 + min(n - 1, 31), r0 + min(n - 1, 32)])
    rng = synth.rng(seed, 9)
    rows.update(int(x) for x in rng.integers(0, plan.n_local, size=n_extra))
    return sorted(rows)


@pytest.mark.slow
def test_prefill_zigzag_gqa_workload(cpa):
    """Zigzag prefill shard: causal GQA, 32 query heads on 8 kv heads, d=128,
    16384-token prompt, C=4, rank 1 (blocks 1 and 6), bf16 in."""
    c = synth.workload("gqa_zigzag_prefill_16k")
    plan = cpa.cp_plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    T = sum(c["new_len"])
    qb = synth.bf16_normal(2, 1, (plan.n_local, c["Hq"], c["Dqk"]))
    kb = synth.bf16_normal(2, 2, (T, c["Hkv"], c["Dqk"]))
    vb = synth.bf16_normal(2, 3, (T, c["Hkv"], c["Dv"]))
    o, l = cpa.attn_prefill_shard(H.bf16_tensor(qb), H.bf16_tensor(kb), H.bf16_tensor(vb), plan.segments, c["scale"])
    _sync()
    rows = _sample_rows(plan, 48, 2)
    ref = plans.plan_zigzag(c["C"], c["rank"], c["new_len"], c["prefix_len"])
    ro, rl = att.prefill_shard(qb, kb, ref.segments, c["scale"], v=vb, rows=rows, decode=formats.bf16_bits_to_f64)
    e = H.check_lowp(H.host(o)[rows], H.host(l)[rows], ro, rl, "zigzag GQA workload")
    print("zigzag GQA workload errors (O abs, LSE abs, O rel):", e)
    # every row written: finite outputs everywhere
    assert bool(torch_isfinite_all(o)) and bool(torch_isfinite_all(l))


def torch_isfinite_all(t):
    import torch
    return torch.isfinite(t.float()).all().item()


# ------------------------------------------------------------------ MLA prefill

def _run_mla(cpa, strategy, C, rank, new_len, prefix, seed, out_f32=False, spiky=False, rows=None):
    import torch
    fn = cpa.cp_plan_zigzag if strategy == "zigzag" else cpa.cp_plan_interleave
    plan = fn(C, rank, new_len, prefix)
    ref_plan = (plans.plan_zigzag if strategy == "zigzag" else plans.plan_interleave)(C, rank, new_len, prefix)
    T_kv = int(sum(new_len) + (sum(prefix) if prefix else 0))
    rng = np.random.default_rng(seed)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((max(plan.n_local, 1), 64, 576)).astype(np.float32))[:plan.n_local]
    lx = rng.standard_normal((T_kv, 1, 576)).astype(np.float32)
    if spiky:
        lx[rng.integers(0, T_kv, size=max(1, T_kv // 40))] *= 5.0
    lb = synth.f32_to_bf16_bits(lx)
    scale = (6.0 if spiky else 1.0) / math.sqrt(576)
    o, l = cpa.attn_prefill_shard(H.bf16_tensor(qb), H.bf16_tensor(lb), None, plan.segments, scale,
                                  out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    _sync()
    if plan.n_local == 0:
        return
    ro, rl = att.prefill_shard(qb, lb, ref_plan.segments, scale, dv=512, rows=rows, decode=formats.bf16_bits_to_f64)
    go, gl = H.host(o), H.host(l)
    if rows is not None:
        go, gl = go[rows], gl[rows]
    chk = H.check_lowp_scaled if spiky else H.check_lowp
    chk(go, gl, ro, rl, f"MLA {strategy} C={C} r={rank} L={new_len} P={prefix}")


def test_prefill_mla_zigzag_prefix(cpa):
    for rank in range(2):
        _run_mla(cpa, "zigzag", 2, rank, [200], [70], 60 + rank)
    _run_mla(cpa, "zigzag", 4, 3, [130, 5], [0, 64], 62, out_f32=True)


def test_prefill_mla_interleave_ragged(cpa):
    _run_mla(cpa, "interleave", 3, 1, [90, 1, 140], [10, 0, 63], 63)


def test_prefill_mla_spiky(cpa):
    # planted large latents are large values too (value = latent): f32 output
    _run_mla(cpa, "zigzag", 2, 0, [300], [30], 64, spiky=True, out_f32=True)
