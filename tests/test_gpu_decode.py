"""GPU parity: LSE merge and split-KV decode shards against the oracle."""

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


def test_merge_worked_example_fig8(cpa, golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "merge_fig8.json")))
    # shard outputs and LSEs of the example: V = I4, GPU0 {0,2}, GPU1 {1,3}
    o = np.zeros((2, 1, 1, 4))
    o[0, 0, 0, [0, 2]] = g["local_probs"][0]
    o[1, 0, 0, [1, 3]] = g["local_probs"][1]
    lse = np.log(np.array(g["local_sums"], dtype=np.float64)).reshape(2, 1, 1)
    out, lo = cpa.attn_merge_states(H.f32_tensor(o), H.f32_tensor(lse))
    _sync()
    assert np.allclose(H.host(out)[0, 0], g["true_probs"], atol=1e-6)
    assert abs(H.host(lo)[0, 0] - math.log(8)) < 1e-6


@pytest.mark.parametrize("S,N,Hh,Dv", [(1, 3, 5, 8), (4, 7, 3, 128), (8, 64, 64, 512), (3, 2, 2, 1028),
                                         (12, 5, 3, 264), (16, 3, 4, 64), (9, 2, 3, 772)])
def test_merge_random_states(cpa, S, N, Hh, Dv):
    rng = np.random.default_rng(S * 1000 + Dv)
    o = rng.standard_normal((S, N, Hh, Dv)).astype(np.float32)
    lse = (rng.standard_normal((S, N, Hh)) * 4).astype(np.float32)
    if S > 1:
        lse[0, 0, :] = -np.inf          # an empty shard carries no mass
        lse[:, -1, -1] = -np.inf        # an all-empty row: O = 0, LSE = -inf
        lse[1 % S, 1 % N, 0] = 80.0     # large LSE values must not overflow
    ref_o, ref_l = att.merge_states(o.astype(np.float64), lse.astype(np.float64))
    out, lo = cpa.attn_merge_states(H.f32_tensor(o), H.f32_tensor(lse))
    _sync()
    H.check_f32(H.host(out), H.host(lo), ref_o, ref_l, "merge f32")
    import torch
    outb, lob = cpa.attn_merge_states(H.f32_tensor(o), H.f32_tensor(lse), out_dtype=torch.bfloat16)
    _sync()
    H.check_lowp(H.host(outb), H.host(lob), ref_o, ref_l, "merge bf16 out")


def _decode_case(cpa, B, Hq, Hkv, D, L, shards, qdt, kvdt, seed, ragged=False):
    """GQA decode: every shard against the oracle, then the merge against
    unsharded attention."""
    import torch
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(D)
    if qdt == "f32":
        q = rng.standard_normal((B, Hq, D)).astype(np.float32)
        qd, qv = H.f32_tensor(q), q.astype(np.float64)
    else:
        qb = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
        qd, qv = H.bf16_tensor(qb), formats.bf16_bits_to_f64(qb)
    kx = rng.standard_normal((B, L, Hkv, D)).astype(np.float32)
    vx = rng.standard_normal((B, L, Hkv, D)).astype(np.float32)
    sd, sc = None, None  # FP8: per-token scale (device, host)
    if kvdt == "f32":
        kd, vd, kv64, vv64 = H.f32_tensor(kx), H.f32_tensor(vx), kx.astype(np.float64), vx.astype(np.float64)
    elif kvdt == "fp8":
        kc, vc, sc = synth.gqa_kv_to_e4m3(kx, vx)
        kd, vd, sd = H.u8_tensor(kc), H.u8_tensor(vc), H.f32_tensor(sc)
        kv64, vv64 = kc, vc  # the oracle decodes the codes itself
    else:
        kb, vb = synth.f32_to_bf16_bits(kx), synth.f32_to_bf16_bits(vx)
        kd, vd, kv64, vv64 = H.bf16_tensor(kb), H.bf16_tensor(vb), formats.bf16_bits_to_f64(kb), formats.bf16_bits_to_f64(vb)
    odec = dict(decode=formats.e4m3_to_f64, kv_scale=sc) if kvdt == "fp8" else {}
    parts_o, parts_l = [], []
    for (s0, s1) in shards:
        beg = np.full(B, s0, np.int32)
        end = np.full(B, s1, np.int32)
        if ragged:  # per-request ranges inside the shard, one empty
            end = np.minimum(end, s0 + (np.arange(B) * 37) % max(1, s1 - s0 + 1)).astype(np.int32)
        o, l = cpa.attn_decode_shard(qd, kd, vd, H.i32_tensor(beg), H.i32_tensor(end), s1 - s0, scale, kv_scale=sd)
        _sync()
        ro, rl = att.decode_shard(qv, kv64, beg, end, scale, vcache=vv64, **odec)
        chk = H.check_f32 if (qdt == "f32" and kvdt == "f32") else H.check_lowp
        chk(H.host(o), H.host(l), ro, rl, f"shard {s0}:{s1}")
        parts_o.append(o)
        parts_l.append(l)
    if not ragged:
        mo, ml = cpa.attn_merge_states(torch.stack(parts_o), torch.stack(parts_l))
        _sync()
        fo, fl = att.decode_shard(qv, kv64, [0] * B, [L] * B, scale, vcache=vv64, **odec)
        chk = H.check_f32 if (qdt == "f32" and kvdt == "f32") else H.check_lowp
        chk(H.host(mo), H.host(ml), fo, fl, "merged vs unsharded")


def test_decode_gqa_f32_workload(cpa):
    """Split-KV decode + merge, fp32: batch 1, 8 query heads on 1 kv head,
    head dim 128, 4096-token context cut into 4 contiguous 1024-token shards."""
    c = synth.workload("gqa_decode_f32_4k")
    B, Hq, Hkv, D, L = c["B"], c["Hq"], c["Hkv"], c["Dqk"], c["L"]
    q = synth.f32_normal(1, 1, (B, Hq, D))
    k = synth.f32_normal(1, 2, (B, L, Hkv, D), chunk=1)
    v = synth.f32_normal(1, 3, (B, L, Hkv, D), chunk=1)
    import torch
    shards = plans.contiguous_shards(L, c["C"])
    qd, kd, vd = H.f32_tensor(q), H.f32_tensor(k), H.f32_tensor(v)
    po, pl = [], []
    for (s0, s1) in shards:
        o, l = cpa.attn_decode_shard(qd, kd, vd, H.i32_tensor([s0]), H.i32_tensor([s1]), s1 - s0, c["scale"])
        po.append(o); pl.append(l)
    mo, ml = cpa.attn_merge_states(torch.stack(po), torch.stack(pl))
    _sync()
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    for i, (s0, s1) in enumerate(shards):
        ro, rl = att.decode_shard(q64, k64, [s0], [s1], c["scale"], vcache=v64)
        H.check_f32(H.host(po[i]), H.host(pl[i]), ro, rl, f"shard {i}")
    fo, fl = att.decode_shard(q64, k64, [0], [L], c["scale"], vcache=v64)
    H.check_f32(H.host(mo), H.host(ml), fo, fl, "merged")


@pytest.mark.parametrize("B,Hq,Hkv,D,L,nsh", [(2, 8, 2, 64, 300, 3), (3, 32, 8, 128, 1000, 4), (1, 4, 4, 256, 77, 2)])
def test_decode_gqa_f32_shapes(cpa, B, Hq, Hkv, D, L, nsh):
    _decode_case(cpa, B, Hq, Hkv, D, L, plans.contiguous_shards(L, nsh), "f32", "f32", B * 7 + D)


def test_decode_gqa_bf16_and_ragged(cpa):
    _decode_case(cpa, 3, 16, 4, 128, 700, plans.contiguous_shards(700, 3), "bf16", "bf16", 17)
    _decode_case(cpa, 5, 8, 1, 128, 500, [(100, 400)], "bf16", "bf16", 18, ragged=True)


@pytest.mark.parametrize("B,Hq,Hkv,D,L,nsh,qdt", [(3, 16, 4, 128, 700, 3, "bf16"), (2, 8, 2, 64, 300, 2, "f32"),
                                                  (1, 4, 4, 256, 77, 2, "bf16")])
def test_decode_gqa_fp8(cpa, B, Hq, Hkv, D, L, nsh, qdt):
    """GQA over an FP8 E4M3 cache with one scale per token for its key and
    value (bf16 and f32 queries, head dims 64 / 128 / 256), every shard and
    the merge against the oracle, and ragged per-request ranges."""
    _decode_case(cpa, B, Hq, Hkv, D, L, plans.contiguous_shards(L, nsh), qdt, "fp8", 31 + D)
    _decode_case(cpa, 5, 8, 2, D, 500, [(100, 400)], qdt, "fp8", 32 + D, ragged=True)


@pytest.mark.parametrize("kvdt", ["bf16", "fp8", "f32"])
def test_decode_gqa_group_over_16_heads(cpa, kvdt):
    """A GQA group wider than the 16 heads of one workgroup (40 query heads on
    2 kv heads: 20 per group, two head blocks, the second with 4 heads)."""
    qdt = "f32" if kvdt == "f32" else "bf16"
    _decode_case(cpa, 2, 40, 2, 128, 400, plans.contiguous_shards(400, 2), qdt, kvdt, 55)


def test_decode_gqa_rejects_misaligned_rows(cpa):
    """K/V rows are streamed in 16-byte pieces: a cache view whose token
    stride is not a multiple of 16 bytes is rejected before any launch."""
    import torch
    q = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    base = torch.zeros((1, 40, 1, 68), dtype=torch.bfloat16, device="cuda")
    k = base[..., :64]  # token stride 68 elements = 136 bytes
    be = H.i32_tensor([0])
    en = H.i32_tensor([40])
    with pytest.raises(cpa.CpaError) as ex:
        cpa.attn_decode_shard(q, k, k, be, en, 40, 0.125)
    assert ex.value.status == cpa.CPA_E_INVAL


def _mla_inputs(B, L, fp8, seed, std=0.5):
    rng = np.random.default_rng(seed)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 576)).astype(np.float32))
    x = (rng.standard_normal((B, L, 1, 576)) * std).astype(np.float32)
    if fp8:
        codes, sc = synth.f32_to_e4m3(x)
        return qb, codes, sc[..., 0]
    return qb, synth.f32_to_bf16_bits(x), None


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,L,ranges", [
    (2, 64, [(0, 64)]),                      # exactly two tiles
    (3, 1000, [(0, 333), (333, 1000)]),      # ragged tails, several splits
    (4, 130, [(5, 5), (0, 1), (7, 130)]),    # empty shard, single key
    (8, 1000, [(0, 1000), (100, 900)]),      # 8 requests: each request's splits on one XCD
    (16, 600, [(0, 600)]),
])
def test_decode_mla_small(cpa, fp8, B, L, ranges):
    import torch
    qb, cache, sc = _mla_inputs(B, L, fp8, B * 100 + L + fp8)
    scale = 1.0 / math.sqrt(576)
    qd = H.bf16_tensor(qb)
    cd = H.u8_tensor(cache) if fp8 else H.bf16_tensor(cache)
    sd = H.f32_tensor(sc) if fp8 else None
    q64 = formats.bf16_bits_to_f64(qb)
    dec = formats.e4m3_to_f64 if fp8 else formats.bf16_bits_to_f64
    for (s0, s1) in ranges:
        beg, end = np.full(B, s0, np.int32), np.full(B, s1, np.int32)
        o, l = cpa.attn_decode_shard(qd, cd, None, H.i32_tensor(beg), H.i32_tensor(end), s1 - s0, scale,
                                     kv_scale=sd)
        _sync()
        ro, rl = att.decode_shard(q64, cache, beg, end, scale, dv=512, decode=dec, kv_scale=sc)
        H.check_lowp(H.host(o), H.host(l), ro, rl, f"mla fp8={fp8} [{s0},{s1})")
        if s1 == s0:
            assert np.all(H.host(o) == 0) and np.all(np.isneginf(H.host(l)))


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_mla_spiky_scores(cpa, fp8):
    """Planted keys with large logits exercise the running-max rescale."""
    B, L = 2, 512
    qb, cache, sc = _mla_inputs(B, L, fp8, 77 + fp8)
    rng = np.random.default_rng(5)
    q64 = formats.bf16_bits_to_f64(qb)
    scale = 8.0 / math.sqrt(576)
    if not fp8:
        # copy a query row into a few late keys so their scores dominate
        for t in (100, 301, 510):
            cache[:, t, 0, :] = qb[:, 3, :]
    qd = H.bf16_tensor(qb)
    cd = H.u8_tensor(cache) if fp8 else H.bf16_tensor(cache)
    sd = H.f32_tensor(sc) if fp8 else None
    dec = formats.e4m3_to_f64 if fp8 else formats.bf16_bits_to_f64
    beg, end = np.zeros(B, np.int32), np.full(B, L, np.int32)
    o, l = cpa.attn_decode_shard(qd, cd, None, H.i32_tensor(beg), H.i32_tensor(end), L, scale, kv_scale=sd)
    _sync()
    ro, rl = att.decode_shard(q64, cache, beg, end, scale, dv=512, decode=dec, kv_scale=sc)
    H.check_lowp(H.host(o), H.host(l), ro, rl, "mla spiky")


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_mla_workspace_reuse_ragged(cpa, fp8):
    """One caller workspace (random bytes at first) reused by consecutive
    calls with per-request ragged ranges: the split states and the per-call
    arrival counters in it must never leak between calls. Request 0 is empty,
    request 1 has a single key."""
    import torch
    B, L = 4, 1000
    qb, cache, sc = _mla_inputs(B, L, fp8, 991 + fp8)
    scale = 1.0 / math.sqrt(576)
    qd = H.bf16_tensor(qb)
    cd = H.u8_tensor(cache) if fp8 else H.bf16_tensor(cache)
    sd = H.f32_tensor(sc) if fp8 else None
    q64 = formats.bf16_bits_to_f64(qb)
    dec = formats.e4m3_to_f64 if fp8 else formats.bf16_bits_to_f64
    need = cpa.attn_decode_workspace_size(B, 64, 512, L)
    ws = torch.from_numpy(np.random.default_rng(3).integers(0, 256, need, dtype=np.uint8)).to(H.dev())
    for beg, end in (([5, 0, 10, 0], [5, 1, 700, 1000]),
                     ([0, 3, 0, 999], [1000, 4, 1, 1000]),
                     ([5, 0, 10, 0], [5, 1, 700, 1000])):
        beg, end = np.array(beg, np.int32), np.array(end, np.int32)
        o, l = cpa.attn_decode_shard(qd, cd, None, H.i32_tensor(beg), H.i32_tensor(end), L, scale,
                                     kv_scale=sd, workspace=ws)
        _sync()
        ro, rl = att.decode_shard(q64, cache, beg, end, scale, dv=512, decode=dec, kv_scale=sc)
        H.check_lowp(H.host(o), H.host(l), ro, rl, f"mla workspace reuse fp8={fp8}")
        empty = beg == end
        assert np.all(H.host(o)[empty] == 0) and np.all(np.isneginf(H.host(l)[empty]))
