"""GPU parity: multi-query (speculative / MTP) decode shards against the
oracle -- each rank's partial state, and the merged states against causal
attention of the query rows over the whole request."""

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


def _local(layout, cache, L_list, C, r, n_repl=0, repl=None):
    """Rank r's local cache [B, rows, ...] built on the host from the full
    cache (replicated rows first for round robin)."""
    B = cache.shape[0]
    held = []
    for L in L_list:
        if layout == "contiguous":
            s0, s1 = plans.contiguous_shards(L, C)[r]
            held.append(list(range(s0, s1)))
        else:
            held.append(plans.round_robin_own_tokens(L, C, r))
    rows = n_repl + max(1, max(len(h) for h in held))
    loc = np.zeros((B, rows) + cache.shape[2:], cache.dtype)
    for b, h in enumerate(held):
        if n_repl:
            loc[b, :n_repl] = repl[b]
        loc[b, n_repl:n_repl + len(h)] = cache[b, h]
    return loc


def _mla_case(cpa, layout, fp8, B, Q, L_list, C, seed, n_repl=0):
    import torch
    rng = np.random.default_rng(seed)
    Lm = max(L_list)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, Q, 64, 576)).astype(np.float32))
    x = (rng.standard_normal((B, Lm + n_repl, 1, 576)) * 0.5).astype(np.float32)
    if fp8:
        cache, sc = synth.f32_to_e4m3(x)
        sc = sc[..., 0]
    else:
        cache, sc = synth.f32_to_bf16_bits(x), None
    main, repl = cache[:, n_repl:], cache[:, :n_repl]
    smain, srepl = (sc[:, n_repl:], sc[:, :n_repl]) if fp8 else (None, None)
    scale = 1.0 / math.sqrt(576)
    q64 = formats.bf16_bits_to_f64(qb)
    dec = formats.e4m3_to_f64 if fp8 else formats.bf16_bits_to_f64
    qd = H.bf16_tensor(qb)
    lay = cpa.CPA_LAYOUT_CONTIGUOUS if layout == "contiguous" else cpa.CPA_LAYOUT_ROUND_ROBIN
    po, pl = [], []
    for r in range(C):
        loc = _local(layout, main, L_list, C, r, n_repl, repl)
        lsc = _local(layout, smain, L_list, C, r, n_repl, srepl) if fp8 else None
        beg, end, rows = cpa.cp_plan_multi_query(lay, C, r, L_list, Q, n_repl, 0)
        rb, re_ = plans.plan_multi_query(layout, C, r, L_list, Q, n_repl, 0)
        assert np.array_equal(beg, rb) and np.array_equal(end, re_)
        cd = H.u8_tensor(loc) if fp8 else H.bf16_tensor(loc)
        o, l = cpa.attn_decode_shard_mq(qd, cd, None, H.i32_tensor(beg), H.i32_tensor(end),
                                        int((end.reshape(B, Q) - beg[:, None]).max()), scale,
                                        kv_scale=H.f32_tensor(lsc) if fp8 else None)
        _sync()
        ro, rl = att.decode_shard_mq(q64, loc, beg, end, scale, dv=512, decode=dec, kv_scale=lsc)
        H.check_lowp(H.host(o), H.host(l), ro, rl, f"mq {layout} fp8={fp8} rank {r}")
        po.append(o)
        pl.append(l)
    # merged over the ranks = causal attention of every query row over its request
    mo, ml = cpa.attn_merge_states(torch.stack(po).reshape(C, B * Q, 64, 512), torch.stack(pl).reshape(C, B * Q, 64))
    _sync()
    full = np.concatenate([repl, main], axis=1)
    fsc = np.concatenate([srepl, smain], axis=1) if fp8 else None
    fb = np.zeros(B, np.int32)
    fe = np.array([n_repl + L - Q + k + 1 for L in L_list for k in range(Q)], np.int32)
    ro, rl = att.decode_shard_mq(q64, full, fb, fe, scale, dv=512, decode=dec, kv_scale=fsc)
    H.check_lowp(H.host(mo).reshape(B, Q, 64, 512), H.host(ml).reshape(B, Q, 64), ro, rl,
                 f"mq {layout} fp8={fp8} merged vs causal")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("layout,Q,L_list,C", [
    ("contiguous", 4, [700, 6, 333], 2),    # ragged; rank 1 of request 1 starts after row 0 (an empty row)
    ("contiguous", 2, [64, 65], 1),         # exactly two tiles / one key past them
    ("round_robin", 3, [500, 3, 97], 3),
    ("contiguous", 2, [400, 9, 333, 64, 65, 2, 700, 250], 2),  # 8 requests: each request's workgroups on one XCD
])
def test_mla_multi_query(cpa, fp8, layout, Q, L_list, C):
    _mla_case(cpa, layout, fp8, len(L_list), Q, L_list, C, seed=Q * 100 + C + fp8)


def test_mla_multi_query_replicated_rows_q8(cpa):
    _mla_case(cpa, "round_robin", False, 2, 8, [300, 40], 4, seed=41, n_repl=5)


@pytest.mark.parametrize("fp8", [False, True])
def test_mla_q1_matches_single_query_entry(cpa, fp8):
    """Q = 1 through the multi-query entry is the single-query decode: the
    same kernel on the same work, so the results are identical."""
    import torch
    B, L = 5, 900
    rng = np.random.default_rng(7 + fp8)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 576)).astype(np.float32))
    x = (rng.standard_normal((B, L, 1, 576)) * 0.5).astype(np.float32)
    if fp8:
        codes, sc = synth.f32_to_e4m3(x)
        cd, sd = H.u8_tensor(codes), H.f32_tensor(sc[..., 0])
    else:
        cd, sd = H.bf16_tensor(synth.f32_to_bf16_bits(x)), None
    beg = H.i32_tensor([0, 3, 10, 0, 899])
    end = H.i32_tensor([900, 3, 500, 1, 900])
    qd = H.bf16_tensor(qb)
    o1, l1 = cpa.attn_decode_shard(qd, cd, None, beg, end, L, 1 / 24, kv_scale=sd)
    o2, l2 = cpa.attn_decode_shard_mq(qd[:, None], cd, None, beg, end, L, 1 / 24, kv_scale=sd)
    _sync()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


@pytest.mark.parametrize("kvdt", ["f32", "bf16"])
def test_gqa_multi_query(cpa, kvdt):
    """GQA 16/4, d=128: Q=3 query rows, round robin over C=2 with 2
    replicated rows, and contiguous over C=3."""
    import torch
    rng = np.random.default_rng(23)
    B, Q, Hq, Hkv, D = 3, 3, 16, 4, 128
    L_list = [260, 5, 130]
    scale = 1.0 / math.sqrt(D)
    q = rng.standard_normal((B, Q, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, max(L_list), Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, max(L_list), Hkv, D)).astype(np.float32)
    if kvdt == "bf16":
        qb, kb, vb = (synth.f32_to_bf16_bits(a) for a in (q, k, v))
        qd, q64 = H.bf16_tensor(qb), formats.bf16_bits_to_f64(qb)
        k64, v64 = formats.bf16_bits_to_f64(kb), formats.bf16_bits_to_f64(vb)
        up = H.bf16_tensor
        ks, vs = kb, vb
        chk = H.check_lowp
    else:
        qd, q64, k64, v64 = H.f32_tensor(q), q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
        up = H.f32_tensor
        ks, vs = k, v
        chk = H.check_f32
    for layout, C in (("round_robin", 2), ("contiguous", 3)):
        lay = cpa.CPA_LAYOUT_CONTIGUOUS if layout == "contiguous" else cpa.CPA_LAYOUT_ROUND_ROBIN
        n_repl = 2 if layout == "round_robin" else 0
        rk = ks[:, :n_repl]
        rv = vs[:, :n_repl]
        po, pl = [], []
        for r in range(C):
            lk = _local(layout, ks, L_list, C, r, n_repl, rk)
            lv = _local(layout, vs, L_list, C, r, n_repl, rv)
            beg, end, _ = cpa.cp_plan_multi_query(lay, C, r, L_list, Q, n_repl, 1 % C if n_repl else 0)
            o, l = cpa.attn_decode_shard_mq(qd, up(lk), up(lv), H.i32_tensor(beg), H.i32_tensor(end),
                                            max(L_list) + n_repl, scale)
            _sync()
            lk64 = formats.bf16_bits_to_f64(lk) if kvdt == "bf16" else lk.astype(np.float64)
            lv64 = formats.bf16_bits_to_f64(lv) if kvdt == "bf16" else lv.astype(np.float64)
            ro, rl = att.decode_shard_mq(q64, lk64, beg, end, scale, vcache=lv64)
            chk(H.host(o), H.host(l), ro, rl, f"gqa mq {layout} rank {r}")
            po.append(o)
            pl.append(l)
        mo, ml = cpa.attn_merge_states(torch.stack(po).reshape(C, B * Q, Hq, D), torch.stack(pl).reshape(C, B * Q, Hq))
        _sync()
        fk = np.concatenate([k64[:, :n_repl], k64], axis=1)
        fv = np.concatenate([v64[:, :n_repl], v64], axis=1)
        fe = np.array([n_repl + L - Q + kk + 1 for L in L_list for kk in range(Q)], np.int32)
        ro, rl = att.decode_shard_mq(q64, fk, np.zeros(B, np.int32), fe, scale, vcache=fv)
        chk(H.host(mo).reshape(B, Q, Hq, D), H.host(ml).reshape(B, Q, Hq), ro, rl, f"gqa mq {layout} merged")


def test_multi_query_strided_query_and_output_checks(cpa):
    """Query rows taken from a wider buffer (strided rows) give the same
    result as a packed copy; outputs whose (request, row) dims do not
    collapse into one row index are rejected before any launch."""
    import torch
    rng = np.random.default_rng(4)
    B, Q, L = 2, 3, 200
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, Q + 2, 64, 576)).astype(np.float32))
    cb = synth.f32_to_bf16_bits((rng.standard_normal((B, L, 1, 576)) * 0.5).astype(np.float32))
    qwide, cd = H.bf16_tensor(qb), H.bf16_tensor(cb)
    beg = H.i32_tensor([0, 0])
    end = H.i32_tensor([198, 199, 200, 100, 150, 0])
    o1, l1 = cpa.attn_decode_shard_mq(qwide[:, 1:1 + Q], cd, None, beg, end, L, 1 / 24)
    o2, l2 = cpa.attn_decode_shard_mq(qwide[:, 1:1 + Q].contiguous(), cd, None, beg, end, L, 1 / 24)
    _sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    bad_o = torch.empty((B, Q + 1, 64, 512), dtype=torch.float32, device="cuda")[:, :Q]
    with pytest.raises(cpa.CpaError):
        cpa.attn_decode_shard_mq(qwide[:, :Q], cd, None, beg, end, L, 1 / 24, o_part=bad_o)
