"""GPU parity: round-robin decode ownership -- local caches written by slot
(rank = slot mod C, row = slot / C), C partial decode launches over them and
the LSE merge, against the float64 oracle over the unsharded cache; entries
replicated on every rank are counted by one designated rank only."""

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


def _inputs(B, Lmax, n_repl, fp8, seed):
    rng = np.random.default_rng(seed)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 576)).astype(np.float32))
    x = (rng.standard_normal((B, n_repl + Lmax, 1, 576)) * 0.5).astype(np.float32)
    if fp8:
        codes, sc = synth.f32_to_e4m3(x)
        return qb, codes, sc[..., 0].astype(np.float32)
    return qb, synth.f32_to_bf16_bits(x), None


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("C,ctx,n_repl,repl_rank", [
    (4, [1000, 37, 2], 3, 1),    # ragged contexts, three replicated entries, designated rank 1
    (3, [65, 0, 130], 0, 0),     # an empty request, nothing replicated
    (8, [5, 2048, 1], 2, 7),     # more ranks than tokens for some requests
])
def test_round_robin_decode_matches_unsharded(cpa, fp8, C, ctx, n_repl, repl_rank):
    import torch
    B, Lmax = len(ctx), max(ctx)
    qb, cache, sc = _inputs(B, Lmax, n_repl, fp8, 1000 * C + Lmax + fp8)
    # cache rows [0, n_repl): the replicated entries; rows n_repl + p: slot p
    dev = H.dev()
    cdt = torch.uint8 if fp8 else torch.bfloat16
    full = (H.u8_tensor(cache) if fp8 else H.bf16_tensor(cache))[:, :, 0, :]      # [B, n_repl + Lmax, 576]
    full_sc = H.f32_tensor(sc) if fp8 else None                                    # [B, n_repl + Lmax]
    # the entries to write: every stored slot of every request
    req = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(ctx)])
    slot = np.concatenate([np.arange(L, dtype=np.int64) for L in ctx])
    src = full[torch.from_numpy(req).long().to(dev), torch.from_numpy(n_repl + slot).to(dev)].contiguous()
    src_sc = full_sc[torch.from_numpy(req).long().to(dev), torch.from_numpy(n_repl + slot).to(dev)].contiguous() \
        if fp8 else None
    req_d, slot_d = H.i32_tensor(req), torch.from_numpy(slot).to(dev)
    q = H.bf16_tensor(qb)
    scale = 1.0 / math.sqrt(576)
    o_parts, l_parts = [], []
    for r in range(C):
        beg, end, rows = cpa.cp_plan_round_robin(C, r, ctx, n_repl, repl_rank)
        local = torch.zeros((B, max(rows, 1), 1, 576), dtype=cdt, device=dev)
        local[:, :n_repl, 0] = full[:, :n_repl]
        cpa.attn_cache_write_round_robin(C, r, src, slot_d, req_d, local[:, :, 0, :], n_repl=n_repl)
        lsc = None
        if fp8:
            lsc = torch.ones((B, max(rows, 1)), dtype=torch.float32, device=dev)
            lsc[:, :n_repl] = full_sc[:, :n_repl]
            cpa.attn_cache_write_round_robin(C, r, src_sc[:, None], slot_d, req_d, lsc[:, :, None], n_repl=n_repl)
        torch.cuda.synchronize()
        # the written local cache holds exactly this rank's slots, in order (bit-exact)
        got = local.cpu().numpy() if fp8 else local.view(torch.int16).cpu().numpy().view(np.uint16)
        for b, L in enumerate(ctx):
            own = plans.round_robin_own_tokens(L, C, r)
            want = cache[b, [n_repl + p for p in own], 0]
            assert np.array_equal(got[b, n_repl:n_repl + len(own), 0], want)
            if fp8:
                assert np.array_equal(lsc.cpu().numpy()[b, n_repl:n_repl + len(own)], sc[b, [n_repl + p for p in own]])
        o, l = cpa.attn_decode_shard(q, local, None, H.i32_tensor(beg), H.i32_tensor(end), int(max(end - beg)),
                                     scale, kv_scale=lsc)
        o_parts.append(o)
        l_parts.append(l)
    mo, ml = cpa.attn_merge_states(torch.stack(o_parts), torch.stack(l_parts))
    torch.cuda.synchronize()
    # oracle: every request over its replicated entries and all its slots, each once
    dec = formats.e4m3_to_f64 if fp8 else formats.bf16_bits_to_f64
    ro, rl = att.decode_shard(formats.bf16_bits_to_f64(qb), cache, np.zeros(B, np.int32),
                              np.array([n_repl + L for L in ctx], np.int32), scale, dv=512, decode=dec,
                              kv_scale=sc)
    H.check_lowp(H.host(mo), H.host(ml), ro, rl, f"round robin C={C} fp8={fp8}")


def test_cache_write_skips_foreign_and_out_of_range_entries(cpa):
    import torch
    dev = H.dev()
    src = torch.arange(6 * 8, dtype=torch.float32, device=dev).reshape(6, 8)
    slot = torch.tensor([0, 1, 2, 5, -1, 9], dtype=torch.int64, device=dev)
    req = torch.tensor([0, 0, 1, 1, 0, 0], dtype=torch.int32, device=dev)
    dst = torch.full((2, 2, 8), -7.0, dtype=torch.float32, device=dev)
    cpa.attn_cache_write_round_robin(2, 1, src, slot, req, dst, n_repl=0)   # rank 1 of 2: odd slots
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    s = src.cpu().numpy()
    assert np.array_equal(d[0, 0], s[1])            # request 0, slot 1 -> row 0
    assert np.all(d[0, 1] == -7.0)                  # slot 9 -> row 4: past the cache, skipped
    assert np.all(d[1] == -7.0)                     # slot 2 is rank 0's; slot 5 -> row 2: past the cache
