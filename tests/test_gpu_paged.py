"""GPU parity: split-KV decode over a paged cache (attn_decode_shard_paged)
against the oracle's paged decode, and against the contiguous decode on the
same rows (bit-identical: only the addressing differs)."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as att
from oracle import formats
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


def _ranges(B, n_log, seed, full=False):
    """Logical [begin, end) per request inside n_log positions: ragged, one
    empty range, one full range."""
    rng = np.random.default_rng(seed)
    if full:
        return np.zeros(B, np.int32), np.full(B, n_log, np.int32)
    beg = rng.integers(0, n_log // 3, B).astype(np.int32)
    end = rng.integers(n_log // 2, n_log + 1, B).astype(np.int32)
    beg[0], end[0] = 0, n_log
    if B > 2:
        end[1] = beg[1]  # empty
    return beg, end


def _table(B, n_blocks, n_pages, seed, shared=0, bad=False):
    t = synth.page_table(21, seed, B, n_blocks, n_pages, shared=shared)
    if bad:  # entries outside the pool read page 0
        t[0, 1] = -1
        t[-1, -1] = n_pages + 5
    return t


def _gather(pool, table, ps, n_log):
    """The contiguous per-request cache the pool holds under the table
    ([B, n_log, ...]); entries outside the pool read page 0."""
    n_pages = pool.shape[0] // ps
    t = np.where((table >= 0) & (table < n_pages), table, 0).astype(np.int64)
    pos = np.arange(n_log)
    rows = t[:, pos // ps] * ps + pos % ps
    return pool[rows]


@pytest.mark.parametrize("fp8,ps,shared,bad,B", [(False, 64, 0, False, 4), (False, 16, 2, True, 4), (True, 32, 0, False, 4),
                                                 (True, 256, 1, True, 4), (True, 1, 0, False, 4),
                                                 (False, 64, 1, False, 8), (True, 64, 0, True, 8)])
def test_mla_paged_vs_oracle(cpa, fp8, ps, shared, bad, B):
    """B = 8: the requests divide over the 8 XCDs, so each request's splits
    run on one XCD (the other work-unit order)."""
    H_, L = 64, 700
    n_blocks = (L + ps - 1) // ps
    n_pages = shared + B * (n_blocks - shared) + 3
    table = _table(B, n_blocks, n_pages, ps + 7 * fp8, shared=shared, bad=bad)
    rng = np.random.default_rng(ps)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, H_, 576)).astype(np.float32))
    x = (rng.standard_normal((n_pages * ps, 1, 576)) * 0.5).astype(np.float32)
    beg, end = _ranges(B, L, ps)
    scale = 1.0 / math.sqrt(576)
    if fp8:
        codes, sc = synth.f32_to_e4m3(x)
        kp, sp = H.u8_tensor(codes), H.f32_tensor(sc[:, 0])
        ref_pool, odec = codes, dict(decode=formats.e4m3_to_f64, kv_scale=sc[:, 0])
    else:
        bits = synth.f32_to_bf16_bits(x)
        kp, sp = H.bf16_tensor(bits), None
        ref_pool, odec = formats.bf16_bits_to_f64(bits), {}
    o, l = cpa.attn_decode_shard_paged(H.bf16_tensor(qb), kp, None, H.i32_tensor(table), ps, H.i32_tensor(beg),
                                       H.i32_tensor(end), L, scale, kv_scale=sp)
    _sync()
    ro, rl = att.decode_shard_paged(formats.bf16_bits_to_f64(qb), ref_pool, table, ps, beg, end, scale, dv=512,
                                    **odec)
    H.check_lowp(H.host(o), H.host(l), ro, rl, f"MLA paged fp8={fp8} ps={ps}")


@pytest.mark.parametrize("kvdt,D,ps", [("bf16", 128, 16), ("fp8", 128, 64), ("f32", 64, 32), ("bf16", 256, 8)])
def test_gqa_paged_vs_oracle(cpa, kvdt, D, ps):
    B, Hq, Hkv, L = 3, 16, 4, 500
    n_blocks = (L + ps - 1) // ps
    n_pages = B * n_blocks + 2
    table = _table(B, n_blocks, n_pages, D + ps, bad=True)
    rng = np.random.default_rng(D * ps)
    scale = 1.0 / math.sqrt(D)
    kx = rng.standard_normal((n_pages * ps, Hkv, D)).astype(np.float32)
    vx = rng.standard_normal((n_pages * ps, Hkv, D)).astype(np.float32)
    beg, end = _ranges(B, L, D + ps)
    if kvdt == "f32":
        q = rng.standard_normal((B, Hq, D)).astype(np.float32)
        qd, qv = H.f32_tensor(q), q.astype(np.float64)
    else:
        qb = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
        qd, qv = H.bf16_tensor(qb), formats.bf16_bits_to_f64(qb)
    sd, odec = None, {}
    if kvdt == "f32":
        kd, vd, k64, v64 = H.f32_tensor(kx), H.f32_tensor(vx), kx.astype(np.float64), vx.astype(np.float64)
    elif kvdt == "fp8":
        kc, vc, sc = synth.gqa_kv_to_e4m3(kx[None], vx[None])
        kc, vc, sc = kc[0], vc[0], sc[0]
        kd, vd, sd, k64, v64 = H.u8_tensor(kc), H.u8_tensor(vc), H.f32_tensor(sc), kc, vc
        odec = dict(decode=formats.e4m3_to_f64, kv_scale=sc)
    else:
        kb, vb = synth.f32_to_bf16_bits(kx), synth.f32_to_bf16_bits(vx)
        kd, vd = H.bf16_tensor(kb), H.bf16_tensor(vb)
        k64, v64 = formats.bf16_bits_to_f64(kb), formats.bf16_bits_to_f64(vb)
    o, l = cpa.attn_decode_shard_paged(qd, kd, vd, H.i32_tensor(table), ps, H.i32_tensor(beg), H.i32_tensor(end),
                                       L, scale, kv_scale=sd)
    _sync()
    ro, rl = att.decode_shard_paged(qv, k64, table, ps, beg, end, scale, vpool=v64, **odec)
    chk = H.check_f32 if kvdt == "f32" else H.check_lowp
    chk(H.host(o), H.host(l), ro, rl, f"GQA paged {kvdt} D={D} ps={ps}")


@pytest.mark.parametrize("fp8", [False, True])
def test_mla_paged_equals_contiguous(cpa, fp8):
    """The same rows through a page table and as a contiguous cache give
    bit-identical results (same splits, tiles and arithmetic)."""
    import torch
    B, L, ps = 8, 3000, 64
    n_blocks = L // ps + 1
    n_pages = B * n_blocks
    table = _table(B, n_blocks, n_pages, 99 + fp8)
    rng = np.random.default_rng(5 + fp8)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 576)).astype(np.float32))
    x = (rng.standard_normal((n_pages * ps, 1, 576)) * 0.5).astype(np.float32)
    beg, end = _ranges(B, L, 3)
    if fp8:
        codes, sc = synth.f32_to_e4m3(x)
        pool, spool = codes, sc[:, 0]
        kp, sp = H.u8_tensor(pool), H.f32_tensor(spool)
        kc, scc = H.u8_tensor(_gather(pool, table, ps, L)), H.f32_tensor(_gather(spool, table, ps, L))
    else:
        pool = synth.f32_to_bf16_bits(x)
        kp, sp = H.bf16_tensor(pool), None
        kc, scc = H.bf16_tensor(_gather(pool, table, ps, L)), None
    qd = H.bf16_tensor(qb)
    o1, l1 = cpa.attn_decode_shard_paged(qd, kp, None, H.i32_tensor(table), ps, H.i32_tensor(beg),
                                         H.i32_tensor(end), L, 0.05, kv_scale=sp)
    o2, l2 = cpa.attn_decode_shard(qd, kc, None, H.i32_tensor(beg), H.i32_tensor(end), L, 0.05, kv_scale=scc)
    _sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_paged_equals_contiguous(cpa):
    import torch
    B, Hq, Hkv, D, L, ps = 4, 32, 8, 128, 2000, 32
    n_blocks = L // ps + 1
    n_pages = B * n_blocks
    table = _table(B, n_blocks, n_pages, 55)
    rng = np.random.default_rng(9)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    kb = synth.f32_to_bf16_bits(rng.standard_normal((n_pages * ps, Hkv, D)).astype(np.float32))
    vb = synth.f32_to_bf16_bits(rng.standard_normal((n_pages * ps, Hkv, D)).astype(np.float32))
    beg, end = _ranges(B, L, 4)
    qd = H.bf16_tensor(qb)
    o1, l1 = cpa.attn_decode_shard_paged(qd, H.bf16_tensor(kb), H.bf16_tensor(vb), H.i32_tensor(table), ps,
                                         H.i32_tensor(beg), H.i32_tensor(end), L, 0.08)
    o2, l2 = cpa.attn_decode_shard(qd, H.bf16_tensor(_gather(kb, table, ps, L)),
                                   H.bf16_tensor(_gather(vb, table, ps, L)), H.i32_tensor(beg), H.i32_tensor(end),
                                   L, 0.08)
    _sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_many_pages_more_splits(cpa):
    """Page size 1 and 4096-token ranges for 64 requests: a split of the
    usual plan (4 per request) would touch more pages than one split keeps on
    chip, so the host plans more splits; parity holds (requests 0, 37, 63
    checked)."""
    B, L, ps = 64, 4096, 1
    table = _table(B, L, B * L, 77)
    rng = np.random.default_rng(77)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 576)).astype(np.float32))
    bits = synth.f32_to_bf16_bits((rng.standard_normal((B * L, 1, 576)) * 0.5).astype(np.float32))
    beg, end = np.zeros(B, np.int32), np.full(B, L, np.int32)
    assert cpa.attn_decode_paged_workspace_size(B, 64, 512, L, ps) > cpa.attn_decode_workspace_size(B, 64, 512, L)
    o, l = cpa.attn_decode_shard_paged(H.bf16_tensor(qb), H.bf16_tensor(bits), None, H.i32_tensor(table), ps,
                                       H.i32_tensor(beg), H.i32_tensor(end), L, 0.04)
    _sync()
    rows = [0, 37, 63]
    ro, rl = att.decode_shard_paged(formats.bf16_bits_to_f64(qb), formats.bf16_bits_to_f64(bits), table, ps, beg,
                                    end, 0.04, dv=512, batch=rows)
    H.check_lowp(H.host(o)[rows], H.host(l)[rows], ro[rows], rl[rows], "MLA paged, page size 1")


def test_paged_rejects_bad_arguments(cpa):
    import torch
    q = H.bf16_tensor(np.zeros((2, 64, 576), np.uint16))
    pool = H.bf16_tensor(np.zeros((96, 1, 576), np.uint16))
    t = H.i32_tensor(np.zeros((2, 3), np.int32))
    r = H.i32_tensor(np.zeros(2, np.int32))
    for ps in (0, 24, 1 << 21):  # not a power of two in [1, 2^20]
        with pytest.raises(cpa.CpaError) as ex:
            cpa.attn_decode_shard_paged(q, pool, None, t, ps, r, r, 10, 0.1)
        assert ex.value.status == 1
    with pytest.raises(cpa.CpaError) as ex:  # rows not a multiple of the page size
        cpa.attn_decode_shard_paged(q, pool, None, t, 64, r, r, 10, 0.1)
    assert ex.value.status == 1
    _sync()
