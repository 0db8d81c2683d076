"""attn_decode_shard_noalloc: the decode entry point that allocates nothing
(its split states live in the library's per-device scratch array) gives the
same results as attn_decode_shard with a caller workspace, bit for bit (same
kernels, same split), on consecutive calls whose second input is smaller."""

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cpa():
    import torch
    import context_attention_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _nan(shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _both(cpa, q, cache, vcache, beg, end, max_len, scale, kv_scale=None):
    import torch
    B, Hq = q.shape[0], q.shape[1]
    Dv = vcache.shape[-1] if vcache is not None else 512
    b = H.i32_tensor(beg)
    e = H.i32_tensor(end)
    ws_n = cpa.attn_decode_workspace_size(B, Hq, Dv, max_len)
    ws = torch.full((max(ws_n, 1),), 255, dtype=torch.uint8, device="cuda")
    o_ref, l_ref = _nan((B, Hq, Dv)), _nan((B, Hq))
    cpa.attn_decode_shard(q, cache, vcache, b, e, max_len, scale, kv_scale=kv_scale, o_part=o_ref, lse_part=l_ref,
                          workspace=ws)
    o, l = _nan((B, Hq, Dv)), _nan((B, Hq))
    cpa.attn_decode_shard_noalloc(q, cache, vcache, b, e, max_len, scale, o, l, kv_scale=kv_scale)
    torch.cuda.synchronize()
    return ws_n, (o, l), (o_ref, l_ref)


def _same(got, ref):
    import torch
    (o, l), (o_ref, l_ref) = got, ref
    assert bool(torch.isfinite(o).all()), "unwritten output"
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_mla_two_calls_second_smaller(cpa):
    """MLA latent cache (bf16, then FP8 + per-token scale): a 64-request call
    (4-way internal split, 33.6 MB of split states), then an 8-request call
    with shorter, ragged ranges; each equals attn_decode_shard bit for bit."""
    rng = np.random.default_rng(7)
    for fp8 in (False, True):
        calls = [(64, 4096, np.zeros(64, np.int32), np.full(64, 4096, np.int32)),
                 (8, 1500, rng.integers(0, 300, 8).astype(np.int32), rng.integers(700, 1500, 8).astype(np.int32))]
        for B, L, beg, end in calls:
            q = H.bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 576)).astype(np.float32)))
            x = (rng.standard_normal((B, L, 1, 576)) * 0.5).astype(np.float32)
            if fp8:
                codes, sc = synth.f32_to_e4m3(x)
                cache, kvs = H.u8_tensor(codes), H.f32_tensor(sc[..., 0])
            else:
                cache, kvs = H.bf16_tensor(synth.f32_to_bf16_bits(x)), None
            max_len = int((end - beg).max())
            ws_n, got, ref = _both(cpa, q, cache, None, beg, end, max_len, 1 / 24, kv_scale=kvs)
            assert ws_n > 0, "the case must use the split scratch"
            _same(got, ref)


def test_noalloc_gqa_two_calls_second_smaller(cpa):
    """GQA f32 cache (8 query heads on 1 kv head, d = 128): 4 requests of
    4096 tokens, then 2 requests of 900."""
    rng = np.random.default_rng(8)
    for B, L in ((4, 4096), (2, 900)):
        q = H.f32_tensor(rng.standard_normal((B, 8, 128)))
        k = H.f32_tensor(rng.standard_normal((B, L, 1, 128)))
        v = H.f32_tensor(rng.standard_normal((B, L, 1, 128)))
        beg, end = np.zeros(B, np.int32), np.full(B, L, np.int32)
        ws_n, got, ref = _both(cpa, q, k, v, beg, end, L, 1 / np.sqrt(128))
        assert ws_n > 0
        _same(got, ref)


def test_noalloc_rejects_shapes_beyond_its_scratch(cpa):
    """A shape whose split states exceed the library's 48 MiB scratch is
    rejected on the host with CPA_E_CAPACITY and nothing is written."""
    import torch
    B, L = 200, 2048  # 2 splits x 200 requests x 64 heads x 512 dims x 4 B = 52 MB of states
    need = cpa.attn_decode_workspace_size(B, 64, 512, L)
    if need <= 48 << 20:
        pytest.skip("this device splits so little that the shape fits the scratch")
    q = torch.zeros((B, 64, 576), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((B, L, 1, 576), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(B, dtype=torch.int32, device="cuda")
    e = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o, l = _nan((B, 64, 512)), _nan((B, 64))
    with pytest.raises(cpa.CpaError) as ex:
        cpa.attn_decode_shard_noalloc(q, cache, None, b, e, L, 1 / 24, o, l)
    assert ex.value.status == cpa.CPA_E_CAPACITY
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all()), "a rejected call must not write"
