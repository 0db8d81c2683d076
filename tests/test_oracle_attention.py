"""Pins for the oracle's attention and merge (CPU only, float64)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import plans


def _lib_causal(q, k, v, scale):
    """torch's float64 CPU flash attention (causal): returns (O, LSE).
    q [H, N, D], k [H, N, D], v [H, N, Dv] (heads already broadcast)."""
    # the library op wants one head size: zero columns change neither the
    # scores (padded q, k) nor the first Dv output columns (padded v)
    D, Dv = q.shape[-1], v.shape[-1]
    W = max(D, Dv)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (W - x.shape[-1],))], -1)
    qt = torch.from_numpy(pad(q))[None]
    kt = torch.from_numpy(pad(k))[None]
    vt = torch.from_numpy(pad(v))[None]
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        qt, kt, vt, 0.0, True, scale=scale)[:2]
    return o[0].numpy()[..., :Dv], lse[0].numpy()


def test_merge_worked_example_fig8(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "merge_fig8.json")))
    # exp-scores 4, 2, 1, 1: scores ln4, ln2, 0, 0 with scale 1 and q = [1]
    s = np.log(np.array(g["exp_scores"], dtype=np.float64))
    keys = s[:, None]
    V = np.eye(4)
    q = np.array([1.0])
    o_full, lse_full = att.attend(q, keys, V, 1.0)
    assert np.allclose(o_full, g["true_probs"], rtol=0, atol=1e-15)
    assert abs(lse_full - math.log(8)) < 1e-15
    parts_o, parts_l = [], []
    for gpu, toks in enumerate(g["gpu_tokens"]):
        o, lse = att.attend(q, keys[toks], V[toks], 1.0)
        assert np.allclose(o[toks], g["local_probs"][gpu], atol=1e-15)
        assert abs(lse - math.log(g["local_sums"][gpu])) < 1e-15
        parts_o.append(o)
        parts_l.append(lse)
    o_m, lse_m = att.merge_states(np.stack(parts_o), np.array(parts_l))
    assert abs(lse_m - math.log(8)) < 1e-15
    assert np.allclose(np.exp(np.array(parts_l) - lse_m), g["rescale"], atol=1e-15)
    assert np.allclose(o_m, g["true_probs"], atol=1e-15)
    # the same through decode_shard on a cache stored in shard order [t0, t2 | t1, t3]
    order = [0, 2, 1, 3]
    kc = keys[order][None, :, None, :]
    vc = V[order][None, :, None, :]
    O0, L0 = att.decode_shard(q[None, None], kc, [0], [2], 1.0, vcache=vc)
    O1, L1 = att.decode_shard(q[None, None], kc, [2], [4], 1.0, vcache=vc)
    o_m2, lse_m2 = att.merge_states(np.stack([O0, O1]), np.stack([L0, L1]))
    assert np.allclose(o_m2[0, 0], g["true_probs"], atol=1e-15)


def test_single_key_and_equal_scores_closed_forms():
    rng = np.random.default_rng(0)
    q = rng.standard_normal(16)
    k = rng.standard_normal((1, 16))
    v = rng.standard_normal((1, 8))
    o, lse = att.attend(q, k, v, 0.3)
    assert np.allclose(o, v[0], atol=0) and abs(lse - 0.3 * float(k[0] @ q)) < 1e-14
    n = 37
    kk = np.repeat(k, n, axis=0)
    vv = rng.standard_normal((n, 8))
    o, lse = att.attend(q, kk, vv, 0.3)
    assert np.allclose(o, vv.mean(0), atol=1e-14)
    assert abs(lse - (0.3 * float(k[0] @ q) + math.log(n))) < 1e-13
    o, lse = att.attend(q, np.zeros((0, 16)), np.zeros((0, 8)), 0.3)
    assert np.all(o == 0) and lse == -np.inf


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (6, 2), (8, 8)])
@pytest.mark.parametrize("prefix", [0, 5])
def test_c1_equals_library_causal_attention(Hq, Hkv, prefix):
    """C = 1 is ordinary causal attention over the whole request (prefix
    included): compare with torch's float64 causal flash attention."""
    rng = np.random.default_rng(Hq * 10 + prefix)
    L, D, Dv = 23, 16, 12
    T = prefix + L
    q_all = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, Dv))
    scale = 1.0 / math.sqrt(D)
    p = plans.plan_zigzag(1, 0, [L], [prefix])
    q_local = q_all[prefix + p.tok_index]
    O, LSE = att.prefill_shard(q_local, k, p.segments, scale, v=v)
    G = Hq // Hkv
    kb = np.repeat(k, G, axis=1).transpose(1, 0, 2).copy()
    vb = np.repeat(v, G, axis=1).transpose(1, 0, 2).copy()
    o_ref, lse_ref = _lib_causal(q_all.transpose(1, 0, 2).copy(), kb, vb, scale)
    assert np.allclose(O, o_ref.transpose(1, 0, 2)[prefix:], atol=1e-13)
    assert np.allclose(LSE, lse_ref.T[prefix:], atol=1e-13)


def test_mla_value_is_latent_prefix():
    rng = np.random.default_rng(3)
    L, H, D, Dv = 9, 4, 10, 6
    q = rng.standard_normal((L, H, D))
    lat = rng.standard_normal((L, 1, D))
    p = plans.plan_zigzag(1, 0, [L])
    O1, L1 = att.prefill_shard(q, lat, p.segments, 0.5, dv=Dv)
    O2, L2 = att.prefill_shard(q, lat, p.segments, 0.5, v=lat[..., :Dv].copy())
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("strategy", ["zigzag", "interleave"])
def test_union_of_ranks_equals_unsharded(strategy):
    """Every query owned by exactly one rank and each rank attending to the
    true causal history: the union of all ranks' rows equals unsharded
    attention (brute force on tiny inputs, every C)."""
    rng = np.random.default_rng(5)
    new_len, prefix = [11, 0, 7, 3], [4, 2, 0, 1]
    Hq, Hkv, D = 4, 2, 8
    scale = 0.4
    cu_kv = np.concatenate([[0], np.cumsum(np.array(new_len) + np.array(prefix))])
    T_kv = int(cu_kv[-1])
    k = rng.standard_normal((T_kv, Hkv, D))
    v = rng.standard_normal((T_kv, Hkv, D))
    q_kv = rng.standard_normal((T_kv, Hq, D))  # a query for every stored token
    cu_new = np.concatenate([[0], np.cumsum(new_len)])
    # global row of flattened new token g: kv row of (request, prefix + offset)
    def kvrow(g):
        j = np.searchsorted(cu_new, g, side="right") - 1
        return cu_kv[j] + np.asarray(prefix)[j] + (g - cu_new[j])
    # reference: per request, library causal attention over its whole sequence
    ref_o = np.zeros((T_kv, Hq, D))
    ref_l = np.zeros((T_kv, Hq))
    G = Hq // Hkv
    for j in range(len(new_len)):
        a, b = cu_kv[j], cu_kv[j + 1]
        if b == a:
            continue
        o, l = _lib_causal(q_kv[a:b].transpose(1, 0, 2).copy(),
                           np.repeat(k[a:b], G, 1).transpose(1, 0, 2).copy(),
                           np.repeat(v[a:b], G, 1).transpose(1, 0, 2).copy(), scale)
        ref_o[a:b] = o.transpose(1, 0, 2)
        ref_l[a:b] = l.T
    fn = plans.plan_zigzag if strategy == "zigzag" else plans.plan_interleave
    for C in range(1, 7):
        got = np.zeros(sum(new_len), dtype=int)
        for r in range(C):
            p = fn(C, r, new_len, prefix)
            if p.n_local == 0:
                continue
            rows = kvrow(p.tok_index)
            O, LSE = att.prefill_shard(q_kv[rows], k, p.segments, scale, v=v)
            assert np.allclose(O, ref_o[rows], atol=1e-13)
            assert np.allclose(LSE, ref_l[rows], atol=1e-13)
            got[p.tok_index] += 1
        assert np.all(got == 1)


def test_split_kv_merge_equals_unsharded():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, L = 3, 6, 2, 12, 50
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, L, Hkv, D))
    vc = rng.standard_normal((B, L, Hkv, D))
    full_o, full_l = att.decode_shard(q, kc, [0] * B, [L] * B, 0.7, vcache=vc)
    # reference: library causal attention of the last row = attention over all L keys
    G = Hq // Hkv
    for b in range(B):
        qq = np.concatenate([np.zeros((L - 1, Hq, D)), q[b][None]], 0).transpose(1, 0, 2).copy()
        o, l = _lib_causal(qq, np.repeat(kc[b], G, 1).transpose(1, 0, 2).copy(),
                           np.repeat(vc[b], G, 1).transpose(1, 0, 2).copy(), 0.7)
        assert np.allclose(full_o[b], o[:, -1], atol=1e-13)
        assert np.allclose(full_l[b], l[:, -1], atol=1e-13)
    for C in (1, 2, 3, 4, 7, 50, 64):
        sh = plans.contiguous_shards(L, C)
        parts = [att.decode_shard(q, kc, [s] * B, [e] * B, 0.7, vcache=vc) for s, e in sh]
        o, l = att.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.allclose(o, full_o, atol=1e-13) and np.allclose(l, full_l, atol=1e-13)
        assert not np.any(np.isnan(o))


def test_merge_properties():
    rng = np.random.default_rng(2)
    S, N, Dv = 5, 7, 9
    o = rng.standard_normal((S, N, Dv))
    l = rng.standard_normal((S, N)) * 3
    om, lm = att.merge_states(o, l)
    perm = rng.permutation(S)
    om2, lm2 = att.merge_states(o[perm], l[perm])
    assert np.allclose(om, om2, atol=1e-14) and np.allclose(lm, lm2, atol=1e-14)
    # associativity: merge of merges
    a = att.merge_states(o[:2], l[:2])
    b = att.merge_states(o[2:], l[2:])
    om3, lm3 = att.merge_states(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
    assert np.allclose(om, om3, atol=1e-14) and np.allclose(lm, lm3, atol=1e-14)
    # a -inf state carries no mass
    o_e = np.concatenate([o, rng.standard_normal((1, N, Dv))])
    l_e = np.concatenate([l, np.full((1, N), -np.inf)])
    om4, lm4 = att.merge_states(o_e, l_e)
    assert np.allclose(om, om4, atol=1e-15) and np.allclose(lm, lm4, atol=1e-15)
    # two equal states: same O, lse + ln 2
    om5, lm5 = att.merge_states(np.stack([o[0], o[0]]), np.stack([l[0], l[0]]))
    assert np.allclose(om5, o[0], atol=1e-15) and np.allclose(lm5, l[0] + math.log(2), atol=1e-14)
    # S = 1 is the identity
    om6, lm6 = att.merge_states(o[:1], l[:1])
    assert np.allclose(om6, o[0]) and np.allclose(lm6, l[0])
    # all empty: O = 0, lse = -inf, no NaN
    om7, lm7 = att.merge_states(np.zeros((3, N, Dv)), np.full((3, N), -np.inf))
    assert np.all(om7 == 0) and np.all(lm7 == -np.inf)
    # huge LSE values do not overflow
    om8, lm8 = att.merge_states(o[:2], l[:2] + 1e4)
    assert np.allclose(lm8, att.merge_states(o[:2], l[:2])[1] + 1e4)


def test_merge_states_agrees_with_statistics_form():
    """The LSE merge of Long Context 3.3 and the (m, l, u) combine of the
    DeepSeek-V4 notes, section 5, give the same output."""
    rng = np.random.default_rng(4)
    n, D, Dv = 40, 8, 5
    q = rng.standard_normal(D)
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, Dv))
    shards = [range(0, 13), range(13, 14), range(14, 40)]
    ms, ls, us, os_, lses = [], [], [], [], []
    for sh in shards:
        idx = list(sh)
        m, ell, u = att.shard_stats(q, k[idx], v[idx], 0.9)
        ms.append(m); ls.append(ell); us.append(u)
        o, lse = att.attend(q, k[idx], v[idx], 0.9)
        os_.append(o); lses.append(lse)
        assert abs(lse - (m + math.log(ell))) < 1e-13
    o1, Z, m = att.merge_stats(ms, ls, us)
    o2, lse2 = att.merge_states(np.stack(os_), np.array(lses))
    assert np.allclose(o1, o2, atol=1e-14)
    assert abs(lse2 - (m + math.log(Z))) < 1e-13
    o3, lse3 = att.attend(q, k, v, 0.9)
    assert np.allclose(o3, o2, atol=1e-14) and abs(lse3 - lse2) < 1e-13


def test_fp8_decode_uses_scale_per_token():
    from oracle import formats
    import synth
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 20, 1, 16)).astype(np.float32) * 0.5
    codes, scale = synth.f32_to_e4m3(x)  # scale [1, 20, 1]: one per token
    q = rng.standard_normal((1, 3, 16))
    O, L = att.decode_shard(q, codes, [0], [20], 0.25, dv=8, decode=formats.e4m3_to_f64,
                            kv_scale=scale[..., 0])
    deq = formats.e4m3_to_f64(codes) * scale[..., None]
    O2, L2 = att.decode_shard(q, deq, [0], [20], 0.25, dv=8)
    assert np.allclose(O, O2, atol=1e-15) and np.allclose(L, L2, atol=1e-15)


def test_fp8_gqa_decode_scales_keys_and_values():
    """GQA FP8 cache: the token's scale multiplies its key and its value
    (one scale per cache row). Pinned to plain decode over the explicitly
    dequantised K and V, and to the fact that a common scale c on every
    token equals decode with the query times c and the output times c."""
    from oracle import formats
    import synth
    rng = np.random.default_rng(81)
    B, L, Hkv, Hq, D = 2, 23, 2, 6, 16
    kx = rng.standard_normal((B, L, Hkv, D)).astype(np.float32)
    vx = rng.standard_normal((B, L, Hkv, D)).astype(np.float32)
    kc, _ = synth.f32_to_e4m3(kx)
    vc, _ = synth.f32_to_e4m3(vx)
    scale = rng.uniform(0.25, 3.0, (B, L)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D))
    beg, end = [0, 5], [23, 17]
    O, Lse = att.decode_shard(q, kc, beg, end, 0.3, vcache=vc, decode=formats.e4m3_to_f64, kv_scale=scale)
    s64 = scale.astype(np.float64)[:, :, None, None]
    kd, vd = formats.e4m3_to_f64(kc) * s64, formats.e4m3_to_f64(vc) * s64
    O2, L2 = att.decode_shard(q, kd, beg, end, 0.3, vcache=vd)
    assert np.allclose(O, O2, atol=1e-14) and np.allclose(Lse, L2, atol=1e-13)
    c = 4.0
    Oc, Lc = att.decode_shard(q, kc, beg, end, 0.3, vcache=vc, decode=formats.e4m3_to_f64,
                              kv_scale=np.full((B, L), c, np.float32))
    O3, L3 = att.decode_shard(q * c, formats.e4m3_to_f64(kc), beg, end, 0.3, vcache=formats.e4m3_to_f64(vc))
    assert np.allclose(Oc, c * O3, atol=1e-12) and np.allclose(Lc, L3, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (8, 2), (6, 3)])
def test_decode_equals_library_last_row(Hq, Hkv):
    """A decode query over the whole cache [0, L) is the causal attention of
    the sequence's last token (Long Context 1.1 and 3.2): compare
    decode_shard with torch's float64 causal flash attention, GQA heads
    broadcast in contiguous groups, and with two shards merged."""
    rng = np.random.default_rng(40 + Hq + Hkv)
    L, D = 19, 16
    G = Hq // Hkv
    q_all = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    scale = 0.3
    kb = np.repeat(k, G, axis=1).transpose(1, 0, 2).copy()
    vb = np.repeat(v, G, axis=1).transpose(1, 0, 2).copy()
    o_ref, lse_ref = _lib_causal(q_all.transpose(1, 0, 2).copy(), kb, vb, scale)
    q = q_all[L - 1][None]                      # [1, Hq, D]
    O, LSE = att.decode_shard(q, k[None], [0], [L], scale, vcache=v[None])
    assert np.allclose(O[0], o_ref[:, L - 1], atol=1e-13)
    assert np.allclose(LSE[0], lse_ref[:, L - 1], atol=1e-13)
    parts = [att.decode_shard(q, k[None], [s0], [s1], scale, vcache=v[None]) for s0, s1 in ((0, 7), (7, L))]
    Om, Lm = att.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.allclose(Om[0], o_ref[:, L - 1], atol=1e-13)
    assert np.allclose(Lm[0], lse_ref[:, L - 1], atol=1e-13)
