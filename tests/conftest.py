import inspect
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU or GPU time)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


# ---------------------------------------------------------------- poisoning
#
# Every output buffer the GPU tests let the binding allocate is filled with
# NaN first (workspaces with 0xff bytes, also NaN as f32), so an output row,
# head or split state a kernel never writes cannot pass as a stale or zero
# value: it fails the NaN checks of tests/helpers.py.

def _nan(shape, dtype, device):
    import torch
    return torch.full(tuple(int(s) for s in shape), float("nan"), dtype=dtype, device=device)


def _ff(nbytes, device):
    import torch
    return torch.full((max(int(nbytes), 1),), 255, dtype=torch.uint8, device=device)


def _poisoning(m):
    import torch
    f32 = torch.float32

    def wrap(fn, fill):
        sig = inspect.signature(fn)

        def inner(*args, **kwargs):
            b = sig.bind(*args, **kwargs)
            b.apply_defaults()
            fill(b.arguments)
            return fn(*b.args, **b.kwargs)

        inner.__wrapped__ = fn
        inner.__name__ = fn.__name__
        return inner

    def prefill(a):
        q, v = a["q"], a["v"]
        n, hq = q.shape[0], q.shape[1]
        dv = v.shape[-1] if v is not None else 512
        if a["out"] is None:
            a["out"] = _nan((n, hq, dv), a["out_dtype"] or q.dtype, q.device)
        if a["lse"] is None:
            a["lse"] = _nan((n, hq), f32, q.device)

    def decode(mq):
        def fill(a):
            q, vc = a["q"], a["vcache"]
            B = q.shape[0]
            Q = q.shape[1] if mq else 1
            hq = q.shape[2] if mq else q.shape[1]
            dv = vc.shape[-1] if vc is not None else 512
            lead = (B, Q) if mq else (B,)
            if a["o_part"] is None:
                a["o_part"] = _nan(lead + (hq, dv), f32, q.device)
            if a["lse_part"] is None:
                a["lse_part"] = _nan(lead + (hq,), f32, q.device)
            if a["workspace"] is None:
                need = m.attn_decode_workspace_size(B * Q, hq, dv, a["max_shard_len"])
                if need > 0:
                    a["workspace"] = _ff(need, q.device)
        return fill

    def paged(a):
        q, vp = a["q"], a["vpool"]
        B, hq = q.shape[0], q.shape[1]
        dv = vp.shape[-1] if vp is not None else 512
        if a["o_part"] is None:
            a["o_part"] = _nan((B, hq, dv), f32, q.device)
        if a["lse_part"] is None:
            a["lse_part"] = _nan((B, hq), f32, q.device)
        if a["workspace"] is None:
            need = m.attn_decode_paged_workspace_size(B, hq, dv, a["max_shard_len"], a["page_size"])
            if need > 0:
                a["workspace"] = _ff(need, q.device)

    def sparse(a):
        q, idx = a["q"], a["idx"]
        N = q.shape[0]
        if a["out"] is None:
            a["out"] = _nan((N, 64, 512), f32, q.device)
        if a["lse"] is None:
            a["lse"] = _nan((N, 64), f32, q.device)
        if a["workspace"] is None:
            need = m.attn_sparse_mla_workspace_size(N, idx.shape[1])
            if need > 0:
                a["workspace"] = _ff(need, q.device)

    def merge(a):
        o = a["o_parts"]
        _, N, H, Dv = o.shape
        if a["out"] is None:
            a["out"] = _nan((N, H, Dv), a["out_dtype"] or f32, o.device)
        if a["lse_out"] is None:
            a["lse_out"] = _nan((N, H), f32, o.device)

    return {
        "attn_prefill_shard": wrap(m.attn_prefill_shard, prefill),
        "attn_decode_shard": wrap(m.attn_decode_shard, decode(False)),
        "attn_decode_shard_mq": wrap(m.attn_decode_shard_mq, decode(True)),
        "attn_decode_shard_paged": wrap(m.attn_decode_shard_paged, paged),
        "attn_sparse_mla": wrap(m.attn_sparse_mla, sparse),
        "attn_merge_states": wrap(m.attn_merge_states, merge),
    }


@pytest.fixture(autouse=True)
def _poison_gpu_outputs(request, monkeypatch):
    """For tests marked gpu: the binding's attention calls get NaN-filled
    outputs and 0xff-filled workspaces unless the test passes its own."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import context_attention_long_amd as m
    for name, fn in _poisoning(m).items():
        monkeypatch.setattr(m, name, fn)
    yield
