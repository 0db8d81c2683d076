"""The C-ABI library loads and exports every function include/cpattn.h
declares; argument validation rejects bad calls on the host (CPU only: no
call here launches device work)."""

import ctypes
import os
import re

import pytest

import context_attention_long_amd as cpa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cpattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("cp_plan_zigzag", "cp_plan_interleave", "attn_prefill_shard", "attn_decode_shard",
              "attn_merge_states", "cpa_last_error"):
        assert n in names
    assert set(names) == set(cpa.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = cpa.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert L.cpa_abi_version() == 102


def test_nm_exports_are_c_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", cpa.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in _declared():
        assert n in syms, n  # plain (unmangled) C names


def test_struct_layouts():
    assert ctypes.sizeof(cpa.CpaTensor) == 8 + 4 + 4 + 32 + 32
    assert ctypes.sizeof(cpa.CpaSegment) == 32
    assert ctypes.sizeof(cpa.CpaPlan) == 9 * 8


def test_plan_errors():
    with pytest.raises(cpa.CpaError) as e:
        cpa.cp_plan_zigzag(0, 0, [4])
    assert e.value.status == cpa.CPA_E_INVAL
    with pytest.raises(cpa.CpaError):
        cpa.cp_plan_zigzag(4, 4, [4])
    with pytest.raises(cpa.CpaError):
        cpa.cp_plan_interleave(4, -1, [4])
    with pytest.raises(cpa.CpaError):
        cpa.cp_plan_interleave(4, 0, [-1])
    with pytest.raises(cpa.CpaError):
        cpa.cp_plan_zigzag(2, 0, [2 ** 31 - 10], [100])  # positions must fit int32
    with pytest.raises(cpa.CpaError):
        cpa.cp_decode_shards(-1, 4)


def test_plan_capacity_idiom():
    L = cpa.lib()
    out = cpa.CpaPlan()
    nl = (ctypes.c_int32 * 2)(19, 7)
    st = L.cp_plan_zigzag(4, 1, 2, nl, None, ctypes.byref(out))
    assert st == cpa.CPA_E_CAPACITY
    assert out.n_local == 5 + 2 and out.n_seg == 4 and out.n_padded == 5 + 2
    assert b"need" in L.cpa_last_error()


def test_device_calls_reject_bad_arguments_before_launch():
    """Validation runs on the host: these calls fail without touching a GPU."""
    L = cpa.lib()
    t = cpa.CpaTensor()
    t.ndim = 3
    t.dtype = cpa.CPA_F32
    # NULL descriptors / data
    assert L.attn_merge_states(1, None, None, None, None, None) == cpa.CPA_E_INVAL
    o = cpa.CpaTensor(); o.ndim = 4; o.dtype = cpa.CPA_F32
    for i, s in enumerate((2, 3, 4, 8)):
        o.shape[i] = s
    o.data = 16  # never dereferenced: validation fails first
    o.stride[3] = 1; o.stride[2] = 8; o.stride[1] = 32; o.stride[0] = 96
    l = cpa.CpaTensor(); l.ndim = 3; l.dtype = cpa.CPA_F32
    for i, s in enumerate((2, 3, 5)):  # wrong H
        l.shape[i] = s
    l.data = 16; l.stride[2] = 1; l.stride[1] = 5; l.stride[0] = 15
    out = cpa.CpaTensor(); out.ndim = 3; out.dtype = cpa.CPA_F32
    for i, s in enumerate((3, 4, 8)):
        out.shape[i] = s
    out.data = 16; out.stride[2] = 1; out.stride[1] = 8; out.stride[0] = 32
    assert L.attn_merge_states(2, ctypes.byref(o), ctypes.byref(l), ctypes.byref(out), None, None) == cpa.CPA_E_INVAL
    assert b"lse_parts" in L.cpa_last_error()
    # misaligned data pointer
    l.shape[2] = 4; l.stride[1] = 4; l.stride[0] = 12
    o.data = 20
    assert L.attn_merge_states(2, ctypes.byref(o), ctypes.byref(l), ctypes.byref(out), None, None) == cpa.CPA_E_INVAL
    assert b"aligned" in L.cpa_last_error()
    # prefill: missing segments / wrong dtype
    q = cpa.CpaTensor(); q.ndim = 3; q.dtype = cpa.CPA_F32
    assert L.attn_prefill_shard(ctypes.byref(q), ctypes.byref(q), None, None, 0, 1.0,
                                ctypes.byref(q), ctypes.byref(q), None) != cpa.CPA_OK
