"""Host-side checks of the C-ABI library (no GPU work): every function the
header declares is exported, the host scheduler reproduces the oracle's
schedule bit for bit, and invalid arguments are rejected before anything is
enqueued."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
import sparse_kv_attention_sfi_amd as S
from sparse_kv_attention_sfi_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "sfi.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfi_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 19
    lib = C.CDLL(B.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert S.sfi_version() == 1


def test_status_strings():
    assert S.sfi_status_str(0) == "SFI_OK"
    assert S.sfi_status_str(-3) == "SFI_ERR_WORKSPACE"
    assert S.sfi_status_str(-99) == "SFI_ERR_UNKNOWN"


@pytest.mark.parametrize("mode,param,batch", [("fixed", 16, 1), ("geometric", 18, 16), ("geometric", 30, 4),
                                              ("geometric", 2.5, 3), ("geometric", 1, 2)])
def test_scheduler_matches_oracle(mode, param, batch):
    seed = 1234
    s = S.Scheduler(batch, seed, mode, param)
    flags = [[] for _ in range(batch)]
    for _ in range(3000):
        slow, fast = s.step()
        assert sorted(slow + fast) == list(range(batch))
        for b in range(batch):
            flags[b].append(b in slow)
    for b in range(batch):
        assert flags[b] == O.schedule(mode, param, seed + b, 3000)


def test_scheduler_t_max_and_force_slow():
    s = S.Scheduler(2, 7, "fixed", 100, t_max=5)
    seq = [s.step()[0] for _ in range(13)]
    assert [i for i, x in enumerate(seq) if 0 in x] == [0, 6, 12]
    s2 = S.Scheduler(1, 0, "fixed", 10)
    out = [s2.step()[0] for _ in range(3)]
    s2.force_slow(0)
    out += [s2.step()[0] for _ in range(12)]
    ref = O.SpanSchedule("fixed", 10, 0)
    exp = [ref.step() for _ in range(3)]
    ref.force_slow()
    exp += [ref.step() for _ in range(12)]
    assert [bool(x) for x in out] == exp


@pytest.mark.parametrize("mode,param", [("fixed", 0), ("fixed", 2.5), ("geometric", 0.5), ("bogus", 3)])
def test_scheduler_rejects_bad_params(mode, param):
    with pytest.raises((S.SFIError, ValueError, TypeError, C.ArgumentError)):
        S.Scheduler(1, 0, mode, param)


def _desc(batch=1, hq=8, hkv=2, d=64, dtype=B.SFI_F32, cap=100, ctx=(100,)):
    ctx_arr = np.asarray(ctx, dtype=np.int32)
    desc = B.sfi_kv_desc(batch, hq, hkv, d, dtype, cap, 0x1000, 0x2000,
                         ctx_arr.ctypes.data_as(C.POINTER(C.c_int32)), 0.0)
    return desc, ctx_arr


def test_validation_rejects_before_launch():
    """Fake device addresses are never touched: every call fails validation."""
    lib = S.lib()
    ids = np.zeros(1, dtype=np.int32)
    pid = ids.ctypes.data_as(C.POINTER(C.c_int32))
    fake = C.c_void_p(0x3000)
    cases = [
        dict(hq=6, hkv=4),          # not a multiple
        dict(hq=24, hkv=2),         # group 12 unsupported
        dict(d=96),                 # head_dim
        dict(dtype=7),              # dtype
        dict(cap=0),                # capacity
        dict(ctx=(101,)),           # ctx beyond capacity
        dict(ctx=(0,)),             # empty context
    ]
    for kw in cases:
        desc, keep = _desc(**kw)
        st = lib.sfi_slow_step(C.byref(desc), pid, 1, fake, fake, None, fake, 1 << 40, None)
        assert st in (B.SFI_ERR_INVALID_ARG, B.SFI_ERR_UNSUPPORTED), kw
        assert lib.sfi_last_error()
    desc, keep = _desc()
    bad_ids = np.array([1], dtype=np.int32)
    st = lib.sfi_slow_step(C.byref(desc), bad_ids.ctypes.data_as(C.POINTER(C.c_int32)), 1, fake, fake, None,
                           fake, 1 << 40, None)
    assert st == B.SFI_ERR_INVALID_ARG
    dup = np.array([0, 0], dtype=np.int32)
    desc2, keep2 = _desc(batch=2, ctx=(100, 100))
    st = lib.sfi_slow_step(C.byref(desc2), dup.ctypes.data_as(C.POINTER(C.c_int32)), 2, fake, fake, None,
                           fake, 1 << 40, None)
    assert st == B.SFI_ERR_INVALID_ARG and b"twice" in lib.sfi_last_error()
    st = lib.sfi_slow_step(C.byref(desc), pid, 1, fake, fake, None, fake, 16, None)
    assert st == B.SFI_ERR_WORKSPACE
    sp = B.sfi_support_params(4, 16, 8, 1.5)
    st = lib.sfi_select(C.byref(desc), C.byref(sp), pid, 1, fake, fake, fake, fake, 1 << 40, None)
    assert st == B.SFI_ERR_INVALID_ARG                         # lambda outside [0, 1]
    sp0 = B.sfi_support_params(0, 0, 0, 0.1)
    st = lib.sfi_fast_step(C.byref(desc), C.byref(sp0), pid, 1, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == B.SFI_ERR_INVALID_ARG                         # empty support
    assert lib.sfi_slow_step(C.byref(desc), pid, 0, fake, fake, None, fake, 0, None) == 0   # nothing to do
    sp = B.sfi_support_params(4, 16, 8, 0.1)
    fused = lib.sfi_slow_step_select
    assert fused(C.byref(desc), C.byref(sp), pid, 1, fake, fake, None, fake, fake, None, None, fake, 1 << 40,
                 None) == B.SFI_ERR_INVALID_ARG                # mass is required
    assert b"mass" in lib.sfi_last_error()
    assert fused(C.byref(desc), C.byref(sp), pid, 1, fake, fake, fake, fake, fake, fake, None, fake, 1 << 40,
                 None) == B.SFI_ERR_INVALID_ARG                # packed_k without packed_v
    need = lib.sfi_workspace_bytes(C.byref(desc), C.byref(sp), B.SFI_OP_SLOW_SELECT)
    assert fused(C.byref(desc), C.byref(sp), pid, 1, fake, fake, fake, fake, fake, None, None, fake, need - 1,
                 None) == B.SFI_ERR_WORKSPACE


def test_fault_injection_fails_select_before_launch(monkeypatch):
    monkeypatch.setenv("SFI_FAULT_INJECT", "select")
    desc, keep = _desc()
    ids = np.zeros(1, dtype=np.int32)
    sp = B.sfi_support_params(4, 16, 8, 0.1)
    fake = C.c_void_p(0x3000)
    st = S.lib().sfi_select(C.byref(desc), C.byref(sp), ids.ctypes.data_as(C.POINTER(C.c_int32)), 1, fake, fake,
                            fake, fake, 1 << 40, None)
    assert st == B.SFI_ERR_INJECTED


def test_workspace_bytes_grow_with_shape():
    d1, k1 = _desc(cap=1000)
    d2, k2 = _desc(cap=100000)
    sp = B.sfi_support_params(16, 256, 2048, 0.1)
    lib = S.lib()
    for op in (B.SFI_OP_SLOW, B.SFI_OP_SELECT, B.SFI_OP_FAST, B.SFI_OP_SLOW_SELECT):
        a = lib.sfi_workspace_bytes(C.byref(d1), C.byref(sp), op)
        b = lib.sfi_workspace_bytes(C.byref(d2), C.byref(sp), op)
        assert 0 < a <= b
    fused = lib.sfi_workspace_bytes(C.byref(d2), C.byref(sp), B.SFI_OP_SLOW_SELECT)
    assert fused == max(lib.sfi_workspace_bytes(C.byref(d2), C.byref(sp), op)
                        for op in (B.SFI_OP_SLOW, B.SFI_OP_SELECT))
    bad, kb = _desc(d=96)
    assert lib.sfi_workspace_bytes(C.byref(bad), C.byref(sp), B.SFI_OP_SLOW) == 0
