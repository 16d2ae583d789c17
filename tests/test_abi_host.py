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
    text = open(os.path.join(ROOT, "include", "sfi.h")).read()
    major = int(re.search(r"#define SFI_VERSION_MAJOR (\d+)", text).group(1))
    minor = int(re.search(r"#define SFI_VERSION_MINOR (\d+)", text).group(1))
    assert S.sfi_version() == major * 100 + minor      # the library was built from this header


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
        dict(hq=512, hkv=512),      # more KV heads than supported
        dict(batch=70000),          # batch beyond the supported bound
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
    for ns, w in ((1 << 31) - 1, 16), (4, (1 << 31) - 1):
        spw = B.sfi_support_params(ns, w, 8, 0.1)          # window arithmetic would overflow int32
        st = lib.sfi_select(C.byref(desc), C.byref(spw), pid, 1, fake, fake, fake, fake, 1 << 40, None)
        assert st == B.SFI_ERR_INVALID_ARG
    sp0 = B.sfi_support_params(0, 0, 0, 0.1)
    st = lib.sfi_fast_step(C.byref(desc), C.byref(sp0), pid, 1, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == B.SFI_ERR_INVALID_ARG                         # empty support
    assert lib.sfi_slow_step(C.byref(desc), pid, 0, fake, fake, None, fake, 0, None) == 0   # nothing to do
    full, kf = _desc(cap=100, ctx=(100,))                    # no room for another row
    assert lib.sfi_kv_append(C.byref(full), pid, 1, fake, fake, None) == B.SFI_ERR_INVALID_ARG
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


def test_misaligned_buffers_rejected_before_launch():
    """Every entry point rejects a buffer off its 16-byte (int32 arrays:
    4-byte) boundary before it enqueues anything; the error names it."""
    lib = S.lib()
    ids = np.zeros(1, dtype=np.int32)
    pid = ids.ctypes.data_as(C.POINTER(C.c_int32))
    a = C.c_void_p(0x3000)                  # aligned fake device address
    m8, m2 = C.c_void_p(0x3008), C.c_void_p(0x3002)
    desc, keep = _desc()
    sp = B.sfi_support_params(4, 16, 8, 0.1)
    big = 1 << 40
    calls = {
        "q": lambda: lib.sfi_slow_step(C.byref(desc), pid, 1, m8, a, None, a, big, None),
        "mass": lambda: lib.sfi_select(C.byref(desc), C.byref(sp), pid, 1, m8, a, a, a, big, None),
        "sel_idx": lambda: lib.sfi_select(C.byref(desc), C.byref(sp), pid, 1, a, m2, a, a, big, None),
        "packed_k": lambda: lib.sfi_slow_step_select(C.byref(desc), C.byref(sp), pid, 1, a, a, a, a, a, m8, a, a,
                                                     big, None),
        "out": lambda: lib.sfi_fast_step(C.byref(desc), C.byref(sp), pid, 1, a, a, a, m8, a, big, None),
        "packed_v": lambda: lib.sfi_fast_step_packed(C.byref(desc), C.byref(sp), pid, 1, a, a, m8, a, a, a, big,
                                                     None),
        "packed_k": lambda: lib.sfi_fast_step_packed_noalloc(C.byref(desc), C.byref(sp), pid, 1, a, m8, a, a, a,
                                                             None),
        "sel_cnt": lambda: lib.sfi_pack_support(C.byref(desc), C.byref(sp), pid, 1, a, m2, a, a, None),
        "k_new": lambda: lib.sfi_kv_append(C.byref(_desc(ctx=(99,))[0]), pid, 1, m8, a, None),
        "support_out": lambda: lib.sfi_debug_support(C.byref(desc), C.byref(sp), pid, 1, a, a, m2, a, 64, None),
        "workspace": lambda: lib.sfi_slow_step(C.byref(desc), pid, 1, a, a, None, m8, big, None),
    }
    for name, call in calls.items():
        assert call() == B.SFI_ERR_INVALID_ARG, name
        err = lib.sfi_last_error().decode()
        assert name in err and "aligned" in err, (name, err)
    assert lib.sfi_workspace_init(m8, 4096, None) == B.SFI_ERR_INVALID_ARG
    kd, keep2 = _desc()
    kd.k = 0x1004
    assert lib.sfi_slow_step(C.byref(kd), pid, 1, a, a, None, a, big, None) == B.SFI_ERR_INVALID_ARG
    assert b"desc->k" in lib.sfi_last_error()
    kd, keep3 = _desc()
    kd.ctx_len = 0x1002                      # device context lengths off their 4-byte boundary
    assert lib.sfi_fast_step(C.byref(kd), C.byref(sp), pid, 1, a, a, a, a, a, big, None) == B.SFI_ERR_INVALID_ARG
    assert b"desc->ctx_len" in lib.sfi_last_error()


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


def test_slow_plan_covers_every_row():
    """The slow step's launch plan: every sequence gets at least one split, no
    split is smaller than one block of rows per wave, and no KV head needs
    more partial slots than the merge accepts.  At the 128K layer the 8 KV
    heads' 1M rows spread over about 1024 workgroups: 128 splits per head."""
    lib = S.lib()
    cases = (((131072,), 131072, 8, 128, B.SFI_BF16), ((1, 300, 65536, 8192), 65536, 8, 128, B.SFI_BF16),
             ((5000, 17), 5000, 2, 64, B.SFI_F32))
    for ctx, cap, hkv, d, dt in cases:
        desc, keep = _desc(batch=len(ctx), hq=4 * hkv, hkv=hkv, d=d, dtype=dt, cap=cap, ctx=ctx)
        ids = np.arange(len(ctx), dtype=np.int32)
        out = np.full(len(ctx), -1, dtype=np.int32)
        unit = 4 * 16384 // (d * (2 if dt == B.SFI_BF16 else 4))   # 4 waves x one 16 KiB block each
        for with_mass in (0, 1):
            st = lib.sfi_slow_plan(C.byref(desc), ids.ctypes.data_as(C.POINTER(C.c_int32)), len(ctx), with_mass,
                                   out.ctypes.data_as(C.POINTER(C.c_int32)))
            assert st == 0
            for t, n in zip(ctx, out):
                assert 1 <= n <= 512 and n <= -(-t // unit), (t, n)
                if with_mass and t <= 512 * 1024:
                    assert -(-t // n) <= 1024, (t, n)   # splits short enough for the logit buffer
    assert S.sfi_slow_plan is not None
    desc, keep = _desc(batch=1, hq=32, hkv=8, d=128, dtype=B.SFI_BF16, cap=131072, ctx=(131072,))
    one = np.zeros(1, dtype=np.int32)
    out = np.zeros(1, dtype=np.int32)
    assert lib.sfi_slow_plan(C.byref(desc), one.ctypes.data_as(C.POINTER(C.c_int32)), 1, 1,
                             out.ctypes.data_as(C.POINTER(C.c_int32))) == 0 and out[0] == 128
    # four rows of 128K: the dense step keeps 4096-row splits, the step with mass 1024-row ones
    desc4, keep4 = _desc(batch=4, hq=32, hkv=8, d=128, dtype=B.SFI_BF16, cap=131072, ctx=(131072,) * 4)
    four = np.arange(4, dtype=np.int32)
    out4 = np.zeros(4, dtype=np.int32)
    assert lib.sfi_slow_plan(C.byref(desc4), four.ctypes.data_as(C.POINTER(C.c_int32)), 4, 0,
                             out4.ctypes.data_as(C.POINTER(C.c_int32))) == 0 and list(out4) == [32] * 4
    assert lib.sfi_slow_plan(C.byref(desc4), four.ctypes.data_as(C.POINTER(C.c_int32)), 4, 1,
                             out4.ctypes.data_as(C.POINTER(C.c_int32))) == 0 and list(out4) == [128] * 4
    desc, keep = _desc(ctx=(100,))
    bad = np.array([3], dtype=np.int32)
    assert lib.sfi_slow_plan(C.byref(desc), bad.ctypes.data_as(C.POINTER(C.c_int32)), 1, 1,
                             out.ctypes.data_as(C.POINTER(C.c_int32))) == B.SFI_ERR_INVALID_ARG


def test_fast_plan_chunks_cover_the_support():
    """The fast step's launch plan: chunks of the per-workgroup row count cover
    the largest support (sinks + window + min(top_k, candidates))."""
    lib = S.lib()
    sp = B.sfi_support_params(16, 256, 2048, 0.1)
    ctx = (131072, 3000, 300, 5)
    desc, keep = _desc(batch=4, hq=32, hkv=8, d=128, dtype=B.SFI_BF16, cap=131072, ctx=ctx)
    ids = np.arange(4, dtype=np.int32)
    out = np.zeros(4, dtype=np.int32)
    assert lib.sfi_fast_plan(C.byref(desc), C.byref(sp), ids.ctypes.data_as(C.POINTER(C.c_int32)), 4,
                             out.ctypes.data_as(C.POINTER(C.c_int32))) == 0
    sizes = [min(16, t) + max(0, t - max(16, t - 256)) + min(2048, max(0, t - 272)) for t in ctx]
    assert sizes == [2320, 2320, 300, 5]
    # 4 waves x 2 tiles x 16 rows = 128 support rows per workgroup by default
    assert out.tolist() == [max(1, -(-s // 128)) for s in sizes]


def test_noalloc_fast_step_rejects_what_its_fixed_scratch_cannot_hold():
    """The fast step without a workspace fails with SFI_ERR_UNSUPPORTED, before
    anything is enqueued, when the rows, the counters or the chunk states
    exceed its fixed per-device scratch (fake device addresses: never
    touched)."""
    lib = S.lib()
    a = C.c_void_p(0x3000)
    call = lib.sfi_fast_step_packed_noalloc
    # 65 rows: more than one launch group
    desc, keep = _desc(batch=65, ctx=(100,) * 65)
    ids = np.arange(65, dtype=np.int32)
    sp = B.sfi_support_params(4, 16, 8, 0.1)
    assert call(C.byref(desc), C.byref(sp), ids.ctypes.data_as(C.POINTER(C.c_int32)), 65, a, a, a, a, a,
                None) == B.SFI_ERR_UNSUPPORTED
    assert b"64" in lib.sfi_last_error()
    # 64 rows x 32 KV heads: more chunk counters than the scratch has
    desc, keep = _desc(batch=64, hq=32, hkv=32, ctx=(100,) * 64)
    ids = np.arange(64, dtype=np.int32)
    assert call(C.byref(desc), C.byref(sp), ids.ctypes.data_as(C.POINTER(C.c_int32)), 64, a, a, a, a, a,
                None) == B.SFI_ERR_UNSUPPORTED
    assert b"counters" in lib.sfi_last_error()
    # 16 rows of 256 query heads with a 65536-row support: 136 MB of chunk states
    desc, keep = _desc(batch=16, hq=256, hkv=32, d=128, dtype=B.SFI_BF16, cap=70000, ctx=(70000,) * 16)
    ids = np.arange(16, dtype=np.int32)
    big = B.sfi_support_params(16, 256, 65000, 0.1)
    assert call(C.byref(desc), C.byref(big), ids.ctypes.data_as(C.POINTER(C.c_int32)), 16, a, a, a, a, a,
                None) == B.SFI_ERR_UNSUPPORTED
    assert b"fixed scratch holds" in lib.sfi_last_error()
    # a duplicate id is caught without the heap-allocating check
    desc, keep = _desc(batch=2, ctx=(100, 100))
    dup = np.array([1, 1], dtype=np.int32)
    assert call(C.byref(desc), C.byref(sp), dup.ctypes.data_as(C.POINTER(C.c_int32)), 2, a, a, a, a, a,
                None) == B.SFI_ERR_INVALID_ARG
    assert b"twice" in lib.sfi_last_error()


def test_selector_option_ranges_and_the_key_norm_restriction():
    """The optional Selector steps' parameters are range-checked before any
    launch; the key-norm correction needs the fused refresh (sfi_select
    rejects it); too many KV heads for the score pass's LDS are unsupported;
    and turning an option on enlarges the Selector's workspace."""
    lib = S.lib()
    a = C.c_void_p(0x3000)
    ids = np.zeros(1, dtype=np.int32)
    pid = ids.ctypes.data_as(C.POINTER(C.c_int32))
    desc, keep = _desc(batch=1, hq=32, hkv=8, d=128, dtype=B.SFI_BF16, cap=4000, ctx=(4000,))
    base = B.sfi_support_params(16, 256, 512, 0.1)
    for kw in (dict(knorm_beta=-1.0), dict(knorm_c=float("nan")), dict(nms_radius=33), dict(nms_radius=-1),
               dict(nms_decay=1.5), dict(excl=-0.5), dict(excl=float("inf"))):
        sp = S.support_params(16, 256, 512, 0.1, **kw)
        assert lib.sfi_select(C.byref(desc), C.byref(sp), pid, 1, a, a, a, a, 1 << 40, None) == B.SFI_ERR_INVALID_ARG, kw
    sp = S.support_params(16, 256, 512, 0.1, knorm_beta=1.0)
    assert lib.sfi_select(C.byref(desc), C.byref(sp), pid, 1, a, a, a, a, 1 << 40, None) == B.SFI_ERR_UNSUPPORTED
    assert b"key norms" in lib.sfi_last_error()
    wide, kw2 = _desc(batch=1, hq=256, hkv=256, d=64, dtype=B.SFI_BF16, cap=4000, ctx=(4000,))
    sp = S.support_params(16, 256, 512, 0.1, nms_radius=8, nms_decay=0.5)
    assert lib.sfi_select(C.byref(wide), C.byref(sp), pid, 1, a, a, a, a, 1 << 40, None) == B.SFI_ERR_UNSUPPORTED
    for op in (B.SFI_OP_SELECT, B.SFI_OP_SLOW_SELECT):
        plain = lib.sfi_workspace_bytes(C.byref(desc), C.byref(base), op)
        opt = lib.sfi_workspace_bytes(C.byref(desc), C.byref(S.support_params(16, 256, 512, 0.1, excl=1.0)), op)
        assert 0 < plain < opt


def test_scheduler_errors_leave_a_message():
    """Every failing scheduler call sets sfi_last_error() with its own message
    (not a stale one from an earlier call); the out-of-memory status has its
    own name."""
    lib = S.lib()
    h = C.c_void_p()
    cases = [((1, 0, B.SFI_SPAN_GEOMETRIC, 0.5, 0), b"geometric mean"),
             ((1, 0, B.SFI_SPAN_FIXED, 2.5, 0), b"fixed span"),
             ((0, 0, B.SFI_SPAN_FIXED, 4.0, 0), b"batch"),
             ((1, 0, 99, 4.0, 0), b"span mode"),
             ((1, 0, B.SFI_SPAN_FIXED, 4.0, -1), b"t_max")]
    for args, msg in cases:
        lib.sfi_status_str(0)
        st = lib.sfi_sched_create(*args, C.byref(h))
        assert st == B.SFI_ERR_INVALID_ARG and msg in lib.sfi_last_error(), (args, lib.sfi_last_error())
    s = S.Scheduler(2, 1, "fixed", 4)
    with pytest.raises(S.SFIError, match="out of range"):
        s.force_slow(5)
    assert lib.sfi_sched_step(None, None, None, None, None) == B.SFI_ERR_INVALID_ARG
    assert b"sfi_sched_step" in lib.sfi_last_error()
    assert S.sfi_status_str(B.SFI_ERR_NO_MEMORY) == "SFI_ERR_NO_MEMORY"
