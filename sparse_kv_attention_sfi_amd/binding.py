"""ctypes binding of ``libsfi.so`` (declared in ``include/sfi.h``).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the current GPU (PyTorch provides the
device memory and the stream); host arrays are numpy int32.  Loading fails
loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfi.so")

SFI_OK, SFI_ERR_INVALID_ARG, SFI_ERR_UNSUPPORTED, SFI_ERR_WORKSPACE, SFI_ERR_HIP, SFI_ERR_INJECTED = 0, -1, -2, -3, -4, -5
SFI_ERR_NO_MEMORY = -6
SFI_F32, SFI_BF16 = 0, 1
SFI_OP_SLOW, SFI_OP_SELECT, SFI_OP_FAST, SFI_OP_SLOW_SELECT = 0, 1, 2, 3
SFI_SPAN_FIXED, SFI_SPAN_GEOMETRIC = 0, 1
(SFI_K_SLOW_PARTIAL, SFI_K_SLOW_COMBINE, SFI_K_SELECT, SFI_K_FAST, SFI_K_APPEND, SFI_K_PACK, SFI_K_FAST_MERGE,
 SFI_K_FAST_PACK) = range(8)
KERNEL_NAMES = {SFI_K_SLOW_PARTIAL: "slow_partial", SFI_K_SLOW_COMBINE: "slow_combine",
                SFI_K_SELECT: "select", SFI_K_FAST: "fast_partial", SFI_K_APPEND: "append",
                SFI_K_PACK: "pack", SFI_K_FAST_MERGE: "fast_merge", SFI_K_FAST_PACK: "fast_pack"}


class SFIError(RuntimeError):
    def __init__(self, status, where, message):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


class sfi_kv_desc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("kv_dtype", C.c_int32), ("kv_capacity", C.c_int64),
                ("k", C.c_void_p), ("v", C.c_void_p), ("ctx_len_host", C.POINTER(C.c_int32)),
                ("scale", C.c_float), ("ctx_len", C.c_void_p)]


class sfi_support_params(C.Structure):
    _fields_ = [("n_sink", C.c_int32), ("n_recent", C.c_int32), ("top_k", C.c_int32),
                ("lambda_", C.c_float), ("knorm_beta", C.c_float), ("knorm_c", C.c_float),
                ("nms_radius", C.c_int32), ("nms_decay", C.c_float), ("excl", C.c_float)]


_lib = None


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_kv_attention_sfi_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, SZ, VP = C.POINTER, C.c_int32, C.c_int64, C.c_size_t, C.c_void_p
        D, S = P(sfi_kv_desc), P(sfi_support_params)
        sig = {
            "sfi_version": (I32, []),
            "sfi_status_str": (C.c_char_p, [I32]),
            "sfi_last_error": (C.c_char_p, []),
            "sfi_workspace_bytes": (SZ, [D, S, I32]),
            "sfi_workspace_init": (I32, [VP, SZ, VP]),
            "sfi_slow_step": (I32, [D, P(I32), I32, VP, VP, VP, VP, SZ, VP]),
            "sfi_select": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, SZ, VP]),
            "sfi_fast_step": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, VP, SZ, VP]),
            "sfi_fast_step_pack": (I32, [D, S, P(I32), I32, P(I32), VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
            "sfi_kv_append": (I32, [D, P(I32), I32, VP, VP, VP]),
            "sfi_pack_support": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, VP]),
            "sfi_fast_step_packed": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, VP, VP, SZ, VP]),
            "sfi_fast_step_packed_noalloc": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, VP, VP]),
            "sfi_slow_plan": (I32, [D, P(I32), I32, I32, P(I32)]),
            "sfi_fast_plan": (I32, [D, S, P(I32), I32, P(I32)]),
            "sfi_slow_step_select": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
            "sfi_slow_step_select_async": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP, VP]),
            "sfi_debug_support": (I32, [D, S, P(I32), I32, VP, VP, VP, VP, I32, VP]),
            "sfi_sched_create": (I32, [I32, C.c_uint64, I32, C.c_double, I32, P(VP)]),
            "sfi_sched_step": (I32, [VP, P(I32), P(I32), P(I32), P(I32)]),
            "sfi_sched_force_slow": (I32, [VP, I32]),
            "sfi_sched_destroy": (None, [VP]),
            "sfi_profile_enable": (I32, [I32]),
            "sfi_profile_reset": (I32, []),
            "sfi_profile_read": (I32, [I32, P(C.c_double), P(I64)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, where):
    if status != SFI_OK:
        msg = lib().sfi_last_error().decode(errors="replace")
        raise SFIError(status, where, msg)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    """A raw hipStream_t handle from an int, a torch stream, or None (torch's current stream)."""
    if stream is not None:
        return C.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ids(seq_ids):
    a = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32)), int(a.shape[0])


class KVDesc:
    """One layer's KV cache [B, Hkv, T_cap, D] plus context lengths.

    ctx_len: host context lengths, or with ``ctx_dev`` (a device int32
    tensor [B] holding the lengths the kernels read when they run, which
    sfi_kv_append advances) their upper bounds.  Keeps the ctypes descriptor,
    the host array and the device tensor alive."""

    def __init__(self, k, v, ctx_len, n_q_heads, scale=0.0, ctx_dev=None):
        import torch
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("k and v must both be [B, Hkv, T_cap, D]")
        if k.dtype != v.dtype or k.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k and v must be float32 or bfloat16 of the same dtype")
        if not (k.is_cuda and v.is_cuda and k.is_contiguous() and v.is_contiguous()):
            raise ValueError("k and v must be contiguous device tensors")
        self.k, self.v = k, v
        B, Hkv, cap, D = k.shape
        self.ctx = np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int32).reshape(B))
        self.dtype = k.dtype
        if ctx_dev is not None:
            _need(ctx_dev, torch.int32, (B,), "ctx_dev")
        self.ctx_dev = ctx_dev
        self.desc = sfi_kv_desc(B, int(n_q_heads), Hkv, D,
                                SFI_BF16 if k.dtype == torch.bfloat16 else SFI_F32, cap,
                                k.data_ptr(), v.data_ptr(),
                                self.ctx.ctypes.data_as(C.POINTER(C.c_int32)), float(scale),
                                None if ctx_dev is None else ctx_dev.data_ptr())

    @property
    def batch(self):
        return self.desc.batch

    @property
    def n_q_heads(self):
        return self.desc.n_q_heads

    @property
    def n_kv_heads(self):
        return self.desc.n_kv_heads

    @property
    def head_dim(self):
        return self.desc.head_dim

    @property
    def capacity(self):
        return self.desc.kv_capacity


def support_params(n_sink, n_recent, top_k, lam, knorm_beta=0.0, knorm_c=0.0, nms_radius=0, nms_decay=0.0,
                   excl=0.0):
    """Support parameters; the optional Selector steps (key-norm prior,
    Soft-NMS, exclusivity) are off at their zero defaults."""
    return sfi_support_params(int(n_sink), int(n_recent), int(top_k), float(lam), float(knorm_beta),
                              float(knorm_c), int(nms_radius), float(nms_decay), float(excl))


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------- entry points
def sfi_workspace_bytes(kv: KVDesc, sp=None, op=SFI_OP_SLOW):
    n = lib().sfi_workspace_bytes(C.byref(kv.desc), C.byref(sp) if sp is not None else None, int(op))
    if n == 0 and op != SFI_OP_SELECT:
        _check(SFI_ERR_INVALID_ARG, "sfi_workspace_bytes")
    return int(n)


def sfi_workspace_init(ws, stream=None):
    if ws is None:
        return
    _check(lib().sfi_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "sfi_workspace_init")


def alloc_workspace(kv: KVDesc, sp=None, ops=(SFI_OP_SLOW, SFI_OP_SELECT, SFI_OP_FAST, SFI_OP_SLOW_SELECT)):
    """One workspace large enough for every op in ``ops`` (torch allocation),
    prepared with sfi_workspace_init."""
    import torch
    need = max(sfi_workspace_bytes(kv, sp, op) for op in ops if sp is not None or op == SFI_OP_SLOW)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=kv.k.device)
    sfi_workspace_init(ws)
    return ws


def sfi_slow_step(kv: KVDesc, seq_ids, q, out, mass=None, ws=None, stream=None):
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    if mass is not None:
        _need(mass, torch.float32, (B, Hkv, kv.capacity), "mass")
    _, ids, n = _ids(seq_ids)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_slow_step(C.byref(kv.desc), ids, n, _ptr(q), _ptr(out), _ptr(mass), _ptr(ws), nbytes,
                               _stream(stream)), "sfi_slow_step")


def sfi_slow_plan(kv: KVDesc, seq_ids, with_mass=True):
    """Split-K partials per KV head the slow step forms for each listed row
    (with_mass: the step that writes mass, else the dense-only step)."""
    _, ids, n = _ids(seq_ids)
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(lib().sfi_slow_plan(C.byref(kv.desc), ids, n, 1 if with_mass else 0,
                               out.ctypes.data_as(C.POINTER(C.c_int32))), "sfi_slow_plan")
    return out[:n].tolist()


def sfi_fast_plan(kv: KVDesc, sp, seq_ids):
    """Partials per KV head the fast step forms for each listed row."""
    _, ids, n = _ids(seq_ids)
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(lib().sfi_fast_plan(C.byref(kv.desc), C.byref(sp), ids, n, out.ctypes.data_as(C.POINTER(C.c_int32))),
           "sfi_fast_plan")
    return out[:n].tolist()


def sfi_select(kv: KVDesc, sp, seq_ids, mass, sel_idx, sel_cnt, ws=None, stream=None):
    import torch
    B, Hkv = kv.batch, kv.n_kv_heads
    _need(mass, torch.float32, (B, Hkv, kv.capacity), "mass")
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    _, ids, n = _ids(seq_ids)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_select(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(mass), _ptr(sel_idx), _ptr(sel_cnt),
                            _ptr(ws), nbytes, _stream(stream)), "sfi_select")


def sfi_slow_step_select(kv: KVDesc, sp, seq_ids, q, out, mass, sel_idx, sel_cnt, packed_k=None, packed_v=None,
                         ws=None, stream=None):
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    _need(mass, torch.float32, (B, Hkv, kv.capacity), "mass")
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    if packed_k is not None or packed_v is not None:
        _need(packed_k, kv.dtype, (B, Hkv, sp.top_k, D), "packed_k")
        _need(packed_v, kv.dtype, (B, Hkv, sp.top_k, D), "packed_v")
    _, ids, n = _ids(seq_ids)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_slow_step_select(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(q), _ptr(out), _ptr(mass),
                                      _ptr(sel_idx), _ptr(sel_cnt), _ptr(packed_k), _ptr(packed_v), _ptr(ws),
                                      nbytes, _stream(stream)), "sfi_slow_step_select")


def sfi_slow_step_select_async(kv: KVDesc, sp, seq_ids, q, out, mass, sel_idx, sel_cnt, packed_k, packed_v, ws,
                               stream, select_stream):
    """Like sfi_slow_step_select, with the Selector on ``select_stream`` (see
    include/sfi.h for the ordering the caller owes)."""
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    _need(mass, torch.float32, (B, Hkv, kv.capacity), "mass")
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    if packed_k is not None or packed_v is not None:
        _need(packed_k, kv.dtype, (B, Hkv, sp.top_k, D), "packed_k")
        _need(packed_v, kv.dtype, (B, Hkv, sp.top_k, D), "packed_v")
    if stream is None or select_stream is None or _stream(stream).value == _stream(select_stream).value:
        raise ValueError("stream and select_stream must be two distinct streams")
    _, ids, n = _ids(seq_ids)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_slow_step_select_async(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(q), _ptr(out), _ptr(mass),
                                            _ptr(sel_idx), _ptr(sel_cnt), _ptr(packed_k), _ptr(packed_v),
                                            _ptr(ws), nbytes, _stream(stream), _stream(select_stream)),
           "sfi_slow_step_select_async")


def sfi_fast_step(kv: KVDesc, sp, seq_ids, q, sel_idx, sel_cnt, out, ws, stream=None):
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    _, ids, n = _ids(seq_ids)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_fast_step(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(q), _ptr(sel_idx), _ptr(sel_cnt),
                               _ptr(out), _ptr(ws), nbytes, _stream(stream)), "sfi_fast_step")


def sfi_fast_step_pack(kv: KVDesc, sp, seq_ids, q, sel_idx, sel_cnt, out, packed_k, packed_v, ws, stream=None,
                       pack_flags=None):
    """pack_flags: one flag per listed row (None: every row packs); a row
    whose flag is 0 reads the packed rows an earlier call wrote."""
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    _need(packed_k, kv.dtype, (B, Hkv, sp.top_k, D), "packed_k")
    _need(packed_v, kv.dtype, (B, Hkv, sp.top_k, D), "packed_v")
    _, ids, n = _ids(seq_ids)
    flags = None
    if pack_flags is not None:
        flags = np.ascontiguousarray(np.asarray(pack_flags, dtype=np.int32))
        if flags.shape != (n,):
            raise ValueError(f"pack_flags must hold one flag per listed row ({n}), got shape {flags.shape}")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_fast_step_pack(C.byref(kv.desc), C.byref(sp), ids, n,
                                    None if flags is None else flags.ctypes.data_as(C.POINTER(C.c_int32)), _ptr(q),
                                    _ptr(sel_idx), _ptr(sel_cnt), _ptr(out), _ptr(packed_k), _ptr(packed_v), _ptr(ws),
                                    nbytes, _stream(stream)),
           "sfi_fast_step_pack")


def sfi_pack_support(kv: KVDesc, sp, seq_ids, sel_idx, sel_cnt, packed_k, packed_v, stream=None):
    import torch
    B, Hkv, D = kv.batch, kv.n_kv_heads, kv.head_dim
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    _need(packed_k, kv.dtype, (B, Hkv, sp.top_k, D), "packed_k")
    _need(packed_v, kv.dtype, (B, Hkv, sp.top_k, D), "packed_v")
    _, ids, n = _ids(seq_ids)
    _check(lib().sfi_pack_support(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(sel_idx), _ptr(sel_cnt),
                                  _ptr(packed_k), _ptr(packed_v), _stream(stream)), "sfi_pack_support")


def sfi_fast_step_packed(kv: KVDesc, sp, seq_ids, q, packed_k, packed_v, sel_cnt, out, ws, stream=None):
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    _need(packed_k, kv.dtype, (B, Hkv, sp.top_k, D), "packed_k")
    _need(packed_v, kv.dtype, (B, Hkv, sp.top_k, D), "packed_v")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    _, ids, n = _ids(seq_ids)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sfi_fast_step_packed(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(q), _ptr(packed_k),
                                      _ptr(packed_v), _ptr(sel_cnt), _ptr(out), _ptr(ws), nbytes,
                                      _stream(stream)), "sfi_fast_step_packed")


def sfi_fast_step_packed_noalloc(kv: KVDesc, sp, seq_ids, q, packed_k, packed_v, sel_cnt, out, stream=None):
    """sfi_fast_step_packed with the library's fixed per-device scratch in
    place of a workspace (the call allocates nothing)."""
    import torch
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    _need(q, kv.dtype, (B, Hq, D), "q")
    _need(out, torch.float32, (B, Hq, D), "out")
    _need(packed_k, kv.dtype, (B, Hkv, sp.top_k, D), "packed_k")
    _need(packed_v, kv.dtype, (B, Hkv, sp.top_k, D), "packed_v")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    _, ids, n = _ids(seq_ids)
    _check(lib().sfi_fast_step_packed_noalloc(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(q), _ptr(packed_k),
                                              _ptr(packed_v), _ptr(sel_cnt), _ptr(out), _stream(stream)),
           "sfi_fast_step_packed_noalloc")


def sfi_kv_append(kv: KVDesc, seq_ids, k_new, v_new, stream=None):
    B, Hkv, D = kv.batch, kv.n_kv_heads, kv.head_dim
    _need(k_new, kv.dtype, (B, Hkv, D), "k_new")
    _need(v_new, kv.dtype, (B, Hkv, D), "v_new")
    _, ids, n = _ids(seq_ids)
    _check(lib().sfi_kv_append(C.byref(kv.desc), ids, n, _ptr(k_new), _ptr(v_new), _stream(stream)),
           "sfi_kv_append")


def sfi_debug_support(kv: KVDesc, sp, seq_ids, sel_idx, sel_cnt, support_out, support_cnt, stream=None):
    import torch
    B, Hkv = kv.batch, kv.n_kv_heads
    _need(sel_idx, torch.int32, (B, Hkv, sp.top_k), "sel_idx")
    _need(sel_cnt, torch.int32, (B, Hkv), "sel_cnt")
    if support_out.dim() != 3 or support_out.shape[:2] != (B, Hkv):
        raise ValueError("support_out must be [B, Hkv, cap]")
    _need(support_out, torch.int32, tuple(support_out.shape), "support_out")
    _need(support_cnt, torch.int32, (B, Hkv), "support_cnt")
    _, ids, n = _ids(seq_ids)
    _check(lib().sfi_debug_support(C.byref(kv.desc), C.byref(sp), ids, n, _ptr(sel_idx), _ptr(sel_cnt),
                                   _ptr(support_out), _ptr(support_cnt), int(support_out.shape[2]),
                                   _stream(stream)), "sfi_debug_support")


# ---------------------------------------------------------------- scheduler
class Scheduler:
    """Host boundary scheduler (sfi_sched_*)."""

    def __init__(self, batch, seed, mode, span_param, t_max=0):
        self._h = C.c_void_p()
        modes = {"fixed": SFI_SPAN_FIXED, "geometric": SFI_SPAN_GEOMETRIC}
        if mode not in modes and mode not in modes.values():
            raise ValueError(f"unknown span mode {mode!r}")
        m = modes.get(mode, mode)
        _check(lib().sfi_sched_create(int(batch), C.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(m),
                                      float(span_param), int(t_max), C.byref(self._h)), "sfi_sched_create")
        self.batch = int(batch)
        self._slow = (C.c_int32 * self.batch)()
        self._fast = (C.c_int32 * self.batch)()

    def step(self):
        """Returns (slow_ids, fast_ids) as lists for the next decode step."""
        ns, nf = C.c_int32(), C.c_int32()
        _check(lib().sfi_sched_step(self._h, self._slow, C.byref(ns), self._fast, C.byref(nf)), "sfi_sched_step")
        return list(self._slow[:ns.value]), list(self._fast[:nf.value])

    def force_slow(self, seq):
        _check(lib().sfi_sched_force_slow(self._h, int(seq)), "sfi_sched_force_slow")

    def close(self):
        if self._h:
            lib().sfi_sched_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- timing
def sfi_profile_enable(on=True):
    _check(lib().sfi_profile_enable(1 if on else 0), "sfi_profile_enable")


def sfi_profile_reset():
    _check(lib().sfi_profile_reset(), "sfi_profile_reset")


def sfi_profile_read(kernel):
    ms, n = C.c_double(), C.c_int64()
    _check(lib().sfi_profile_read(int(kernel), C.byref(ms), C.byref(n)), "sfi_profile_read")
    return ms.value, n.value


def sfi_version():
    return int(lib().sfi_version())


def sfi_status_str(status):
    return lib().sfi_status_str(int(status)).decode()
