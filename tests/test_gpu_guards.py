"""Guard bytes: every output, packed buffer and the workspace sits between
guard regions filled with a pattern; after every entry point has run on a
ragged batch, no byte outside the documented extents has changed."""
import numpy as np
import pytest
import torch

import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import random_cache

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side (keeps the 256-byte alignment of the views)


class Guarded:
    """A view of `shape` inside a byte buffer with guard regions around it."""

    def __init__(self, shape, dtype, device, fill_byte=0x5A):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.buf = torch.full((GUARD + n * esz + GUARD,), fill_byte, dtype=torch.uint8, device=device)
        self.fill = fill_byte
        self.view = self.buf[GUARD:GUARD + n * esz].view(dtype).view(shape)

    def intact(self):
        return bool(torch.all(self.buf[:GUARD] == self.fill)) and bool(torch.all(self.buf[-GUARD:] == self.fill))


def test_no_write_outside_outputs_and_workspace():
    ctx = [3000, 700, 50, 2999]
    B, Hq, Hkv, D, cap, k = len(ctx), 32, 8, 128, 3000, 256
    kv, q = random_cache(B, Hq, Hkv, cap, D, torch.bfloat16, ctx, seed=31, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 64, k, 0.1)
    need = max(S.sfi_workspace_bytes(kv, sp, op) for op in
               (S.SFI_OP_SLOW, S.SFI_OP_SELECT, S.SFI_OP_FAST, S.SFI_OP_SLOW_SELECT))
    ws = Guarded((need,), torch.uint8, dev)
    S.sfi_workspace_init(ws.view)
    out = Guarded((B, Hq, D), torch.float32, dev)
    mass = Guarded((B, Hkv, cap), torch.float32, dev)
    sel = Guarded((B, Hkv, k), torch.int32, dev)
    cnt = Guarded((B, Hkv), torch.int32, dev)
    pk = Guarded((B, Hkv, k, D), torch.bfloat16, dev)
    pv = Guarded((B, Hkv, k, D), torch.bfloat16, dev)
    ids = [0, 1, 2, 3]
    S.sfi_slow_step_select(kv, sp, ids, q, out.view, mass.view, sel.view, cnt.view, pk.view, pv.view, ws.view)
    S.sfi_fast_step_packed(kv, sp, ids, q, pk.view, pv.view, cnt.view, out.view, ws.view)
    S.sfi_fast_step(kv, sp, ids, q, sel.view, cnt.view, out.view, ws.view)
    S.sfi_slow_step(kv, ids, q, out.view, mass.view, ws.view)
    S.sfi_select(kv, sp, ids, mass.view, sel.view, cnt.view, ws.view)
    S.sfi_pack_support(kv, sp, ids, sel.view, cnt.view, pk.view, pv.view)
    side = torch.cuda.Stream()
    S.sfi_slow_step_select_async(kv, sp, ids, q, out.view, mass.view, sel.view, cnt.view, pk.view, pv.view,
                                 ws.view, torch.cuda.current_stream(), side)
    torch.cuda.current_stream().wait_stream(side)
    sup = Guarded((B, Hkv, 16 + 64 + k), torch.int32, dev)
    sup_cnt = Guarded((B, Hkv), torch.int32, dev)
    S.sfi_debug_support(kv, sp, ids, sel.view, cnt.view, sup.view, sup_cnt.view)
    torch.cuda.synchronize()
    for name, g in (("workspace", ws), ("out", out), ("mass", mass), ("sel_idx", sel), ("sel_cnt", cnt),
                    ("packed_k", pk), ("packed_v", pv), ("support", sup), ("support_cnt", sup_cnt)):
        assert g.intact(), name
    # the mass beyond each context stays untouched too (the pattern's float value)
    pattern = mass.buf[:4].view(torch.float32)[0]
    for b, T in enumerate(ctx):
        assert torch.all(mass.view[b, :, T:] == pattern), b


def test_kv_append_writes_one_row_per_sequence():
    """The append writes row ctx_len[b] of each listed sequence and nothing
    else of the cache."""
    ctx = [10, 200, 4095]
    B, Hq, Hkv, D, cap = 3, 8, 2, 64, 4096
    kv, _ = random_cache(B, Hq, Hkv, cap, D, torch.float32, ctx, seed=5)
    dev = kv.k.device
    before_k, before_v = kv.k.clone(), kv.v.clone()
    kn = torch.randn(B, Hkv, D, device=dev)
    vn = torch.randn(B, Hkv, D, device=dev)
    S.sfi_kv_append(kv, [0, 2], kn, vn)
    torch.cuda.synchronize()
    mask = torch.zeros(B, Hkv, cap, dtype=torch.bool, device=dev)
    mask[0, :, 10] = True
    mask[2, :, 4095] = True
    assert torch.equal(kv.k[~mask], before_k[~mask]) and torch.equal(kv.v[~mask], before_v[~mask])
    assert torch.equal(kv.k[0, :, 10], kn[0]) and torch.equal(kv.v[2, :, 4095], vn[2])
