"""The fast step's rows per wave are a launch parameter (SFI_FAST_TILES = 1, 2
or 4 tiles of 16 rows; the library reads it once per process).  bf16 waves of
2 and 4 tiles take the MFMA P.V path (one or two 32-row groups), 1 tile and
fp32 the VALU path.  Each setting runs in a child process (one at a time) on
ragged batches and is checked against the oracle; packed, gather and the
packing fast step (all rows packing, or mixed with rows reading packed rows)
must stay bit-identical."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, check_support, np64, oracle_slow, random_cache

for dtype, D, G in ((torch.bfloat16, 128, 4), (torch.bfloat16, 64, 8), (torch.bfloat16, 128, 1),
                    (torch.float32, 64, 4)):
    ctx = [5000, 1300, 333, 40]
    B, Hkv, ns, W, k = len(ctx), 2, 16, 64, 700
    kv, q = random_cache(B, G * Hkv, Hkv, 5000, D, dtype, ctx, seed=D + G, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(ns, W, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = list(range(B))
    out = torch.empty(B, G * Hkv, D, device=dev)
    mass = torch.empty(B, Hkv, 5000, device=dev)
    sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    pk = torch.empty(B, Hkv, k, D, dtype=dtype, device=dev)
    pv = torch.empty_like(pk)
    S.sfi_slow_step_select(kv, sp, ids, q, out, mass, sel, cnt, pk, pv, ws)
    out_p = torch.full_like(out, 7.0)
    out_g = torch.full_like(out, 7.0)
    S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, out_p, ws)
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_g, ws)
    # the packing fast step: every row packing into empty buffers, then rows
    # that pack beside rows reading the packed rows (one mixed launch); outputs
    # equal the gather step's and the packed rows the refresh's bit for bit
    for flags in ([1, 1, 1, 1], [1, 0, 0, 1]):
        pk2 = pk.clone() if 0 in flags else torch.full_like(pk, float("nan"))
        pv2 = pv.clone() if 0 in flags else torch.full_like(pv, float("nan"))
        out_k = torch.full_like(out, 7.0)
        S.sfi_fast_step_pack(kv, sp, ids, q, sel, cnt, out_k, pk2, pv2, ws, pack_flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(out_k, out_g), (dtype, D, G, flags)
        for b in ids:
            for g in range(Hkv):
                c = int(cnt[b, g])
                assert torch.equal(pk2[b, g, :c], pk[b, g, :c]) and torch.equal(pv2[b, g, :c], pv[b, g, :c])
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_g), (dtype, D, G)
    for b in ids:
        T = ctx[b]
        _, f_ref = oracle_slow(kv, q, b)
        sels = []
        for g in range(Hkv):
            s = sel[b, g, :int(cnt[b, g])].cpu().numpy().astype(np.int64)
            check_support(s, f_ref[g], T, ns, W, k, 0.1, f"b{b} g{g}")
            sels.append(s)
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, ns, W, sels)
        err = float(np.max(np.abs(np64(out_p[b]) - ref)))
        assert err < OUT_TOL, (dtype, D, G, b, err)
    print("ok", dtype, D, G, flush=True)
print("all ok", flush=True)
"""


@pytest.mark.parametrize("tiles", [1, 2, 4])
def test_fast_step_rows_per_wave(tiles):
    env = dict(os.environ, SFI_FAST_TILES=str(tiles))
    print(f"SFI_FAST_TILES={tiles}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and "all ok" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
