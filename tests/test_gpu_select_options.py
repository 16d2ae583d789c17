"""GPU parity of the optional Selector steps (gist.science technical summary,
2.B: the key-norm correction of the prior, Soft-NMS within a head and the
exclusivity between heads) against the oracle's select_heads: supports exact
beyond the score gap, tie-tolerant inside it, on ragged batches, alone and
combined, through the fused refresh (with packing) and the separate Selector
call."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, check_mass, check_support_scores, np64, oracle_slow, random_cache

pytestmark = pytest.mark.gpu

OPTIONS = {
    "nms": dict(nms_radius=2, nms_decay=0.5),
    "nms_wide": dict(nms_radius=32, nms_decay=1.0),
    "excl": dict(excl=1.0),
    "knorm": dict(knorm_beta=1.0, knorm_c=1.0),
    "knorm_strong": dict(knorm_beta=8.0, knorm_c=0.0),
    "all": dict(knorm_beta=0.7, knorm_c=0.5, nms_radius=3, nms_decay=0.6, excl=2.0),
}


def _planted(kv, q, seed):
    """Heavy positions (a run of neighbours and scattered ones) and extreme
    key norms on some candidates, so that every option changes selections."""
    g = torch.Generator()
    g.manual_seed(seed)
    B, Hkv, cap, D = kv.k.shape
    G = kv.n_q_heads // Hkv
    for b in range(B):
        T = int(kv.ctx[b])
        for h in range(Hkv):
            u = q[b, h * G].float()
            u = u / u.norm()
            for j in list(range(40, 52)) + torch.randint(60, max(61, T - 300), (24,), generator=g).tolist():
                if j < T:
                    kv.k[b, h, j] = (kv.k[b, h, j].float() + 3.0 * u).to(kv.k.dtype)
            big = torch.randint(20, max(21, T - 300), (6,), generator=g).tolist()
            for j in big:
                if j < T:
                    kv.k[b, h, j] = (kv.k[b, h, j].float() * 12.0).to(kv.k.dtype)


def _buffers(kv, k):
    dev = kv.k.device
    B, Hq, Hkv, D = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim
    return dict(out=torch.full((B, Hq, D), float("nan"), device=dev),
                mass=torch.full((B, Hkv, kv.capacity), -1.0, device=dev),
                sel=torch.full((B, Hkv, k), -7, dtype=torch.int32, device=dev),
                cnt=torch.full((B, Hkv), -7, dtype=torch.int32, device=dev),
                pk=torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev),
                pv=torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev))


@pytest.mark.parametrize("name", sorted(OPTIONS))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_refresh_with_options_matches_oracle(name, dtype):
    opts = OPTIONS[name]
    ctx = [9000, 3100, 700]
    ns, W, k, lam = 8, 64, 300, 0.1
    kv, q = random_cache(3, 16, 4, 9000, 128, dtype, ctx, seed=81, q_scale=2.0)
    _planted(kv, q, 82)
    sp = S.support_params(ns, W, k, lam, **opts)
    ws = S.alloc_workspace(kv, sp)
    o = _buffers(kv, k)
    ids = [0, 1, 2]
    S.sfi_slow_step_select(kv, sp, ids, q, o["out"], o["mass"], o["sel"], o["cnt"], o["pk"], o["pv"], ws)
    torch.cuda.synchronize()
    kinds = []
    for b, T in enumerate(ctx):
        o_ref, f_ref = oracle_slow(kv, q, b)
        assert np.max(np.abs(np64(o["out"][b]) - o_ref)) < OUT_TOL
        check_mass(np64(o["mass"][b, :, :T]), f_ref, b)
        K64 = np64(kv.k[b, :, :T])
        sels, Sc, cand = O.select_heads(f_ref, K64, T, ns, W, k, lam, **opts)
        for g in range(kv.n_kv_heads):
            c = int(o["cnt"][b, g])
            got = o["sel"][b, g, :c].cpu().numpy()
            kinds.append(check_support_scores(got, sels[g], Sc[g], cand, k, f"{name} b{b} g{g}"))
            rows = torch.from_numpy(got.astype(np.int64)).to(kv.k.device)
            assert torch.equal(o["pk"][b, g, :c], kv.k[b, g].index_select(0, rows))
            assert torch.equal(o["pv"][b, g, :c], kv.v[b, g].index_select(0, rows))
    assert "exact" in kinds


@pytest.mark.parametrize("name", ["nms", "excl", "nms_wide"])
def test_separate_selector_with_options_equals_fused(name):
    """Without the key-norm correction the options also run in sfi_select:
    on the same mass it gives the fused refresh's selection bit for bit."""
    opts = OPTIONS[name]
    ctx = [6000, 2500]
    kv, q = random_cache(2, 32, 8, 6000, 128, torch.bfloat16, ctx, seed=83, q_scale=2.0)
    _planted(kv, q, 84)
    sp = S.support_params(16, 256, 512, 0.1, **opts)
    ws = S.alloc_workspace(kv, sp)
    a, b = _buffers(kv, 512), _buffers(kv, 512)
    S.sfi_slow_step_select(kv, sp, [0, 1], q, a["out"], a["mass"], a["sel"], a["cnt"], None, None, ws)
    S.sfi_slow_step(kv, [0, 1], q, b["out"], b["mass"], ws)
    S.sfi_select(kv, sp, [0, 1], b["mass"], b["sel"], b["cnt"], ws)
    torch.cuda.synchronize()
    assert torch.equal(a["mass"], b["mass"])
    assert torch.equal(a["sel"], b["sel"]) and torch.equal(a["cnt"], b["cnt"])


def test_options_change_the_gpu_selection_and_zero_options_do_not():
    """The options move the GPU's selection (as they move the oracle's), and
    an all-zero option set is the plain Selector bit for bit."""
    ctx = [8000]
    kv, q = random_cache(1, 32, 8, 8000, 128, torch.bfloat16, ctx, seed=85, q_scale=2.0)
    _planted(kv, q, 86)
    ws = S.alloc_workspace(kv, S.support_params(16, 256, 400, 0.1, **OPTIONS["all"]))
    res = {}
    for name, opts in (("plain", {}), ("zero", dict(knorm_beta=0.0, nms_radius=5, nms_decay=0.0, excl=0.0)),
                       ("all", OPTIONS["all"])):
        sp = S.support_params(16, 256, 400, 0.1, **opts)
        o = _buffers(kv, 400)
        S.sfi_slow_step_select(kv, sp, [0], q, o["out"], o["mass"], o["sel"], o["cnt"], o["pk"], o["pv"], ws)
        torch.cuda.synchronize()
        res[name] = o
    for key in res["plain"]:
        assert torch.equal(res["plain"][key], res["zero"][key]), key
    assert not torch.equal(res["plain"]["sel"], res["all"]["sel"])
