"""GPU tests of decode-cache upkeep (dash_cache_append) through the C ABI.

After a run of appends the K/V caches must hold exactly the appended rows,
every chunk the appends completed must hold its summary -- bit for bit what
dash_summarize computes on the cache, and within the summary bound of the
oracle's summary -- and nothing else may change.  A generation loop (append,
then decode) must match the oracle's decode of the sequence so far.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_hierarchical_attention_dash_amd import ops
from sparse_hierarchical_attention_dash_amd import workloads as W

from gpu_helpers import LSE_TOL, TOL, check_summaries, flush, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _dt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


CASES = [
    # name, dtype, batch, cap, Hkv, D, B, start lengths, steps
    ("bf16-d128-b64", "bf16", 3, 512, 2, 128, 64, [0, 63, 300], 200),
    ("f32-d64-b128", "f32", 2, 512, 2, 64, 128, [1, 255], 150),
    ("bf16-d64-b128-hkv1", "bf16", 2, 384, 1, 64, 128, [127, 0], 130),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_appends_fill_caches_and_summaries(case):
    name, dtype, batch, cap, Hkv, D, B, start, steps = case
    flush(f"cache append {name}")
    rng = np.random.default_rng(31)
    seq_k = rng.standard_normal((batch, cap, Hkv, D)).astype(np.float32)
    seq_v = rng.standard_normal((batch, cap, Hkv, D)).astype(np.float32)
    qbar = (0.1 * rng.standard_normal((Hkv, D))).astype(np.float32)
    kdev, kx = to_dev(seq_k, dtype)
    vdev, vx = to_dev(seq_v, dtype)
    qb = torch.from_numpy(qbar).cuda()
    kc = torch.full((batch, cap, Hkv, D), SENTINEL, dtype=_dt(dtype), device="cuda")
    vc = torch.full_like(kc, SENTINEL)
    kb = torch.full((batch, cap // B, Hkv, D), SENTINEL, dtype=_dt(dtype), device="cuda")
    # the prefixes: rows copied in, their complete chunks summarised
    for b in range(batch):
        n0 = start[b]
        kc[b, :n0] = kdev[b, :n0]
        vc[b, :n0] = vdev[b, :n0]
        if n0 >= B:
            kb[b, :n0 // B] = ops.summarize(kc[b, :n0 // B * B].contiguous(), qb, B)
    for t in range(steps):
        sl = torch.tensor([start[b] + t + 1 for b in range(batch)], dtype=torch.int32,
                          device="cuda")
        idx = torch.tensor([start[b] + t for b in range(batch)], device="cuda")
        kn = kdev[torch.arange(batch, device="cuda"), idx].contiguous()
        vn = vdev[torch.arange(batch, device="cuda"), idx].contiguous()
        ops.cache_append(kn, vn, sl, qb, kc, vc, kb, B)
    torch.cuda.synchronize()
    end = [start[b] + steps for b in range(batch)]
    for b in range(batch):
        n = end[b]
        assert torch.equal(kc[b, :n], kdev[b, :n]) and torch.equal(vc[b, :n], vdev[b, :n])
        assert bool((kc[b, n:] == SENTINEL).all()) and bool((vc[b, n:] == SENTINEL).all())
        C = n // B
        assert bool((kb[b, C:] == SENTINEL).all())
        if C == 0:
            continue
        ref = ops.summarize(kc[b, :C * B].contiguous(), qb, B)
        torch.cuda.synchronize()
        assert torch.equal(kb[b, :C], ref), f"{name} b={b}: cached != dash_summarize"
        ora = O.summarize(kx[b, :C * B], qbar.astype(np.float64), B, to_bf16=(dtype == "bf16"))
        check_summaries(kb[b, :C].to(torch.float64).cpu().numpy(), ora, dtype, kx[b, :C * B], B)


def test_generation_loop_matches_oracle_decode():
    # append each new token, then decode it; compare with the oracle's decode
    # of the sequence so far (on the cached summaries, checked above)
    flush("generation loop")
    batch, cap, Hq, Hkv, D, B = 2, 1024, 32, 2, 128, 64
    alpha, gamma, sigma = 1.5, 20.0, 1.0
    start, steps = [100, 500], 140
    d = W.gen_decode(batch, cap, Hq, Hkv, D, seed=41)
    rng = np.random.default_rng(42)
    qs = rng.standard_normal((steps, batch, Hq, D)).astype(np.float32)
    kdev, kx = to_dev(d["k_cache"], "bf16")
    vdev, vx = to_dev(d["v_cache"], "bf16")
    qdev, qx = to_dev(qs, "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    kc = torch.zeros((batch, cap, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kb = torch.zeros((batch, cap // B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    for b in range(batch):
        kc[b, :start[b]] = kdev[b, :start[b]]
        vc[b, :start[b]] = vdev[b, :start[b]]
        C = start[b] // B
        kb[b, :C] = ops.summarize(kc[b, :C * B].contiguous(), qb, B)
    ws = ops.decode_workspace(qdev[0], kc, B)
    ar = torch.arange(batch, device="cuda")
    check_at = {0, 27, 28, 29, steps - 1}       # 128 = 100 + 28: a chunk completes
    for t in range(steps):
        L = [start[b] + t + 1 for b in range(batch)]
        sl = torch.tensor(L, dtype=torch.int32, device="cuda")
        idx = torch.tensor([x - 1 for x in L], device="cuda")
        ops.cache_append(kdev[ar, idx].contiguous(), vdev[ar, idx].contiguous(), sl, qb, kc, vc,
                         kb, B)
        out, lse, _ = ops.attn_decode(qdev[t], kc, vc, sl, kb, B, alpha=alpha, gamma=gamma,
                                      sigma=sigma, return_lse=True, workspace=ws)
        if t not in check_at:
            continue
        torch.cuda.synchronize()
        kbx = kb.to(torch.float64).cpu().numpy()
        o = out.to(torch.float64).cpu().numpy()
        le = lse.cpu().numpy()
        for b in range(batch):
            r = O.decode(qx[t, b], kx[b], vx[b], kbx[b], L[b], B, alpha, gamma, sigma, True)
            err = np.max(np.abs(o[b] - r["out"]))
            assert err <= TOL["bf16"], (t, b, err)
            assert np.max(np.abs(le[:, b] - r["lse"])) <= LSE_TOL["bf16"], (t, b)
    # the summaries the loop cached are the oracle's
    torch.cuda.synchronize()
    for b in range(batch):
        n = start[b] + steps
        C = n // B
        ora = O.summarize(kx[b, :C * B], d["qbar"].astype(np.float64), B, to_bf16=True)
        check_summaries(kb[b, :C].to(torch.float64).cpu().numpy(), ora, "bf16", kx[b, :C * B], B)


FUSED_CASES = [
    # name, dtype, batch, cap, Hq, Hkv, D, B, start lengths, steps, estimate_diagonal
    ("bf16-g16", "bf16", 3, 512, 32, 2, 128, 64, [1, 62, 300], 70, False),
    ("bf16-g16-diag", "bf16", 2, 512, 32, 2, 128, 64, [60, 200], 40, True),
    ("bf16-d64-b128-g4", "bf16", 2, 512, 8, 2, 64, 128, [126, 0], 40, False),
    ("f32-g1", "f32", 2, 256, 2, 2, 64, 64, [62, 5], 20, False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: c[0])
def test_fused_append_step_equals_append_then_decode(case):
    # dash_attn_decode_append against dash_cache_append + dash_attn_decode on
    # twin caches: outputs, LSE, masks and all three caches bit for bit, over
    # steps that complete chunks (the fused path for bf16 without estimates,
    # the separate launch otherwise)
    name, dtype, batch, cap, Hq, Hkv, D, B, start, steps, diag = case
    flush(f"fused append step {name}")
    rng = np.random.default_rng(53)
    seq_k = rng.standard_normal((batch, cap, Hkv, D)).astype(np.float32)
    seq_v = rng.standard_normal((batch, cap, Hkv, D)).astype(np.float32)
    qs = rng.standard_normal((steps, batch, Hq, D)).astype(np.float32)
    qbar = (0.1 * rng.standard_normal((Hkv, D))).astype(np.float32)
    kdev, _ = to_dev(seq_k, dtype)
    vdev, _ = to_dev(seq_v, dtype)
    qdev, _ = to_dev(qs, dtype)
    qb = torch.from_numpy(qbar).cuda()
    kc = torch.full((batch, cap, Hkv, D), SENTINEL, dtype=_dt(dtype), device="cuda")
    vc = torch.full_like(kc, SENTINEL)
    kb = torch.full((batch, cap // B, Hkv, D), SENTINEL, dtype=_dt(dtype), device="cuda")
    for b in range(batch):
        n0 = start[b]
        kc[b, :n0] = kdev[b, :n0]
        vc[b, :n0] = vdev[b, :n0]
        if n0 >= B:
            kb[b, :n0 // B] = ops.summarize(kc[b, :n0 // B * B].contiguous(), qb, B)
    kc2, vc2, kb2 = kc.clone(), vc.clone(), kb.clone()
    ws = ops.decode_workspace(qdev[0], kc, B)
    ws2 = ops.decode_workspace(qdev[0], kc, B)
    ar = torch.arange(batch, device="cuda")
    kw = dict(alpha=1.5, gamma=8.0, sigma=1.0, return_lse=True, return_active_blocks=True,
              estimate_diagonal=diag)
    completed = 0
    for t in range(steps):
        L = [start[b] + t + 1 for b in range(batch)]
        completed += sum(1 for x in L if x % B == 0)
        sl = torch.tensor(L, dtype=torch.int32, device="cuda")
        idx = torch.tensor([x - 1 for x in L], device="cuda")
        kn, vn = kdev[ar, idx].contiguous(), vdev[ar, idx].contiguous()
        ops.cache_append(kn, vn, sl, qb, kc, vc, kb, B)
        o1, l1, a1 = ops.attn_decode(qdev[t], kc, vc, sl, kb, B, workspace=ws, qbar=qb, **kw)
        o2, l2, a2 = ops.attn_decode_append(qdev[t], kn, vn, kc2, vc2, sl, kb2, qb, B,
                                            workspace=ws2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), (t, "out")
        assert torch.equal(l1, l2), (t, "lse")
        assert torch.equal(a1, a2), (t, "active_blocks")
    assert completed > 0
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2) and torch.equal(kb, kb2)
    flush(f"  {name}: {steps} steps, {completed} chunks completed, bit-exact")
