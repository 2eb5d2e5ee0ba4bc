"""GPU parity of the HIP library (through its C ABI) against the CPU oracle.

Sizes span several 64-key blocks, several mask words where it matters and a
ragged tail; each case prints its name before it touches the GPU.
Tolerances: outputs max-abs 2e-2 (bf16) / 1e-4 (fp32); mask bits identical
except within 1e-4 of the entmax threshold (logit units).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_hierarchical_attention_dash_amd import ops
from sparse_hierarchical_attention_dash_amd import workloads as W

from gpu_helpers import (BAND, LSE_TOL, TOL, check_summaries, compare_masks, flush, pack_bits,
                         prefill_case, oracle_mask_on, to_dev, unpack_bits)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ phase 0

@pytest.mark.parametrize("dtype,D,B", [("bf16", 128, 64), ("bf16", 64, 128), ("f32", 64, 64),
                                       ("f32", 128, 128)])
def test_summarize(dtype, D, B):
    flush(f"summarize {dtype} D={D} B={B}")
    d = W.gen_prefill(5 * B + 17, 2, 2, D, seed=11)
    k, kx = to_dev(d["k"], dtype)
    kb = ops.summarize(k, torch.from_numpy(d["qbar"]).cuda(), B)
    torch.cuda.synchronize()
    ref = O.summarize(kx, d["qbar"], B, to_bf16=(dtype == "bf16"))
    got = kb.to(torch.float64).cpu().numpy()
    assert got.shape == ref.shape == (5, 2, D)
    check_summaries(got, ref, dtype, kx, B)


def test_summarize_zero_query_is_mean_and_varlen():
    flush("summarize varlen, q_bar = 0")
    lens = [63, 64, 200, 1, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(12)
    k32 = rng.standard_normal((cu[-1], 2, 128)).astype(np.float32)
    k, kx = to_dev(k32, "bf16")
    qb = np.zeros((2, 128), np.float32)
    kb = ops.summarize(k, torch.from_numpy(qb).cuda(), 64, cu_seqlens=torch.from_numpy(cu).cuda(),
                       max_seqlen=max(lens))
    torch.cuda.synchronize()
    ref = O.summarize_varlen(kx, qb, cu, 64, to_bf16=True)
    got = kb.to(torch.float64).cpu().numpy()[:ref.shape[0]]
    off = 0
    for s_, n_ in enumerate(lens):
        c = n_ // 64
        a = int(cu[s_])
        check_summaries(got[off:off + c], ref[off:off + c], "bf16", kx[a:a + n_], 64)
        off += c


# ------------------------------------------------------------------ phase 1

ROUTE_CASES = [
    # name, dtype, L, Hq, Hkv, D, B, alpha, gamma, sigma
    ("g16-a15", "bf16", 1000, 32, 2, 128, 64, 1.5, 30.0, 1.0),
    ("g16-a125", "bf16", 1000, 32, 2, 128, 64, 1.25, 20.0, 0.7),
    ("g4-a2", "bf16", 900, 8, 2, 64, 64, 2.0, 40.0, 1.0),
    ("g1-a1", "bf16", 700, 2, 2, 128, 128, 1.0, 5.0, 1.0),
    ("g2-f32", "f32", 777, 4, 2, 64, 64, 1.5, 25.0, 2.0),
    ("g16-words", "bf16", 64 * 140 + 9, 32, 2, 128, 64, 1.5, 30.0, 1.0),  # 3 mask words
    ("g32-a2", "bf16", 1000, 32, 1, 128, 64, 2.0, 30.0, 1.0),
    ("g16-d64-a2", "bf16", 900, 32, 2, 64, 64, 2.0, 40.0, 0.5),
    ("g16-b128", "bf16", 2000, 32, 2, 128, 128, 1.5, 30.0, 1.0),
    # nearly flat logits: most chunks are threshold candidates, so the
    # streaming routing hands its row groups to the one-row-per-workgroup path
    ("g16-flat", "bf16", 64 * 100 + 9, 32, 2, 128, 64, 1.5, 0.3, 1.0),
    ("g32-flat-a125", "bf16", 64 * 90, 32, 1, 128, 64, 1.25, 0.5, 1.0),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: c[0])
def test_route_stage(case):
    name, dtype, L, Hq, Hkv, D, B, alpha, gamma, sigma = case
    flush(f"route {name}")
    d = W.gen_prefill(L, Hq, Hkv, D, seed=21)
    C = L // B
    kbar32 = W.gen_summaries(C, Hkv, D, seed=21)
    q, qx = to_dev(d["q"], dtype)
    kb, kbx = to_dev(kbar32, dtype)
    gqa = Hq != Hkv
    mask, lp, tau = ops.route(q, kb, Hkv, B, alpha=alpha, gamma=gamma, sigma=sigma,
                              enable_gqa=gqa, log_prior=True, tau=True)
    torch.cuda.synchronize()
    S = -(-L // B)
    rows = list(range(L)) if L <= 1200 else sorted(
        set(np.random.default_rng(1).integers(0, L, 300).tolist()) | set(range(L - 70, L)))
    G = Hq // Hkv
    s = 1.0 / math.sqrt(D)
    om, olp, oth = O.route_sequence(qx, kbx, B, alpha, gamma, sigma, G, s, rows=rows,
                                    num_slots=S)
    margin = O.routing_margin(qx, kbx, B, gamma, s, G, oth, rows, S)
    bits = unpack_bits(mask, S)[:, rows]
    flips = compare_masks(bits, om[:, rows], margin, f"route {name}")
    # bits of chunks a row cannot route to are zero, also past the slots
    W_ = mask.shape[2]
    allbits = unpack_bits(mask, W_ * 64)
    for j, i in enumerate(rows):
        assert not allbits[:, i, i // B:].any()
    # thresholds (logit units)
    th = tau.cpu().numpy().astype(np.float64)[:, rows]
    ot = oth[:, rows]
    fin = np.isfinite(ot)
    assert np.array_equal(np.isfinite(th), fin)
    assert np.array_equal(np.sign(th[~fin]), np.sign(ot[~fin]))
    assert np.max(np.abs(th[fin] - ot[fin]), initial=0.0) < BAND
    # group weights where both sides are active: w = exp(log_prior / sigma)
    both = bits & om[:, rows]
    g = lp.cpu().numpy().astype(np.float64)[:, rows]
    if sigma > 0:
        wg = np.exp(g[both] / sigma)
        wo = np.exp(olp[:, rows][both] / sigma)
        assert np.max(np.abs(wg - wo), initial=0.0) < 2e-5
    inactive = (~bits) & (np.arange(S)[None, None, :] < (np.array(rows) // B)[None, :, None])
    assert np.all(np.isneginf(g[inactive]))
    flush(f"  route {name}: flips in band {flips}, support "
          f"{bits.sum() / max(1, sum(i // B for i in rows) * Hkv):.3f}")


# ------------------------------------------------------------------ phase 2 alone

SPARSE_CASES = [
    # name, dtype, L, Hq, Hkv, D, B, density
    ("g16-d128", "bf16", 1100, 32, 2, 128, 64, 0.3),
    ("g16-dense", "bf16", 600, 32, 2, 128, 64, 1.0),
    ("g16-empty", "bf16", 600, 32, 2, 128, 64, 0.0),
    ("g4-d64-b128", "bf16", 900, 8, 2, 64, 128, 0.4),
    ("g1", "bf16", 333, 2, 2, 128, 64, 0.5),
    ("g2", "bf16", 500, 4, 2, 128, 64, 0.5),
    ("g8", "bf16", 700, 16, 2, 64, 64, 0.3),
    ("g32", "bf16", 300, 32, 1, 128, 64, 0.3),
    ("f32", "f32", 400, 4, 2, 64, 64, 0.5),
    ("long-3words", "bf16", 64 * 130 + 20, 32, 2, 128, 64, 0.1),
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=lambda c: c[0])
def test_attention_stage(case):
    """Phase 2 alone: the same synthetic routing (mask + log-prior) on both sides."""
    name, dtype, L, Hq, Hkv, D, B, dens = case
    flush(f"sparse attention {name}")
    d = W.gen_prefill(L, Hq, Hkv, D, seed=81)
    mask, lp = W.gen_routing(Hkv, L, B, dens, seed=81)
    q, qx = to_dev(d["q"], dtype)
    k, kx = to_dev(d["k"], dtype)
    v, vx = to_dev(d["v"], dtype)
    ab = torch.from_numpy(pack_bits(mask)).cuda()
    lpt = torch.from_numpy(lp).cuda()
    out, lse = ops.attn_sparse(q, k, v, ab, lpt, B, enable_gqa=(Hq != Hkv), return_lse=True)
    torch.cuda.synchronize()
    rows = list(range(L)) if L <= 1200 else sorted(
        set(np.random.default_rng(2).integers(0, L, 200).tolist()) | set(range(L - 64, L)))
    o_ref, l_ref = O.attention_rows(qx, kx, vx, mask, lp.astype(np.float64), B,
                                    1 / math.sqrt(D), Hq // Hkv, rows)
    o = out.to(torch.float64).cpu().numpy()[rows]
    err = np.max(np.abs(o - o_ref))
    assert err <= TOL[dtype], err
    lerr = np.max(np.abs(lse.cpu().numpy()[:, rows] - l_ref))
    assert lerr <= LSE_TOL[dtype], lerr
    flush(f"  sparse {name}: max-abs {err:.2e} lse {lerr:.2e}")


# ------------------------------------------------------------------ phases 0-2

PREFILL_CASES = [
    # name, dtype, L, Hq, Hkv, D, B, alpha, gamma, sigma, gqa
    ("tiny-f32-g1", "f32", 512, 1, 1, 64, 64, 1.5, 1.0, 1.0, False),
    ("tiny-f32-g20", "f32", 512, 1, 1, 64, 64, 1.5, 20.0, 1.0, False),
    ("tiny-f32-g50", "f32", 512, 1, 1, 64, 64, 1.5, 50.0, 1.0, False),
    ("g16-d128-b64", "bf16", 1000, 32, 2, 128, 64, 1.5, 30.0, 1.0, True),
    ("g4-d64-b128", "bf16", 777, 8, 2, 64, 128, 1.25, 20.0, 0.5, True),
    ("g1-d128-a2", "bf16", 300, 2, 2, 128, 64, 2.0, 30.0, 1.0, False),
    ("g2-softmax-s0", "bf16", 500, 4, 2, 128, 64, 1.0, 3.0, 0.0, True),
    ("g8-b128", "bf16", 1100, 16, 2, 128, 128, 1.5, 30.0, 1.0, True),
    ("g32", "bf16", 400, 32, 1, 128, 64, 1.5, 30.0, 1.0, True),
    ("g4-f32-b128", "f32", 600, 8, 2, 128, 128, 1.5, 30.0, 1.0, True),
    ("short", "bf16", 50, 32, 2, 128, 64, 1.5, 30.0, 1.0, True),
    ("exact-chunk", "bf16", 128, 32, 2, 128, 64, 1.5, 30.0, 1.0, True),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: c[0])
def test_prefill(case):
    name, dtype, L, Hq, Hkv, D, B, alpha, gamma, sigma, gqa = case
    flush(f"prefill {name}")
    d = W.gen_prefill(L, Hq, Hkv, D, seed=31, B=B)
    r = prefill_case(d, B, alpha, gamma, sigma, dtype, gqa=gqa)
    flush(f"  prefill {name}: max-abs {r['err']:.2e} lse {r['lse_err']:.2e} flips {r['flips']}")


def test_prefill_custom_scale_and_needles():
    flush("prefill needles + custom scale")
    d = W.gen_prefill(1500, 32, 2, 128, seed=32, B=64, needles=4)
    r = prefill_case(d, 64, 1.5, 8.0, 1.0, "bf16", scale=0.05)
    flush(f"  max-abs {r['err']:.2e} flips {r['flips']}")


@pytest.mark.parametrize("Hkv,alphas", [
    (2, [1.25, 1.5, 2.0, 1.5, 1.25, 2.0]),
    (1, [1.25, 1.5, 2.0, 1.5, 1.25, 2.0]),
    (2, [1.5, 1.0, 2.0, 1.25, 1.0, 1.5]),   # softmax routing for two of the sequences
])
def test_prefill_varlen_mixed_alpha(Hkv, alphas):
    flush(f"prefill varlen, G = {32 // Hkv}, alphas {alphas}")
    lens = [1, 63, 64, 65, 700, 1300]
    d = W.gen_varlen(lens, 32, Hkv, 128, seed=41, B=64)
    alphas = np.array(alphas, np.float32)
    cu = d["cu_seqlens"]
    q, qx = to_dev(d["q"], "bf16")
    k, kx = to_dev(d["k"], "bf16")
    v, vx = to_dev(d["v"], "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    cut = torch.from_numpy(cu).cuda()
    out, lse, ab = ops.attn_prefill(q, k, v, qb, 64, alpha=1.5, gamma=25.0, sigma=1.0,
                                    alpha_per_seq=torch.from_numpy(alphas).cuda(),
                                    cu_seqlens=cut, max_seqlen=max(lens), return_lse=True,
                                    return_active_blocks=True)
    kb = ops.summarize(k, qb, 64, cu_seqlens=cut, max_seqlen=max(lens))
    torch.cuda.synchronize()
    S = -(-max(lens) // 64)
    res = O.prefill_varlen(qx, kx, vx, d["qbar"], cu, 64, alphas, 25.0, 1.0, to_bf16=True,
                           num_slots=S)
    kbg = kb.to(torch.float64).cpu().numpy()
    bits = unpack_bits(ab, S)
    o = out.to(torch.float64).cpu().numpy()
    le = lse.cpu().numpy()
    off = 0
    for sidx, r in enumerate(res):
        a, b = int(cu[sidx]), int(cu[sidx + 1])
        C = (b - a) // 64
        G = 32 // Hkv
        check_summaries(kbg[off:off + C], r["kbar"], "bf16", kx[a:b], 64)
        om, margin, _ = oracle_mask_on(qx[a:b], kbg[off:off + C], 64, float(alphas[sidx]),
                                       25.0, 1.0, G, 1 / math.sqrt(128), list(range(b - a)), S)
        compare_masks(bits[:, a:b], om, margin, f"varlen seq {sidx}")
        assert np.max(np.abs(o[a:b] - r["out"])) <= TOL["bf16"]
        assert np.max(np.abs(le[:, a:b] - r["lse"])) <= LSE_TOL["bf16"]
        off += C


def test_prefill_deterministic_and_empty():
    flush("prefill determinism")
    d = W.gen_prefill(700, 32, 2, 128, seed=51)
    q, _ = to_dev(d["q"], "bf16")
    k, _ = to_dev(d["k"], "bf16")
    v, _ = to_dev(d["v"], "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    a = ops.attn_prefill(q, k, v, qb, 64, gamma=30.0, return_lse=True, return_active_blocks=True)
    b = ops.attn_prefill(q, k, v, qb, 64, gamma=30.0, return_lse=True, return_active_blocks=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    e = torch.empty((0, 32, 128), dtype=torch.bfloat16, device="cuda")
    ek = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    out, _, _ = ops.attn_prefill(e, ek, ek, qb, 64, gamma=30.0)
    torch.cuda.synchronize()
    assert out.shape == (0, 32, 128)


# ------------------------------------------------------------------ decode

DECODE_CASES = [
    # name, dtype, batch, cap, seqlens, Hq, Hkv, D, B, alpha, gamma, sigma
    ("g16-b64", "bf16", 3, 1024, [1, 500, 1024], 32, 2, 128, 64, 1.5, 20.0, 1.0),
    ("g4-b128", "bf16", 4, 2048, [129, 128, 2000, 700], 8, 2, 64, 128, 1.25, 15.0, 1.0),
    ("g1-a2", "bf16", 2, 640, [640, 65], 2, 2, 128, 64, 2.0, 20.0, 0.5),
    ("g32", "bf16", 2, 1024, [1024, 777], 32, 1, 128, 64, 1.5, 20.0, 1.0),
    ("f32", "f32", 2, 512, [512, 300], 4, 2, 64, 64, 1.5, 20.0, 1.0),
    ("softmax", "bf16", 2, 512, [512, 200], 32, 2, 128, 64, 1.0, 3.0, 1.0),
    # nearly flat logits: more candidates than the decode solve's short list
    # holds, so it solves on the whole row
    ("flat-a15", "bf16", 2, 16384, [16384, 12000], 32, 2, 128, 64, 1.5, 0.5, 1.0),
    ("flat-a2", "bf16", 2, 16384, [16384, 9000], 16, 1, 128, 64, 2.0, 0.05, 1.0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: c[0])
def test_decode_stage(case):
    name, dtype, batch, cap, sl, Hq, Hkv, D, B, alpha, gamma, sigma = case
    flush(f"decode {name}")
    d = W.gen_decode(batch, cap, Hq, Hkv, D, seed=61)
    kb32 = W.gen_summaries(batch * cap // B, Hkv, D, seed=61).reshape(batch, cap // B, Hkv, D)
    q, qx = to_dev(d["q"], dtype)
    kc, kcx = to_dev(d["k_cache"], dtype)
    vc, vcx = to_dev(d["v_cache"], dtype)
    kb, kbx = to_dev(kb32, dtype)
    seqlens = torch.tensor(sl, dtype=torch.int32, device="cuda")
    gqa = Hq != Hkv
    out, lse, ab = ops.attn_decode(q, kc, vc, seqlens, kb, B, alpha=alpha, gamma=gamma,
                                   sigma=sigma, enable_gqa=gqa, return_lse=True,
                                   return_active_blocks=True)
    torch.cuda.synchronize()
    S = cap // B
    bits = unpack_bits(ab, S)
    o = out.to(torch.float64).cpu().numpy()
    le = lse.cpu().numpy()
    G = Hq // Hkv
    for b in range(batch):
        L = sl[b]
        r = O.decode(qx[b], kcx[b], vcx[b], kbx[b], L, B, alpha, gamma, sigma, gqa)
        n = (L - 1) // B
        qq = np.zeros((L, Hq, D))
        qq[L - 1] = qx[b]
        th = np.full((Hq, L), np.nan)
        th[:, L - 1] = r["tau_hat"]
        margin = O.routing_margin(qq, kbx[b], B, gamma, 1 / math.sqrt(D), G, th, [L - 1], S)
        om = np.zeros((Hkv, 1, S), bool)
        om[:, 0, :n] = r["mask"]
        compare_masks(bits[:, b:b + 1], om, margin, f"decode {name} b={b}")
        err = np.max(np.abs(o[b] - r["out"]))
        assert err <= TOL[dtype], err
        assert np.max(np.abs(le[:, b] - r["lse"])) <= LSE_TOL[dtype]


def test_decode_matches_prefill_last_row():
    flush("decode == prefill last row")
    L, B = 1000, 64
    d = W.gen_prefill(L, 32, 2, 128, seed=71)
    q, _ = to_dev(d["q"], "bf16")
    k, _ = to_dev(d["k"], "bf16")
    v, _ = to_dev(d["v"], "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    pre, plse, pab = ops.attn_prefill(q, k, v, qb, B, gamma=30.0, return_lse=True,
                                      return_active_blocks=True)
    cap = 1024
    kc = torch.zeros((1, cap, 2, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[0, :L] = k
    vc[0, :L] = v
    kbar = ops.summarize(kc.view(cap, 2, 128), qb, B).view(1, cap // B, 2, 128)
    out, lse, ab = ops.attn_decode(q[L - 1:L], kc, vc, torch.tensor([L], dtype=torch.int32,
                                   device="cuda"), kbar, B, gamma=30.0, return_lse=True,
                                   return_active_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(ab[:, 0], pab[:, L - 1])
    err = (out[0].float() - pre[L - 1].float()).abs().max().item()
    assert err <= 1e-2, err
    assert (lse[:, 0] - plse[:, L - 1]).abs().max().item() < 1e-3
