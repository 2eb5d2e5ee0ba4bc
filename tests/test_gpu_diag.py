"""GPU parity of the estimate_diagonal option against the CPU oracle.

The own-chunk estimates (dash_summarize_diagonal) are checked like summaries
(fp32 accumulation plus one rounding); routing with them is checked on the
GPU's own estimates (masks identical outside the threshold band, priors and
thresholds within tolerance); prefill and decode end to end to the output
tolerances.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_hierarchical_attention_dash_amd import ops
from sparse_hierarchical_attention_dash_amd import workloads as W

from gpu_helpers import (BAND, LSE_TOL, TOL, check_summaries, compare_masks, flush, to_dev,
                         unpack_bits)

pytestmark = pytest.mark.gpu


def _diag_bound_check(kd_gpu, kd_ora, dtype, k, B):
    """check_summaries on per-position estimates: the bound of a summary over
    at most B keys holds for every prefix of a chunk."""
    L = kd_gpu.shape[0]
    Lp = -(-L // B) * B
    kk = np.zeros((Lp,) + k.shape[1:])
    kk[:L] = k
    rows = np.arange(L)
    # a per-row bound: use the full chunk's key magnitude for every row of it
    chunk_max = np.abs(kk).reshape(Lp // B, B, *k.shape[1:]).max(axis=1)   # [C, Hkv, D]
    fp = (B * 2.0 ** -24 + 1e-6) * chunk_max[rows // B]
    d = np.abs(kd_gpu - kd_ora)
    if dtype == "f32":
        assert np.all(d <= fp + 1e-5 * np.abs(kd_ora)), float(np.max(d))
        return
    ulp = np.abs(kd_ora) * 2.0 ** -7 + 2 * fp
    assert np.all(d <= ulp), float(np.max(d / ulp))
    assert float(np.mean(d > 0)) < 1e-3


@pytest.mark.parametrize("dtype,D,B,L", [("bf16", 128, 64, 1000), ("bf16", 64, 128, 777),
                                         ("f32", 64, 64, 300), ("f32", 128, 128, 260)])
def test_summarize_diagonal(dtype, D, B, L):
    flush(f"diagonal estimates {dtype} D={D} B={B} L={L}")
    d = W.gen_prefill(L, 4, 2, D, seed=51)
    k, kx = to_dev(d["k"], dtype)
    qb = torch.from_numpy(d["qbar"]).cuda()
    kd = ops.summarize_diagonal(k, qb, B)
    torch.cuda.synchronize()
    ora = O.summarize_diagonal(kx, d["qbar"].astype(np.float64), B, to_bf16=(dtype == "bf16"))
    _diag_bound_check(kd.to(torch.float64).cpu().numpy(), ora, dtype, kx, B)


def test_summarize_diagonal_varlen():
    flush("diagonal estimates varlen")
    lens = [130, 64, 1, 200]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = W.gen_prefill(int(cu[-1]), 4, 2, 128, seed=52)
    k, kx = to_dev(d["k"], "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    kd = ops.summarize_diagonal(k, qb, 64, cu_seqlens=torch.from_numpy(cu).cuda(),
                                max_seqlen=max(lens))
    torch.cuda.synchronize()
    g = kd.to(torch.float64).cpu().numpy()
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        ora = O.summarize_diagonal(kx[a:b], d["qbar"].astype(np.float64), 64, to_bf16=True)
        _diag_bound_check(g[a:b], ora, "bf16", kx[a:b], 64)


ROUTE_CASES = [
    # name, dtype, L, Hq, Hkv, D, B, alpha, gamma, sigma
    ("g16-a15", "bf16", 1000, 32, 2, 128, 64, 1.5, 30.0, 1.0),
    ("g4-a2-b128", "bf16", 900, 8, 2, 64, 128, 2.0, 40.0, 1.0),
    ("g2-a125-f32", "f32", 777, 4, 2, 64, 64, 1.25, 25.0, 0.5),
    ("g1-a1", "bf16", 700, 2, 2, 128, 64, 1.0, 5.0, 1.0),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: c[0])
def test_route_with_diagonal_estimate(case):
    name, dtype, L, Hq, Hkv, D, B, alpha, gamma, sigma = case
    flush(f"route + diagonal {name}")
    d = W.gen_prefill(L, Hq, Hkv, D, seed=53)
    q, qx = to_dev(d["q"], dtype)
    k, kx = to_dev(d["k"], dtype)
    qb = torch.from_numpy(d["qbar"]).cuda()
    kb = ops.summarize(k, qb, B)
    kd = ops.summarize_diagonal(k, qb, B)
    gqa = Hq != Hkv
    mask, lp, tau = ops.route(q, kb, Hkv, B, alpha=alpha, gamma=gamma, sigma=sigma,
                              enable_gqa=gqa, log_prior=True, tau=True, kdiag=kd)
    m0, _, _ = ops.route(q, kb, Hkv, B, alpha=alpha, gamma=gamma, sigma=sigma, enable_gqa=gqa)
    torch.cuda.synchronize()
    S = -(-L // B)
    G = Hq // Hkv
    s = 1.0 / math.sqrt(D)
    kbx = kb.to(torch.float64).cpu().numpy()
    kdx = kd.to(torch.float64).cpu().numpy()
    rows = list(range(L))
    om, olp, oth = O.route_sequence(qx, kbx, B, alpha, gamma, sigma, G, s, rows=rows,
                                    num_slots=S, kdiag=kdx)
    margin = O.routing_margin(qx, kbx, B, gamma, s, G, oth, rows, S)
    bits = unpack_bits(mask, S)
    flips = compare_masks(bits, om, margin, f"route+diag {name}")
    th = tau.cpu().numpy().astype(np.float64)
    fin = np.isfinite(oth)
    assert np.array_equal(np.isfinite(th), fin)
    assert np.max(np.abs(th[fin] - oth[fin]), initial=0.0) < BAND
    both = bits & om
    g = lp.cpu().numpy().astype(np.float64)
    if sigma > 0:
        assert np.max(np.abs(np.exp(g[both] / sigma) - np.exp(olp[both] / sigma)),
                      initial=0.0) < 2e-5
    # the estimate takes mass: no chunk becomes active that plain routing
    # leaves out (alpha > 1), up to decisions at the threshold itself
    if alpha > 1.0:
        plain = unpack_bits(m0, S)
        assert (bits & ~plain).sum() <= max(2, flips)
    flush(f"  route+diag {name}: flips in band {flips}")


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B,L", [("bf16", 32, 2, 128, 64, 1000),
                                                ("bf16", 8, 2, 64, 128, 700),
                                                ("f32", 4, 2, 64, 64, 400)])
def test_prefill_with_diagonal_estimate(dtype, Hq, Hkv, D, B, L):
    # the fused call against the oracle's phases 1-2 on the GPU's phase-0
    # outputs (summaries and own-chunk estimates, each checked on its own)
    flush(f"prefill + diagonal {dtype} {Hq}/{Hkv} D={D} B={B} L={L}")
    alpha, gamma, sigma = 1.5, 30.0, 1.0
    d = W.gen_prefill(L, Hq, Hkv, D, seed=54)
    q, qx = to_dev(d["q"], dtype)
    k, kx = to_dev(d["k"], dtype)
    v, vx = to_dev(d["v"], dtype)
    qb = torch.from_numpy(d["qbar"]).cuda()
    out, lse, ab = ops.attn_prefill(q, k, v, qb, B, alpha=alpha, gamma=gamma, sigma=sigma,
                                    return_lse=True, return_active_blocks=True,
                                    estimate_diagonal=True)
    kb = ops.summarize(k, qb, B)
    kd = ops.summarize_diagonal(k, qb, B)
    torch.cuda.synchronize()
    S = -(-L // B)
    G = Hq // Hkv
    s = 1.0 / math.sqrt(D)
    kbx = kb.to(torch.float64).cpu().numpy()
    kdx = kd.to(torch.float64).cpu().numpy()
    rows = sorted(set(np.random.default_rng(5).integers(0, L, 120).tolist()) |
                  {L - 1, B, 2 * B - 1})
    om, olp, oth = O.route_sequence(qx, kbx, B, alpha, gamma, sigma, G, s, rows=rows,
                                    num_slots=S, kdiag=kdx)
    margin = O.routing_margin(qx, kbx, B, gamma, s, G, oth, rows, S)
    bits = unpack_bits(ab, S)[:, rows]
    compare_masks(bits, om[:, rows], margin, "prefill+diag")
    # attention on the GPU's own routing (its bits, the oracle's prior there)
    mfull = np.zeros((Hkv, L, S), bool)
    mfull[:, rows] = bits
    lfull = np.full((Hkv, L, S), -np.inf)
    lfull[:, rows] = np.where(bits, olp[:, rows], -np.inf)
    o_ref, l_ref = O.attention_rows(qx, kx, vx, mfull, lfull, B, s, G, rows)
    o = out.to(torch.float64).cpu().numpy()[rows]
    err = float(np.max(np.abs(o - o_ref)))
    assert err <= TOL[dtype], err
    le = lse.cpu().numpy().astype(np.float64)[:, rows]
    assert float(np.max(np.abs(le - l_ref))) <= LSE_TOL[dtype]


def test_decode_with_diagonal_estimate():
    flush("decode + diagonal")
    B, cap, Hq, Hkv, D = 64, 1024, 32, 2, 128
    alpha, gamma, sigma = 1.5, 20.0, 1.0
    sl = [1000, 640, 65]
    batch = len(sl)
    d = W.gen_decode(batch, cap, Hq, Hkv, D, seed=55)
    q, qx = to_dev(d["q"], "bf16")
    kc, kcx = to_dev(d["k_cache"], "bf16")
    vc, vcx = to_dev(d["v_cache"], "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    kb = ops.summarize(kc.view(batch * cap, Hkv, D), qb, B).view(batch, cap // B, Hkv, D)
    seqlens = torch.tensor(sl, dtype=torch.int32, device="cuda")
    out, lse, ab = ops.attn_decode(q, kc, vc, seqlens, kb, B, alpha=alpha, gamma=gamma,
                                   sigma=sigma, return_lse=True, return_active_blocks=True,
                                   estimate_diagonal=True, qbar=qb)
    # the new rows' estimates as dash_summarize_diagonal gives them
    kds = []
    for b in range(batch):
        n = (sl[b] - 1) // B
        kds.append(ops.summarize_diagonal(kc[b, n * B:sl[b]].contiguous(), qb, B)[-1])
    torch.cuda.synchronize()
    S = cap // B
    bits = unpack_bits(ab, S)
    kbx = kb.to(torch.float64).cpu().numpy()
    o = out.to(torch.float64).cpu().numpy()
    le = lse.cpu().numpy()
    G = Hq // Hkv
    for b in range(batch):
        L = sl[b]
        n = (L - 1) // B
        kd = kds[b].to(torch.float64).cpu().numpy()
        r = O.decode(qx[b], kcx[b], vcx[b], kbx[b], L, B, alpha, gamma, sigma, True, kdiag=kd)
        qq = np.zeros((L, Hq, D))
        qq[L - 1] = qx[b]
        th = np.full((Hq, L), np.nan)
        th[:, L - 1] = r["tau_hat"]
        margin = O.routing_margin(qq, kbx[b], B, gamma, 1 / math.sqrt(D), G, th, [L - 1], S)
        om = np.zeros((Hkv, 1, S), bool)
        om[:, 0, :n] = r["mask"]
        flips = compare_masks(bits[:, b:b + 1], om, margin, f"decode+diag b={b}")
        if flips == 0:
            assert np.max(np.abs(o[b] - r["out"])) <= TOL["bf16"]
            assert np.max(np.abs(le[:, b] - r["lse"])) <= LSE_TOL["bf16"]
