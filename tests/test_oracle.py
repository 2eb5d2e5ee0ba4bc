"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what fixes the expected value: a hand-derived closed form, a
textbook definition solved by a generic optimiser, a brute-force enumeration,
or an independent library routine (torch's scaled_dot_product_attention,
scipy's softmax) on a special case.  A dropped term, a wrong sign, a wrong
index or a transposed operand in the oracle fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.optimize
import scipy.special
import torch
import torch.nn.functional as F

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "entmax_closed_forms.json")))


def sdpa64(q, k, v, mask=None, causal=False, gqa=False):
    """torch SDPA in float64 on the CPU. q [L,Hq,D] -> [L,Hq,D]."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                       enable_gqa=gqa)
    return o[0].numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1, 1e3)])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_bf16(x32.astype(np.float64)), ref)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.0
    assert O.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert O.round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.round_to_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)


# ---------------------------------------------------------------- phase 0

def test_summary_zero_query_is_mean_pooling():
    # q_bar initialised to zero gives uniform mean pooling (Fase 0, Initialisatie)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((200, 2, 16))
    kb = O.summarize(k, np.zeros((2, 16)), 64)
    assert kb.shape == (3, 2, 16)
    for c in range(3):
        np.testing.assert_allclose(kb[c], k[c * 64:(c + 1) * 64].mean(axis=0), atol=1e-14)


def test_summary_is_local_sdpa_of_qbar_over_chunk_keys():
    # local scaled dot-product attention of q_bar over each chunk (torch SDPA)
    rng = np.random.default_rng(2)
    D, B = 32, 16
    k = rng.standard_normal((3 * B + 5, 2, D))
    qbar = rng.standard_normal((2, D))
    kb = O.summarize(k, qbar, B)
    for c in range(3):
        for h in range(2):
            keys = torch.from_numpy(k[c * B:(c + 1) * B, h])[None, None]
            qq = torch.from_numpy(qbar[h])[None, None, None]
            ref = F.scaled_dot_product_attention(qq, keys, keys)[0, 0, 0].numpy()
            np.testing.assert_allclose(kb[c, h], ref, atol=1e-13)


def test_summary_chunk_indexing_and_partial_tail():
    # keys constant per chunk: summary c must be c's constant; tail has none
    B, D = 8, 4
    k = np.zeros((3 * B + 3, 1, D))
    for t in range(k.shape[0]):
        k[t, 0, :] = t // B + 1
    kb = O.summarize(k, np.ones((1, D)), B)
    assert kb.shape[0] == 3
    for c in range(3):
        np.testing.assert_allclose(kb[c, 0], c + 1, atol=1e-14)


def test_summary_permutation_invariant_and_sharp_limit():
    rng = np.random.default_rng(3)
    B, D = 16, 64
    k = rng.standard_normal((B, 1, D))
    qbar = rng.standard_normal((1, D))
    perm = rng.permutation(B)
    np.testing.assert_allclose(O.summarize(k, qbar, B), O.summarize(k[perm], qbar, B), atol=1e-13)
    # q_bar far along key 5 (its own score dominates): summary -> key 5
    t = 5
    big = 1e4 * k[t, 0] / np.linalg.norm(k[t, 0])
    assert np.argmax(k[:, 0] @ big) == t
    np.testing.assert_allclose(O.summarize(k, big[None], B)[0, 0], k[t, 0], atol=1e-9)


def test_summary_bf16_storage_rounds_once():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((128, 1, 32))
    qbar = rng.standard_normal((1, 32)) * 0.1
    exact = O.summarize(k, qbar, 64)
    stored = O.summarize(k, qbar, 64, to_bf16=True)
    assert np.array_equal(stored, O.round_to_bf16(exact))
    # half an ulp of an 8-significant-bit value is at most 2^-8 relative
    assert np.max(np.abs(stored - exact) / np.abs(exact)) <= 2.0 ** -8


# ---------------------------------------------------------------- entmax

@pytest.mark.parametrize("case", GOLD["cases"], ids=lambda c: c["name"])
def test_entmax_hand_derived_closed_forms(case):
    p, tau_hat = O.entmax(np.array(case["u"]), case["alpha"])
    np.testing.assert_allclose(p, case["p"], atol=1e-12)
    assert abs(tau_hat - case["tau_hat"]) < 1e-12


def test_sort_closed_forms_agree_with_bisection():
    rng = np.random.default_rng(5)
    for n in (1, 2, 5, 37, 300):
        for _ in range(5):
            u = rng.standard_normal(n) * rng.uniform(0.1, 30)
            p2, t2 = O.sparsemax_sort(u)
            pb, tb = O.entmax_threshold_bisect(u, 2.0)
            assert abs(t2 - tb) < 1e-12 * max(1, abs(tb))
            np.testing.assert_allclose(p2, pb, atol=1e-12)
            p15, t15 = O.entmax15_sort(u)
            pb, tb = O.entmax_threshold_bisect(u, 1.5)
            assert abs(t15 - tb) < 1e-12 * max(1, abs(tb))
            np.testing.assert_allclose(p15, pb, atol=1e-12)


def _tsallis_argmax(u, alpha):
    """Solve max_{p in simplex} <p,u> + sum(p - p^alpha)/(alpha(alpha-1))
    with a generic constrained optimiser (the textbook definition)."""
    n = len(u)

    def neg(p):
        p = np.clip(p, 0, None)
        return -(p @ u + np.sum(p - p ** alpha) / (alpha * (alpha - 1)))

    res = scipy.optimize.minimize(
        neg, np.full(n, 1.0 / n), method="SLSQP", bounds=[(0, 1)] * n,
        constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
        options=dict(ftol=1e-15, maxiter=1000))
    return np.clip(res.x, 0, None)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 1.75])
def test_entmax_is_the_tsallis_regularised_argmax(alpha):
    rng = np.random.default_rng(6)
    for _ in range(6):
        u = rng.standard_normal(6) * 2
        p, _ = O.entmax(u, alpha)
        ref = _tsallis_argmax(u, alpha)
        np.testing.assert_allclose(p, ref, atol=2e-4)


def _brute_force_support(u, alpha):
    """Enumerate supports S; exactly one admits a threshold t < min_S x with
    sum_S (x_c - t)^(1/(alpha-1)) = 1 and every x_c outside S <= t."""
    x = (alpha - 1) * np.asarray(u, float)
    e = 1 / (alpha - 1)
    n = len(x)
    found = []
    for r in range(1, n + 1):
        for S in itertools.combinations(range(n), r):
            xs = x[list(S)]
            lo_t = xs.min()
            f = lambda t: np.sum((xs - t) ** e) - 1
            if f(lo_t) > 0:       # need the root strictly below min_S x
                continue
            t = scipy.optimize.brentq(f, lo_t - 2.0, lo_t, xtol=1e-15)
            if t >= lo_t:
                continue
            rest = [x[c] for c in range(n) if c not in S]
            if all(xr <= t for xr in rest):
                found.append((set(S), t))
    return found


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_entmax_support_matches_brute_force(alpha):
    rng = np.random.default_rng(7)
    for n in (2, 4, 7):
        for _ in range(8):
            u = rng.standard_normal(n) * rng.uniform(0.5, 6)
            found = _brute_force_support(u, alpha)
            assert len(found) == 1
            S, t = found[0]
            p, tau_hat = O.entmax(u, alpha)
            assert set(np.nonzero(p > 0)[0]) == S
            assert abs(tau_hat * (alpha - 1) - t) < 1e-10


@pytest.mark.parametrize("alpha", [1.0, 1.25, 1.5, 2.0])
def test_batched_rows_equal_single_row_entmax(alpha):
    # the row-batched solver runs the same bisection per row in lockstep
    rng = np.random.default_rng(20)
    n = np.array([0, 1, 2, 7, 30, 30, 13])
    U = rng.standard_normal((len(n), 30)) * 3
    P, th = O.entmax_rows(U, n, alpha)
    for r, nr in enumerate(n):
        p, t = O.entmax(U[r, :nr], alpha)
        np.testing.assert_allclose(P[r, :nr], p, atol=1e-14)
        assert np.all(P[r, nr:] == 0)
        assert t == th[r] or abs(t - th[r]) < 1e-14


def test_entmax_alpha_to_one_is_softmax():
    u = np.array([1.0, 0.5, -1.0])
    sm = scipy.special.softmax(u)
    errs = [np.abs(O.entmax(u, a)[0] - sm).max() for a in (1.1, 1.01, 1.001)]
    assert errs[2] < 5e-4
    assert errs[0] > errs[1] > errs[2]
    # error shrinks about linearly in alpha - 1
    assert 5 < errs[0] / errs[1] < 20 and 5 < errs[1] / errs[2] < 20
    p, tau_hat = O.entmax(u, 1.0)
    np.testing.assert_allclose(p, sm, atol=1e-15)
    assert tau_hat == -math.inf


def test_entmax_invariants():
    rng = np.random.default_rng(8)
    for alpha in (1.25, 1.5, 2.0):
        for n in (1, 3, 50, 400):
            u = rng.standard_normal(n) * 4
            p, tau_hat = O.entmax(u, alpha)
            assert np.all(p >= 0) and abs(p.sum() - 1) < 1e-12
            # KKT: (x_c - tau) = p_c^(alpha-1) on the support, x_c <= tau off it
            x, tau = (alpha - 1) * u, (alpha - 1) * tau_hat
            on = p > 0
            np.testing.assert_allclose(x[on] - tau, p[on] ** (alpha - 1), atol=1e-10)
            assert np.all(x[~on] <= tau + 1e-12)
            # translation invariance
            np.testing.assert_allclose(O.entmax(u + 3.7, alpha)[0], p, atol=1e-10)
        # tiny logits: full support; huge logits: support of one
        u = rng.standard_normal(20)
        assert np.all(O.entmax(1e-6 * u, alpha)[0] > 0)
        assert np.count_nonzero(O.entmax(1e6 * u, alpha)[0]) == 1
    assert O.entmax(np.zeros(0), 1.5)[1] == math.inf


# ---------------------------------------------------------------- phase 1

def test_gqa_average_and_or_mask_golden():
    g = GOLD["gqa_average"]
    heads = np.array(g["heads"])
    # u = gamma * s * <q, kbar>: with kbar_c = u_c e_0, q = e_0, gamma * s = 1
    D = 4
    kb = np.zeros((3, D))
    qg = np.zeros((2, D))
    qg[0, 0], qg[1, 1] = 1.0, 1.0
    kb[:, 0] = heads[0]
    kb[:, 1] = heads[1]
    r = O.route_position(qg, kb, g["alpha"], gamma=2.0, scale=0.5)
    np.testing.assert_allclose(r["u"], heads, atol=1e-15)
    np.testing.assert_allclose(r["wbar"], g["wbar"], atol=1e-12)
    assert list(r["mask"]) == g["mask"]


def test_routing_margin_golden_two_heads():
    # The golden rows as one GQA group of two heads at position 3 with B = 1
    # (chunks 0..2 routable).  u = gamma * s * <q, kbar>: kbar_c = e_c and
    # q_g = u_g / (gamma * s).  With the hand-derived thresholds of the two
    # rows (entmax15_3a, entmax15_3b), the margin of chunk c is
    # min over the heads of |u_gc - tau_hat_g|, worked out here by hand:
    #   head 0: |1 + 0.641941|, |0.5 + 0.641941|, |-1 + 0.641941|
    #   head 1: |-1 + 1.158858|, |0.2 + 1.158858|, |0.3 + 1.158858|
    #   min   : 0.158858 (head 1), 1.141941 (head 0), 0.358059 (head 0)
    cases = {c["name"]: c for c in GOLD["cases"]}
    a, b = cases["entmax15_3a"], cases["entmax15_3b"]
    gamma, s, D, B, L = 2.0, 0.25, 3, 1, 4
    kb = np.zeros((3, 2, D))                 # KV head 1 is a decoy
    kb[:, 0, :] = np.eye(3)
    kb[:, 1, :] = 7.0
    q = np.zeros((L, 4, D))
    q[3, 0] = np.array(a["u"]) / (gamma * s)
    q[3, 1] = np.array(b["u"]) / (gamma * s)
    q[3, 2:] = 5.0
    th = np.full((4, L), np.nan)
    th[0, 3], th[1, 3] = a["tau_hat"], b["tau_hat"]
    th[2:, 3] = 0.0
    mg = O.routing_margin(q, kb, B, gamma, s, 2, th, [3, 1], 5)
    assert mg.shape == (2, 2, 5)
    want = [1.1588584044091477 - 1.0, 0.5 + 0.6419410907075054, 1.0 - 0.6419410907075054]
    np.testing.assert_allclose(mg[0, 0, :3], want, atol=1e-15)
    assert np.all(np.isinf(mg[0, 0, 3:]))      # past the routable range
    assert np.all(np.isinf(mg[:, 1, :]))       # row 1 has no routable chunk
    # heads 2, 3 of KV head 1: u = gamma * s * (3 * 5 * 7) = 0.5 * 105, tau 0
    np.testing.assert_allclose(mg[1, 0, :3], 52.5, atol=1e-12)
    # the thresholds the oracle's own routing finds give the same margins
    _, _, th2 = O.route_sequence(q, kb, B, 1.5, gamma, 1.0, 2, s, rows=[3], num_slots=5)
    np.testing.assert_allclose(O.routing_margin(q, kb, B, gamma, s, 2, th2, [3], 5)[0, 0, :3],
                               want, atol=1e-12)
    # softmax routing thresholds nothing: every margin is infinite
    th[:, 3] = -np.inf
    assert np.all(np.isinf(O.routing_margin(q, kb, B, gamma, s, 2, th, [3], 5)))


def test_summarize_varlen_restarts_the_chunk_grid():
    # Keys constant inside each of a sequence's own chunks (value = 10 * seq +
    # chunk index + head offset), so any summary, whatever q_bar, is that
    # constant; a grid that did not restart at a sequence start would mix two
    # chunks' values.  Sequences: shorter than B (no chunk), exactly B (one
    # chunk), and 2B + 5 (two chunks and a partial tail).
    B, D, Hkv = 8, 4, 2
    lens = [5, 8, 21]
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = np.zeros((cu[-1], Hkv, D))
    expect = []
    for sq, n in enumerate(lens):
        for t in range(n):
            c = t // B
            for h in range(Hkv):
                k[cu[sq] + t, h, :] = 10.0 * sq + c + 100.0 * h
        for c in range(n // B):
            expect.append([[10.0 * sq + c + 100.0 * h] * D for h in range(Hkv)])
    qbar = np.array([[0.3, -1.0, 2.0, 0.5], [1.5, 0.0, -0.7, 0.2]])
    kb = O.summarize_varlen(k, qbar, cu, B)
    np.testing.assert_allclose(kb, np.array(expect), atol=1e-12)
    # mean pooling (q_bar = 0) on ramp keys: chunk c of sequence s averages
    # the packed positions cu[s] + cB ... cu[s] + cB + B - 1
    ramp = np.repeat(np.arange(cu[-1], dtype=float)[:, None, None], Hkv, 1).repeat(D, 2)
    kbm = O.summarize_varlen(ramp, np.zeros((Hkv, D)), cu, B)
    starts = [cu[sq] + c * B for sq, n in enumerate(lens) for c in range(n // B)]
    np.testing.assert_allclose(kbm[:, 0, 0], np.array(starts) + (B - 1) / 2.0, atol=1e-12)
    # bf16 storage rounds each value once
    kbr = O.summarize_varlen(k + 0.001, qbar, cu, B, to_bf16=True)
    np.testing.assert_array_equal(kbr, O.round_to_bf16(np.array(expect) + 0.001))


def test_routing_mask_is_union_of_head_supports():
    rng = np.random.default_rng(9)
    qg = rng.standard_normal((4, 16))
    kb = rng.standard_normal((40, 16))
    r = O.route_position(qg, kb, 1.5, gamma=30.0, scale=0.25)
    union = np.zeros(40, bool)
    for g in range(4):
        union |= O.entmax(r["u"][g], 1.5)[0] > 0
    assert np.array_equal(r["mask"], union)
    assert np.array_equal(r["mask"], r["wbar"] > 0)
    assert 0 < r["mask"].sum() < 40


def test_routable_range_and_head_mapping():
    # Hkv = 2, G = 2: query heads 0,1 -> kv head 0; 2,3 -> kv head 1.
    rng = np.random.default_rng(10)
    B, L, D = 4, 20, 8
    q = rng.standard_normal((L, 4, D))
    kbar = rng.standard_normal((L // B, 2, D))
    kbar[:, 1, :] = 0.0          # kv head 1: all logits zero -> uniform entmax
    mask, logp, tau = O.route_sequence(q, kbar, B, 1.5, 8.0, 1.0, 2, 0.5)
    for i in range(L):
        n = i // B
        assert not mask[:, i, n:].any()
        if n == 0:
            assert np.all(np.isinf(tau[:, i]) & (tau[:, i] > 0))
            continue
        assert mask[1, i, :n].all()
        np.testing.assert_allclose(logp[1, i, :n], math.log(1.0 / n), atol=1e-12)
        assert np.all(tau[2:, i] < 0)          # zero logits: threshold below 0
    # kv head 0 is sparse somewhere (its logits are not flat)
    assert not mask[0, L - 1, :(L - 1) // B].all() or (L - 1) // B == 1


# ------------------------------------------------- estimated diagonal summary

def test_diagonal_estimate_closed_forms():
    rng = np.random.default_rng(24)
    B, L, Hkv, D = 8, 29, 2, 6
    k = rng.standard_normal((L, Hkv, D))
    qb = rng.standard_normal((Hkv, D))
    kd = O.summarize_diagonal(k, qb, B)
    for c in range(-(-L // B)):
        # the first key of a chunk is its own estimate
        np.testing.assert_allclose(kd[c * B], k[c * B], atol=1e-15)
    # at a chunk's last position the estimate is the chunk summary
    full = O.summarize(k, qb, B)
    for c in range(L // B):
        np.testing.assert_allclose(kd[c * B + B - 1], full[c], atol=1e-13)
    # q_bar = 0: the running mean of the chunk's keys so far
    kz = O.summarize_diagonal(k, np.zeros((Hkv, D)), B)
    for i in range(L):
        c0 = (i // B) * B
        np.testing.assert_allclose(kz[i], k[c0:i + 1].sum(axis=0) / (i + 1 - c0), atol=1e-13)
    # a sharp q_bar picks the prefix key of largest <q_bar, k>
    ks = O.summarize_diagonal(k, 1e4 * qb, B)
    for i in (3, 12, 28):
        c0 = (i // B) * B
        for h in range(Hkv):
            j = c0 + int(np.argmax(k[c0:i + 1, h] @ qb[h]))
            np.testing.assert_allclose(ks[i, h], k[j, h], atol=1e-9)


def test_diagonal_entry_shares_the_entmax_mass():
    # sparsemax, one head, routed logits (0, 0) and a diagonal logit 0:
    # p = (1/3, 1/3, 1/3); without the diagonal entry p = (1/2, 1/2)
    D = 4
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    kb = np.zeros((2, D))
    r = O.route_position(q, kb, 2.0, gamma=1.0, scale=1.0, kdiag_h=np.zeros(D))
    np.testing.assert_allclose(r["wbar"], [1 / 3, 1 / 3], atol=1e-12)
    np.testing.assert_allclose(r["p_diag"], [1 / 3], atol=1e-12)
    r0 = O.route_position(q, kb, 2.0, gamma=1.0, scale=1.0)
    np.testing.assert_allclose(r0["wbar"], [0.5, 0.5], atol=1e-12)
    # a diagonal logit 1 above the others takes all of the sparsemax mass
    kd = np.zeros(D)
    kd[0] = 1.0
    r1 = O.route_position(q, kb, 2.0, gamma=1.0, scale=1.0, kdiag_h=kd)
    assert not r1["mask"].any()
    np.testing.assert_allclose(r1["p_diag"], [1.0], atol=1e-12)


def test_diagonal_entry_below_the_support_changes_nothing():
    # a diagonal estimate with a far negative logit stays outside every
    # head's support: mask, prior and threshold equal plain routing
    rng = np.random.default_rng(25)
    B, L, D, G = 4, 40, 8, 2
    q = rng.standard_normal((L, 2 * G, D))
    kbar = rng.standard_normal((L // B, 2, D))
    kd = np.zeros((L, 2, D))
    for i in range(L):
        for h in range(2):
            kd[i, h] = -50.0 * q[i, h * G:(h + 1) * G].sum(axis=0)
    for alpha in (1.5, 2.0, 1.25):
        m0, l0, t0 = O.route_sequence(q, kbar, B, alpha, 3.0, 1.0, G, 0.5)
        m1, l1, t1 = O.route_sequence(q, kbar, B, alpha, 3.0, 1.0, G, 0.5, kdiag=kd)
        assert np.array_equal(m0, m1)
        np.testing.assert_allclose(l1[m1], l0[m0], atol=1e-9)
        np.testing.assert_allclose(t1, t0, atol=1e-9)


def test_diagonal_entry_sequence_matches_single_positions():
    rng = np.random.default_rng(26)
    B, L, D, G = 4, 36, 8, 2
    q = rng.standard_normal((L, 2 * G, D))
    kbar = rng.standard_normal((L // B, 2, D))
    kd = rng.standard_normal((L, 2, D))
    mask, logp, tau = O.route_sequence(q, kbar, B, 1.5, 4.0, 0.7, G, 0.5, kdiag=kd)
    for i in (4, 9, 17, 35):
        n = i // B
        for h in range(2):
            r = O.route_position(q[i, h * G:(h + 1) * G], kbar[:n, h], 1.5, 4.0, 0.5,
                                 kdiag_h=kd[i, h])
            assert np.array_equal(mask[h, i, :n], r["mask"])
            np.testing.assert_allclose(logp[h, i, :n][r["mask"]],
                                       0.7 * np.log(r["wbar"][r["mask"]]), atol=1e-10)
            np.testing.assert_allclose(tau[h * G:(h + 1) * G, i], r["tau_hat"], atol=1e-10)
            # the routed chunks and the diagonal share each head's unit mass
            np.testing.assert_allclose(r["p"].sum(axis=1) + r["p_diag"], 1.0, atol=1e-12)


# ------------------------------------------------- top-k comparison routing

def _topk_by_hand():
    # kv head 0 with G = 2; q_g = e_g and gamma * s = 1 make u_g[c] = kbar[c, g].
    # head 0: u = (ln 8, 0, 0)   -> softmax (8/10, 1/10, 1/10)
    # head 1: u = (0, ln 2, ln 2) -> softmax (1/5, 2/5, 2/5)
    # group score S = (1, 1/2, 1/2): chunks 1 and 2 tie.
    B, L, D = 1, 4, 4
    q = np.zeros((L, 2, D))
    q[:, 0, 0], q[:, 1, 1] = 1.0, 1.0
    kb = np.zeros((L, 1, D))
    kb[:3, 0, 0] = (math.log(8.0), 0.0, 0.0)
    kb[:3, 0, 1] = (0.0, math.log(2.0), math.log(2.0))
    return q, kb, B


def test_topk_scores_and_selection_by_hand():
    q, kb, B = _topk_by_hand()
    for k, want in ((1, [0]), (2, [0, 1]), (3, [0, 1, 2]), (9, [0, 1, 2])):
        mask, logp, score = O.route_topk_sequence(q, kb, B, k, gamma=2.0, G=2,
                                                  scale=0.5, rows=[3])
        np.testing.assert_allclose(score[0, 3, :3], [1.0, 0.5, 0.5], atol=1e-15)
        assert np.flatnonzero(mask[0, 3]).tolist() == want   # tie -> lower index
        assert np.all(logp[0, 3, want] == 0.0)
        assert np.all(np.isneginf(np.delete(logp[0, 3], want)))
        assert np.isnan(score[0, 3, 3])                     # diagonal chunk


def test_topk_single_head_is_topk_of_logits():
    # G = 1: softmax is monotone, so the k largest scores are the k largest
    # logits; enumerate the k-subsets and keep the one of largest logit sum.
    rng = np.random.default_rng(21)
    B, L, D, k = 2, 16, 6, 3
    q = rng.standard_normal((L, 1, D))
    kb = rng.standard_normal((L // B, 1, D))
    mask, _, _ = O.route_topk_sequence(q, kb, B, k, gamma=3.0, G=1, scale=0.4)
    for i in range(L):
        n = i // B
        u = [0.4 * 3.0 * float(q[i, 0] @ kb[c, 0]) for c in range(n)]
        if n <= k:
            assert mask[0, i].tolist() == [c < n for c in range(L // B)]
            continue
        best = max(itertools.combinations(range(n), k), key=lambda t: sum(u[c] for c in t))
        assert np.flatnonzero(mask[0, i]).tolist() == list(best)


def test_topk_invariants():
    rng = np.random.default_rng(22)
    B, L, D, G, k = 4, 64, 8, 4, 5
    q = rng.standard_normal((L, 2 * G, D))
    kb = rng.standard_normal((L // B, 2, D))
    # zero summaries on kv head 1 give equal scores: the lowest indices win
    kb[:, 1, :] = 0.0
    mask, logp, score = O.route_topk_sequence(q, kb, B, k, gamma=5.0, G=G, scale=0.3)
    for h in range(2):
        for i in range(L):
            n = i // B
            sel = mask[h, i]
            assert not sel[n:].any()
            assert sel.sum() == min(k, n)
            if n == 0:
                continue
            np.testing.assert_allclose(score[h, i, :n].sum(), G, atol=1e-12)
            s = score[h, i, :n]
            if sel[:n].all():
                continue
            assert s[sel[:n]].min() >= s[~sel[:n]].max()
            if h == 1:
                assert np.flatnonzero(sel).tolist() == list(range(min(k, n)))


def test_topk_covering_all_chunks_equals_softmax_routing():
    # k >= n: every routable chunk is active, as under alpha = 1 routing
    rng = np.random.default_rng(23)
    B, L, D = 4, 32, 8
    q = rng.standard_normal((L, 4, D))
    kb = rng.standard_normal((L // B, 2, D))
    m1, lp1, _ = O.route_topk_sequence(q, kb, B, L, gamma=4.0, G=2, scale=0.3)
    m2, _, _ = O.route_sequence(q, kb, B, 1.0, 4.0, 0.0, 2, 0.3)
    assert np.array_equal(m1, m2)
    assert np.all(lp1[m1] == 0.0)


# ---------------------------------------------------------------- phase 2

def _tiny(seed, L=40, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((L, Hq, D)), rng.standard_normal((L, Hkv, D)),
            rng.standard_normal((L, Hkv, D)), rng.standard_normal((Hkv, D)) * 0.3)


def test_dense_form_equals_row_sparse_form():
    q, k, v, qb = _tiny(11)
    for alpha, sigma in ((1.5, 1.0), (2.0, 0.5), (1.25, 2.0), (1.0, 1.0)):
        rs = O.prefill(q, k, v, qb, 8, alpha, 6.0, sigma)
        dn = O.prefill(q, k, v, qb, 8, alpha, 6.0, sigma, dense=True)
        np.testing.assert_allclose(rs["out"], dn["out"], atol=1e-12)
        np.testing.assert_allclose(rs["lse"], dn["lse"], atol=1e-12)


def test_all_active_sigma0_is_dense_causal_attention():
    # alpha = 1 activates every chunk; sigma = 0 makes the prior uniform
    q, k, v, qb = _tiny(12)
    r = O.prefill(q, k, v, qb, 8, 1.0, 3.0, 0.0)
    ref = sdpa64(q, k, v, causal=True, gqa=True)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12)


def test_short_sequence_is_plain_causal_attention():
    q, k, v, qb = _tiny(13, L=16)
    r = O.prefill(q, k, v, qb, 16, 1.5, 50.0, 1.0)
    np.testing.assert_allclose(r["out"], sdpa64(q, k, v, causal=True, gqa=True), atol=1e-12)


def test_softmax_routing_prior_is_log_probability_bias():
    # alpha = 1, sigma = 1, G = 1: bias of chunk c is log softmax_c(u); build
    # the additive mask with torch ops and compare to torch SDPA
    rng = np.random.default_rng(14)
    L, B, D = 24, 4, 8
    q = rng.standard_normal((L, 1, D))
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    qb = rng.standard_normal((1, D))
    gamma, s = 5.0, 1 / math.sqrt(D)
    r = O.prefill(q, k, v, qb, B, 1.0, gamma, 1.0)
    kbar = torch.from_numpy(O.summarize(k, qb, B)[:, 0])      # [C, D]
    tq = torch.from_numpy(q[:, 0])
    mask = torch.full((L, L), -math.inf, dtype=torch.float64)
    for i in range(L):
        n = i // B
        if n:
            logw = torch.log_softmax(gamma * s * (kbar[:n] @ tq[i]), 0)
            mask[i, :n * B] = torch.repeat_interleave(logw, B)
        mask[i, n * B:i + 1] = 0.0
    ref = sdpa64(q, k, v, mask=mask.numpy())
    np.testing.assert_allclose(r["out"], ref, atol=1e-12)


def test_single_selected_chunk_attends_that_chunk_and_diagonal():
    # every head of the group routes to chunk 2 only: w_bar = 1, bias = 0
    rng = np.random.default_rng(15)
    L, B, D, G = 48, 8, 16, 2
    q = rng.standard_normal((L, G, D))
    k = rng.standard_normal((L, 1, D)) * 0.1
    v = rng.standard_normal((L, 1, D))
    d = np.zeros(D)
    d[0] = 1.0
    q[:, :, 0] = 5.0
    k[2 * B:3 * B, 0, :] += 40.0 * d          # summary of chunk 2 ~ 40 e_0
    r = O.prefill(q, k, v, np.zeros((1, D)), B, 1.5, 1.0, 1.0)
    i = L - 1
    assert list(np.nonzero(r["mask"][0, i])[0]) == [2]
    idx = list(range(2 * B, 3 * B)) + list(range((i // B) * B, i + 1))
    ref = sdpa64(q[i:i + 1], k[idx], v[idx], gqa=True)
    np.testing.assert_allclose(r["out"][i], ref[0], atol=1e-12)


def test_sigma0_is_block_sparse_attention_on_the_support():
    q, k, v, qb = _tiny(16)
    B = 8
    r = O.prefill(q, k, v, qb, B, 1.5, 8.0, 0.0)
    L = q.shape[0]
    for h in range(2):
        allowed = np.zeros((L, L), bool)
        for i in range(L):
            for c in range(i // B):
                allowed[i, c * B:(c + 1) * B] = r["mask"][h, i, c]
            allowed[i, (i // B) * B:i + 1] = True
        m = np.where(allowed, 0.0, -np.inf)
        ref = sdpa64(q[:, 2 * h:2 * h + 2], k[:, h:h + 1], v[:, h:h + 1], mask=m, gqa=True)
        np.testing.assert_allclose(r["out"][:, 2 * h:2 * h + 2], ref, atol=1e-12)


def test_prior_induced_softmax_is_the_kl_regularised_argmax():
    # Fase 2: softmax maximises z.p - KL(p||u); DashAttention swaps u for g.
    # Solve max z.p - KL(p||g) numerically with g = w_bar^sigma (diagonal 1)
    # and check that the oracle's attention weights are that maximiser.
    rng = np.random.default_rng(17)
    L, B, D = 20, 4, 8
    q = rng.standard_normal((L, 1, D))
    k = rng.standard_normal((L, 1, D))
    v = np.eye(L)[:, None, :]                  # v = one-hot: out = weights
    qb = rng.standard_normal((1, D))
    sigma, gamma = 0.7, 6.0
    # pad q, k, q_bar with zero dims up to L so that v can be the L x L
    # identity (out = attention weights); scores and summaries are unchanged
    # because the attention scale is passed explicitly and the padding is 0
    kk = np.concatenate([k, np.zeros((L, 1, L - D))], axis=2)
    qq = np.concatenate([q, np.zeros((L, 1, L - D))], axis=2)
    qbp = np.concatenate([qb, np.zeros((1, L - D))], 1)
    s = 1 / math.sqrt(D)
    r = O.prefill(qq, kk, v, qbp, B, 1.5, gamma, sigma, scale=s)
    i = L - 1
    route = O.route_position(qq[i], O.summarize(kk, qbp, B)[: i // B, 0], 1.5,
                             gamma, s)
    g = np.zeros(L)
    for c in range(i // B):
        g[c * B:(c + 1) * B] = route["wbar"][c] ** sigma
    g[(i // B) * B:i + 1] = 1.0
    z = (k[:, 0] @ q[i, 0]) / math.sqrt(D)
    on = g > 0

    def neg(p):
        p = np.clip(p, 1e-300, None)
        return -(p @ z[on] - np.sum(p * (np.log(p) - np.log(g[on]))))

    n = int(on.sum())
    res = scipy.optimize.minimize(neg, np.full(n, 1.0 / n), method="SLSQP",
                                  bounds=[(0, 1)] * n,
                                  constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
                                  options=dict(ftol=1e-14, maxiter=2000))
    w = r["out"][i, 0]
    assert np.all(w[~on] == 0)
    np.testing.assert_allclose(w[on], res.x, atol=2e-4)


def test_decode_equals_last_prefill_row():
    q, k, v, qb = _tiny(18, L=43)
    B = 8
    pre = O.prefill(q, k, v, qb, B, 1.5, 7.0, 1.0)
    kbar = O.summarize(k, qb, B)
    for L in (43, 40, 33, 9, 5):
        dec = O.decode(q[L - 1], k, v, kbar, L, B, 1.5, 7.0, 1.0)
        sub = O.prefill(q[:L], k[:L], v[:L], qb, B, 1.5, 7.0, 1.0, rows=[L - 1])
        np.testing.assert_allclose(dec["out"], sub["out"][0], atol=1e-12)
        np.testing.assert_allclose(dec["lse"], sub["lse"][:, 0], atol=1e-12)
    np.testing.assert_allclose(O.decode(q[42], k, v, kbar, 43, B, 1.5, 7.0, 1.0)["out"],
                               pre["out"][42], atol=1e-12)


def test_varlen_is_independent_sequences():
    rng = np.random.default_rng(19)
    lens = [13, 30, 21]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q = rng.standard_normal((T, 2, 8))
    k = rng.standard_normal((T, 1, 8))
    v = rng.standard_normal((T, 1, 8))
    qb = rng.standard_normal((1, 8))
    res = O.prefill_varlen(q, k, v, qb, cu, 4, [1.25, 1.5, 2.0], 5.0, 1.0)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        one = O.prefill(q[a:b], k[a:b], v[a:b], qb, 4, [1.25, 1.5, 2.0][s], 5.0, 1.0)
        np.testing.assert_allclose(res[s]["out"], one["out"], atol=0)
    kb = O.summarize_varlen(k, qb, cu, 4)
    assert kb.shape[0] == sum(n // 4 for n in lens)
