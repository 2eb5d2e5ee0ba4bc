"""DashAttention forward pass, written out plainly in float64 NumPy.

TEST INFRASTRUCTURE ONLY.  This module is the oracle that the HIP library is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It imports nothing from
the HIP package, and the HIP package imports nothing from here.

Sources (the pages are cited by title and section, never by line):

* [NL] "Technische Samenvatting: DashAttention", gist.science/nl/paper/2605.18753,
  sections "Fase 0: Lokale Chunk Samenvatting", "Fase 1: Entmax Chunk
  Routering" (equation  w_hat = alpha-entmax(gamma * z_bar)) and
  "Fase 2: Prior-Geinduceerde Spaarzame Softmax".
* [ZH] "技术摘要：DashAttention", gist.science/zh/paper/2605.18753, sections
  阶段 0 / 阶段 1 / 阶段 2 (the same three phases, same equation).
* [ES] aiexpert.news article "DashAttention alcanza 75% de dispersidad ...",
  the interface paragraph (q, k, v, head_cls, chunk_size, enable_gqa,
  optional active_blocks) and the method paragraph (exact zeros below an
  adaptive per-query threshold).
* alpha-entmax itself is not printed by the pages.  It is the textbook
  Tsallis transformation of Peters, Niculae & Martins (2019), "Sparse
  Sequence-to-Sequence Models"; alpha = 2 is sparsemax of Martins & Astudillo
  (2016), "From Softmax to Sparsemax".

Readings taken where the pages are silent (each one is listed in the design doc):

* Phase-0 "local scaled dot-product attention" uses scale 1/sqrt(D) and the
  chunk's keys as its values, so a summary lives in key space and q_bar = 0
  gives the plain mean of the chunk's keys ([NL] Fase 0, "Initialisatie").
* Only complete chunks get a summary; a query at position i may route to
  chunks c < floor(i / B).  Its own chunk is the diagonal branch, attended
  causally with prior weight 1 (bias 0) ([NL] Fase 2, "Diagonaal Afhandeling").
* Routing logits are u = gamma * s * <q, k_bar>, s the attention scale.
* The prior is g = w_bar ** sigma on routed chunks, with g = 0 wherever
  w_bar = 0 (so the bias is sigma * log(w_bar), and -inf off the support,
  also when sigma = 0) ([NL] Fase 2, "Dynamische Maskering" and the sigma
  sentence of "Diagonaal Afhandeling").  The pages fix g only through these
  properties (its support, sigma as its strength, a uniform prior at
  sigma = 0), so the power form is a reading.  This function's computation of
  it is pinned in the tests: at sigma = 0.7 the attention equals a numerical
  solution of the KL-regularised argmax the pages describe, with prior g; at
  sigma = 1 with softmax routing the bias is the routing's log-probability;
  at sigma = 0 the result is plain block-sparse attention on the support.
* Under GQA the routing probabilities of the query heads sharing a KV head
  are averaged ([NL] Fase 1, "GQA-afhandeling"); query head q uses KV head
  floor(q / G).  A chunk is active iff some head gives it a non-zero
  probability, i.e. iff u > tau_hat for that head.
* alpha = 1 is plain softmax routing: every routable chunk is active.
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# small helpers
# ---------------------------------------------------------------------------

def round_to_bf16(x):
    """Round to the nearest bfloat16 value (8 significant bits), ties to even.

    bfloat16 keeps the float32 exponent range and 8 significant bits.  With
    x = m * 2**e and 0.5 <= |m| < 1, the nearest such value is
    rint(m * 256) * 2**(e - 8); ``np.rint`` rounds halves to even.
    """
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def softmax(a):
    """Numerically stable softmax of a 1-D array."""
    a = np.asarray(a, dtype=F64)
    z = np.exp(a - a.max())
    return z / z.sum()


def _default_scale(D, scale):
    return 1.0 / math.sqrt(D) if (scale is None or scale <= 0) else float(scale)


# ---------------------------------------------------------------------------
# Phase 0: chunk summaries  ([NL] / [ZH] Fase 0 / 阶段 0)
# ---------------------------------------------------------------------------

def summarize(k, qbar, B, to_bf16=False):
    """Summaries of the complete size-B chunks of one sequence.

    k     : [L, Hkv, D] keys of one sequence
    qbar  : [Hkv, D] learned summary query, one per KV head
    returns k_bar [L // B, Hkv, D].

    A learned query q_bar attends to the keys of each chunk with local scaled
    dot-product attention; the chunk's keys serve as the values.  With
    q_bar = 0 the weights are uniform and the summary is the mean key.  When
    the keys are stored in bfloat16 the summary is stored in bfloat16 too
    (rounded to nearest even), since it is cached like a key.
    """
    k = np.asarray(k, dtype=F64)
    qbar = np.asarray(qbar, dtype=F64)
    L, Hkv, D = k.shape
    C = L // B
    s = 1.0 / math.sqrt(D)
    kbar = np.zeros((C, Hkv, D), dtype=F64)
    for c in range(C):
        for h in range(Hkv):
            keys = k[c * B:(c + 1) * B, h, :]           # [B, D]
            scores = s * (keys @ qbar[h])                # [B]
            weights = softmax(scores)
            kbar[c, h] = weights @ keys
    return round_to_bf16(kbar) if to_bf16 else kbar


def summarize_varlen(k, qbar, cu_seqlens, B, to_bf16=False):
    """Packed summaries: each sequence's chunk grid restarts at its start.

    Returns k_bar [sum_s floor(L_s / B), Hkv, D], sequences in order.
    """
    parts = []
    for s in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        parts.append(summarize(k[a:b], qbar, B, to_bf16))
    return np.concatenate(parts, axis=0)


def summarize_diagonal(k, qbar, B, to_bf16=False):
    """Estimated summary of every position's own, partial, chunk.

    The interface carries an ``estimate_diagonal`` flag for a diagonal
    correction of the alpha-entmax normalisation ([ES] aiexpert.news, the
    interface paragraph); the pages say no more.  Reading taken here: the
    chunk that holds position i has no summary yet, so it gets an estimate,
    the same phase-0 attention of q_bar restricted to the keys of that chunk
    at or before i (keys cB .. i, c = floor(i / B)).  At i = cB the estimate
    is k_i itself; at the chunk's last position it is the chunk's summary.

    k [L, Hkv, D], qbar [Hkv, D] -> [L, Hkv, D] (rounded like a summary).
    """
    k = np.asarray(k, dtype=F64)
    qbar = np.asarray(qbar, dtype=F64)
    L, Hkv, D = k.shape
    s = 1.0 / math.sqrt(D)
    out = np.zeros((L, Hkv, D), dtype=F64)
    for i in range(L):
        c0 = (i // B) * B
        for h in range(Hkv):
            keys = k[c0:i + 1, h, :]
            weights = softmax(s * (keys @ qbar[h]))
            out[i, h] = weights @ keys
    return round_to_bf16(out) if to_bf16 else out


# ---------------------------------------------------------------------------
# Phase 1: alpha-entmax routing  ([NL] / [ZH] Fase 1 / 阶段 1)
# ---------------------------------------------------------------------------

def routing_logits(q_vec, kbar_h, gamma, scale):
    """u_c = gamma * s * <q, k_bar_c> for the routable chunks c."""
    q_vec = np.asarray(q_vec, dtype=F64)
    kbar_h = np.asarray(kbar_h, dtype=F64)
    return gamma * scale * (kbar_h @ q_vec)


def entmax_threshold_bisect(u, alpha):
    """alpha-entmax (alpha > 1) by bisection on the threshold.

    With x = (alpha - 1) * u, the solution is p_c = [x_c - tau]_+ ** (1/(alpha-1))
    with tau chosen so that sum(p) = 1 (Peters et al. 2019).  The mass
    sum_c [x_c - t]_+ ** (1/(alpha-1)) falls as t grows; it is >= 1 at
    t = max(x) - 1 (the top entry alone gives 1) and <= 1 at
    t = max(x) - n ** (1 - alpha) (every term is at most 1/n).  Bisect
    between the two until the bracket cannot shrink in float64.

    Returns (p, tau) with tau in x units.
    """
    u = np.asarray(u, dtype=F64)
    n = u.size
    x = (alpha - 1.0) * u
    expo = 1.0 / (alpha - 1.0)
    xmax = x.max()
    lo = xmax - 1.0
    hi = xmax - float(n) ** (1.0 - alpha)

    def mass(t):
        return np.sum(np.clip(x - t, 0.0, None) ** expo)

    for _ in range(4000):
        mid = 0.5 * (lo + hi)
        if not (lo < mid < hi):
            break
        if mass(mid) >= 1.0:
            lo = mid
        else:
            hi = mid
    tau = 0.5 * (lo + hi)
    p = np.clip(x - tau, 0.0, None) ** expo
    p = p / p.sum()
    return p, tau


def sparsemax_sort(u):
    """Sparsemax (alpha = 2), Martins & Astudillo (2016), by sorting.

    Sort descending to z; the support size is the largest k with
    1 + k * z_k > z_1 + ... + z_k, and tau = (z_1 + ... + z_k - 1) / k.
    Returns (p, tau).
    """
    x = np.asarray(u, dtype=F64)
    z = np.sort(x)[::-1]
    ks = np.arange(1, z.size + 1, dtype=F64)
    csum = np.cumsum(z)
    support = ks[1.0 + ks * z > csum]
    kstar = int(support.max())
    tau = (csum[kstar - 1] - 1.0) / kstar
    return np.clip(x - tau, 0.0, None), tau


def entmax15_sort(u):
    """1.5-entmax by sorting (Peters et al. 2019), with x = u / 2.

    For each prefix of the descending order z, with M_k the mean of z_1..z_k
    and S_k = sum_{j<=k} (z_j - M_k)**2, the candidate threshold is
    tau_k = M_k - sqrt(max(0, (1 - S_k) / k)); the support size is the
    largest k with tau_k <= z_k.  Returns (p, tau) with tau in x units.
    """
    x = 0.5 * np.asarray(u, dtype=F64)
    z = np.sort(x)[::-1]
    n = z.size
    ks = np.arange(1, n + 1, dtype=F64)
    means = np.cumsum(z) / ks
    # S_k = sum_{j<=k} z_j**2 - k * M_k**2, the same sum of squared deviations
    ss = np.cumsum(z * z) - ks * means * means
    taus = means - np.sqrt(np.clip((1.0 - ss) / ks, 0.0, None))
    ok = np.nonzero(taus <= z)[0]
    kstar = int(ok.max()) + 1
    tau = taus[kstar - 1]
    return np.clip(x - tau, 0.0, None) ** 2, tau


def entmax(u, alpha):
    """alpha-entmax of one logit row.

    Returns (p, tau_hat), tau_hat being the threshold in logit (u) units:
    a chunk is active iff u > tau_hat.  alpha = 1 is softmax (every entry
    active, tau_hat = -inf).  An empty row gives (empty, +inf).  For
    alpha = 1.5 and alpha = 2 the closed forms are computed as well and
    must agree with the bisection threshold.
    """
    u = np.asarray(u, dtype=F64)
    if u.size == 0:
        return np.zeros(0, dtype=F64), math.inf
    if alpha == 1.0:
        return softmax(u), -math.inf
    if alpha < 1.0:
        raise ValueError("alpha must be >= 1")
    p, tau = entmax_threshold_bisect(u, alpha)
    closed = None
    if alpha == 2.0:
        closed = sparsemax_sort(u)[1]
    elif alpha == 1.5:
        closed = entmax15_sort(u)[1]
    if closed is not None:
        assert abs(closed - tau) <= 1e-9 * max(1.0, abs(tau)), (closed, tau)
    return p, tau / (alpha - 1.0)


def entmax_rows(U, n, alpha):
    """alpha-entmax of many rows at once; row r uses its first n[r] entries.

    The same bisection as ``entmax_threshold_bisect``, run for all rows in
    lockstep (each row keeps its own bracket), followed by the same
    closed-form cross-checks for alpha = 2 and alpha = 1.5.  Returns
    (P [R, C] with zeros past n[r], tau_hat [R]): +inf for empty rows, -inf
    for alpha = 1 (softmax).
    """
    U = np.asarray(U, dtype=F64)
    R, C = U.shape
    n = np.asarray(n, dtype=np.int64)
    valid = np.arange(C)[None, :] < n[:, None]
    P = np.zeros((R, C), dtype=F64)
    tau_hat = np.full(R, math.inf, dtype=F64)
    rows = np.nonzero(n > 0)[0]
    if rows.size == 0:
        return P, tau_hat
    Ur = np.where(valid[rows], U[rows], -np.inf)
    if alpha == 1.0:
        mx = Ur.max(axis=1, keepdims=True)
        z = np.where(valid[rows], np.exp(Ur - mx), 0.0)
        P[rows] = z / z.sum(axis=1, keepdims=True)
        tau_hat[rows] = -math.inf
        return P, tau_hat
    if alpha < 1.0:
        raise ValueError("alpha must be >= 1")
    x = (alpha - 1.0) * Ur
    expo = 1.0 / (alpha - 1.0)
    xmax = x.max(axis=1)
    lo = xmax - 1.0
    hi = xmax - n[rows].astype(F64) ** (1.0 - alpha)

    def mass(t):
        d = np.clip(x - t[:, None], 0.0, None)
        return np.sum(d ** expo, axis=1)

    for _ in range(4000):
        mid = 0.5 * (lo + hi)
        live = (lo < mid) & (mid < hi)
        if not live.any():
            break
        up = mass(mid) >= 1.0
        lo = np.where(live & up, mid, lo)
        hi = np.where(live & ~up, mid, hi)
    tau = 0.5 * (lo + hi)
    Pr = np.clip(x - tau[:, None], 0.0, None) ** expo
    Pr = Pr / Pr.sum(axis=1, keepdims=True)
    if alpha in (2.0, 1.5):
        for j, r in enumerate(rows):
            u = U[r, :n[r]]
            closed = sparsemax_sort(u)[1] if alpha == 2.0 else entmax15_sort(u)[1]
            assert abs(closed - tau[j]) <= 1e-9 * max(1.0, abs(tau[j])), (closed, tau[j])
    P[rows] = Pr
    tau_hat[rows] = tau / (alpha - 1.0)
    return P, tau_hat


def route_position(q_group, kbar_h, alpha, gamma, scale, kdiag_h=None):
    """Route one position for one KV group.

    q_group : [G, D] the query heads of one KV head at this position
    kbar_h  : [n, D] that KV head's summaries of the routable chunks
    kdiag_h : [D] or None: the estimated summary of the position's own chunk
              (``summarize_diagonal``); when given and n > 0 it enters each
              head's entmax as one more entry, after the routed chunks, and
              takes its share of the probability mass
    Returns dict(u [G, n], tau_hat [G], p [G, n], wbar [n], mask [n] bool,
    p_diag [G] or None).

    Each query head gets its own entmax distribution; the group shares the
    average of the G distributions, and a chunk is active when any head
    gives it non-zero probability.
    """
    q_group = np.asarray(q_group, dtype=F64)
    G = q_group.shape[0]
    n = kbar_h.shape[0]
    u = np.zeros((G, n), dtype=F64)
    for g in range(G):
        u[g] = routing_logits(q_group[g], kbar_h, gamma, scale)
    p_diag = None
    if kdiag_h is not None and n > 0:
        ud = np.array([routing_logits(q_group[g], np.asarray(kdiag_h, dtype=F64)[None, :],
                                      gamma, scale)[0] for g in range(G)])
        pf, tau_hat = entmax_rows(np.concatenate([u, ud[:, None]], axis=1),
                                  np.full(G, n + 1), alpha)
        p, p_diag = pf[:, :n], pf[:, n]
    else:
        p, tau_hat = entmax_rows(u, np.full(G, n), alpha)
    wbar = p.mean(axis=0) if n else np.zeros(0, dtype=F64)
    if alpha == 1.0:
        mask = np.ones(n, dtype=bool)
    else:
        mask = np.any(u > tau_hat[:, None], axis=0) if n else np.zeros(0, bool)
    return dict(u=u, tau_hat=tau_hat, p=p, wbar=wbar, mask=mask, p_diag=p_diag)


def route_sequence(q, kbar, B, alpha, gamma, sigma, G, scale, rows=None,
                   num_slots=None, kdiag=None):
    """Phase 1 for one sequence.

    q    : [L, Hq, D];  kbar : [C, Hkv, D] summaries of the complete chunks
    rows : positions to route (default: all)
    kdiag: [L, Hkv, D] or None: estimated summaries of each position's own
           chunk (``summarize_diagonal``), an extra entmax entry of every
           row that has routable chunks (see ``route_position``)
    Returns mask [Hkv, L, S] bool, log_prior [Hkv, L, S] (-inf off the
    support) and tau_hat [Hq, L] (NaN for rows not routed), S = num_slots
    (default ceil(L / B)).  Position i routes to chunks c < floor(i / B).
    """
    q = np.asarray(q, dtype=F64)
    kbar = np.asarray(kbar, dtype=F64)
    L, Hq, D = q.shape
    Hkv = kbar.shape[1]
    S = num_slots if num_slots is not None else -(-L // B)
    rows = np.arange(L) if rows is None else np.asarray(list(rows), dtype=np.int64)
    mask = np.zeros((Hkv, L, S), dtype=bool)
    logp = np.full((Hkv, L, S), -np.inf, dtype=F64)
    tau_hat = np.full((Hq, L), np.nan, dtype=F64)
    if rows.size == 0:
        return mask, logp, tau_hat
    C = int(rows.max()) // B          # routable chunks of the last row
    ns = rows // B                    # routable chunks of each row
    for h in range(Hkv):
        # u[row, g, c] = gamma * s * <q[row, hG+g], kbar[c, h]>, c < n_row
        u = np.zeros((rows.size, G, max(C, 1) + 1), dtype=F64)
        if C:
            u[:, :, :C] = gamma * scale * np.einsum(
                "rgd,cd->rgc", q[rows, h * G:(h + 1) * G, :], kbar[:C, h, :])
        lens = ns.copy()
        if kdiag is not None:
            # the diagonal estimate goes right after each row's routed chunks
            ud = gamma * scale * np.einsum("rgd,rd->rg", q[rows, h * G:(h + 1) * G, :],
                                           np.asarray(kdiag, dtype=F64)[rows, h, :])
            u[np.arange(rows.size), :, ns] = ud
            lens = ns + (ns > 0)
        P, th = entmax_rows(u.reshape(rows.size * G, -1), np.repeat(lens, G), alpha)
        P = P.reshape(rows.size, G, -1)
        th = th.reshape(rows.size, G)
        tau_hat[h * G:(h + 1) * G, rows] = th.T
        wbar = P.mean(axis=1)                                  # [rows, C + 1]
        if alpha == 1.0:
            on = np.arange(u.shape[2])[None, :] < ns[:, None]
        else:
            on = np.any(u > th[:, :, None], axis=1)
            on &= np.arange(u.shape[2])[None, :] < ns[:, None]
        for j, i in enumerate(rows):
            nn = int(ns[j])
            mask[h, i, :nn] = on[j, :nn]
            sel = on[j, :nn]
            with np.errstate(divide="ignore"):
                logp[h, i, :nn][sel] = sigma * np.log(wbar[j, :nn][sel])
    return mask, logp, tau_hat


def routing_margin(q, kbar, B, gamma, scale, G, tau_hat, rows, num_slots):
    """Distance of each routing decision from its threshold.

    For every KV head h, requested row i and routable chunk c < floor(i/B):
    min over the G query heads of h of |u_{q,i,c} - tau_hat_{q,i}|, in logit
    units (+inf elsewhere, and for softmax routing where nothing is
    thresholded).  A decision closer than a numerical tolerance to its
    threshold may legitimately come out either way in finite precision.
    Returns [Hkv, len(rows), num_slots].
    """
    q = np.asarray(q, dtype=F64)
    kbar = np.asarray(kbar, dtype=F64)
    Hkv = kbar.shape[1]
    out = np.full((Hkv, len(rows), num_slots), np.inf, dtype=F64)
    for j, i in enumerate(rows):
        n = i // B
        if n == 0:
            continue
        for h in range(Hkv):
            u = gamma * scale * (q[i, h * G:(h + 1) * G, :] @ kbar[:n, h, :].T)
            th = tau_hat[h * G:(h + 1) * G, i]
            if not np.all(np.isfinite(th)):
                continue
            out[h, j, :n] = np.min(np.abs(u - th[:, None]), axis=0)
    return out


def route_topk_sequence(q, kbar, B, k, gamma, G, scale, rows=None, num_slots=None):
    """Top-k block routing, the comparison mode.

    The hierarchical methods the pages compare against (NSA, InfLLMv2) pick
    the top-k KV blocks by coarse attention scores and then run plain softmax
    attention over the picked tokens ([NL] Probleemstelling; the same passage
    in the Paper Overview and the aiexpert.news article).  The pages do not
    define the coarse score or how a GQA group shares it; the reading taken
    here: each query head's softmax over the routable chunks of its routing
    logits u = gamma * s * <q, k_bar>, summed over the group's G heads, is the
    chunk's score S_c; the min(k, n) chunks of largest S_c are active (equal
    scores: the lower chunk index first), with bias 0.

    Same arguments and layout as route_sequence (k >= 1).  Returns
    mask [Hkv, L, S] bool, log_prior [Hkv, L, S] (0 on the mask, -inf
    elsewhere) and score [Hkv, L, S] (S_c on routable chunks, NaN elsewhere).
    """
    q = np.asarray(q, dtype=F64)
    kbar = np.asarray(kbar, dtype=F64)
    L, Hq, D = q.shape
    Hkv = kbar.shape[1]
    S = num_slots if num_slots is not None else -(-L // B)
    rows = np.arange(L) if rows is None else np.asarray(list(rows), dtype=np.int64)
    mask = np.zeros((Hkv, L, S), dtype=bool)
    logp = np.full((Hkv, L, S), -np.inf, dtype=F64)
    score = np.full((Hkv, L, S), np.nan, dtype=F64)
    for h in range(Hkv):
        for i in rows:
            n = int(i) // B
            if n == 0:
                continue
            sc = np.zeros(n, dtype=F64)
            for g in range(G):
                sc += softmax(routing_logits(q[i, h * G + g], kbar[:n, h], gamma, scale))
            # stable sort on -score: equal scores keep the lower index first
            top = np.argsort(-sc, kind="stable")[:min(int(k), n)]
            mask[h, i, top] = True
            logp[h, i, top] = 0.0
            score[h, i, :n] = sc
    return mask, logp, score


# ---------------------------------------------------------------------------
# Phase 2: prior-induced sparse softmax  ([NL] / [ZH] Fase 2 / 阶段 2)
# ---------------------------------------------------------------------------

def _row_keys_and_bias(i, B, mask_row, logp_row):
    """Key positions a query at position i sees, with their additive bias.

    Routed chunks c < floor(i / B) that are active contribute all B keys
    with bias log_prior[c]; the diagonal chunk contributes keys
    floor(i / B) * B ... i with bias 0.
    """
    ci = i // B
    act = [c for c in range(ci) if mask_row[c]]
    idx = [np.arange(c * B, (c + 1) * B) for c in act] + [np.arange(ci * B, i + 1)]
    bias = [np.full(B, logp_row[c]) for c in act] + [np.zeros(i + 1 - ci * B)]
    return np.concatenate(idx).astype(np.int64), np.concatenate(bias).astype(F64)


def attention_rows(q, k, v, mask, log_prior, B, scale, G, rows):
    """Row-sparse form: for each requested position, attend over its keys.

    Returns out [len(rows), Hq, D], lse [Hq, len(rows)] (natural log).
    Logits are s * <q_i, k_j> + bias_j over the active routed keys and the
    causal diagonal; the result is their softmax applied to v.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    out = np.zeros((len(rows), Hq, D), dtype=F64)
    lse = np.zeros((Hq, len(rows)), dtype=F64)
    for r, i in enumerate(rows):
        for h in range(Hkv):
            idx, bias = _row_keys_and_bias(i, B, mask[h, i], log_prior[h, i])
            qg = q[i, h * G:(h + 1) * G, :]                    # [G, D]
            logits = scale * (qg @ k[idx, h, :].T) + bias[None, :]
            mx = logits.max(axis=1, keepdims=True)
            w = np.exp(logits - mx)
            ssum = w.sum(axis=1, keepdims=True)
            out[r, h * G:(h + 1) * G] = (w / ssum) @ v[idx, h, :]
            lse[h * G:(h + 1) * G, r] = mx[:, 0] + np.log(ssum[:, 0])
    return out, lse


def attention_dense(q, k, v, mask, log_prior, B, scale, G):
    """Dense form: a full causal L x L score matrix plus a bias matrix.

    bias[i, j] = log_prior[c(j)] for j in an active routed chunk of row i,
    0 on the diagonal chunk (j <= i), -inf everywhere else.  Returns
    out [L, Hq, D], lse [Hq, L].
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((L, Hq, D), dtype=F64)
    lse = np.zeros((Hq, L), dtype=F64)
    for h in range(Hkv):
        bias = np.full((L, L), -np.inf, dtype=F64)
        for i in range(L):
            ci = i // B
            for c in range(ci):
                if mask[h, i, c]:
                    bias[i, c * B:(c + 1) * B] = log_prior[h, i, c]
            bias[i, ci * B:i + 1] = 0.0
        for qh in range(h * G, (h + 1) * G):
            scores = scale * (q[:, qh, :] @ k[:, h, :].T) + bias
            mx = scores.max(axis=1, keepdims=True)
            w = np.exp(scores - mx)
            ssum = w.sum(axis=1, keepdims=True)
            out[:, qh, :] = (w / ssum) @ v[:, h, :]
            lse[qh] = mx[:, 0] + np.log(ssum[:, 0])
    return out, lse


# ---------------------------------------------------------------------------
# whole forward passes
# ---------------------------------------------------------------------------

def _group_size(Hq, Hkv, enable_gqa):
    if enable_gqa:
        if Hq % Hkv:
            raise ValueError("Hq must be a multiple of Hkv")
    elif Hq != Hkv:
        raise ValueError("enable_gqa=False needs Hq == Hkv")
    return Hq // Hkv


def prefill(q, k, v, qbar, B, alpha, gamma, sigma, enable_gqa=True,
            to_bf16=False, scale=None, rows=None, dense=False, num_slots=None,
            estimate_diagonal=False):
    """Phases 0-2 for one sequence (causal prefill).

    q [L, Hq, D], k/v [L, Hkv, D], qbar [Hkv, D].  ``to_bf16`` rounds the
    summaries to bfloat16 (inputs stored in bfloat16).  ``rows`` limits
    routing and attention to the given positions (row-sparse form);
    ``dense=True`` uses the dense score-matrix form for every row instead.
    ``estimate_diagonal`` adds each row's estimated own-chunk summary to its
    routing (``route_position``).
    Returns dict(kbar, kdiag, mask, log_prior, tau_hat, out, lse, rows).
    """
    q = np.asarray(q, dtype=F64)
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    G = _group_size(Hq, Hkv, enable_gqa)
    s = _default_scale(D, scale)
    kbar = summarize(k, qbar, B, to_bf16)
    kdiag = summarize_diagonal(k, qbar, B, to_bf16) if estimate_diagonal else None
    rows = list(range(L)) if rows is None else list(rows)
    mask, logp, tau_hat = route_sequence(q, kbar, B, alpha, gamma, sigma, G, s,
                                         rows=rows, num_slots=num_slots, kdiag=kdiag)
    if dense:
        out, lse = attention_dense(q, k, v, mask, logp, B, s, G)
        out, lse = out[rows], lse[:, rows]
    else:
        out, lse = attention_rows(q, k, v, mask, logp, B, s, G, rows)
    return dict(kbar=kbar, kdiag=kdiag, mask=mask, log_prior=logp, tau_hat=tau_hat,
                out=out, lse=lse, rows=rows)


def prefill_varlen(q, k, v, qbar, cu_seqlens, B, alphas, gamma, sigma,
                   enable_gqa=True, to_bf16=False, scale=None,
                   rows_per_seq=None, num_slots=None, estimate_diagonal=False):
    """Packed variable-length prefill: every sequence is independent.

    alphas[s] is sequence s's entmax alpha.  ``rows_per_seq[s]`` lists
    positions local to sequence s (default: all).  Returns a list of
    per-sequence result dicts (see ``prefill``).
    """
    res = []
    for s in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        rows = None if rows_per_seq is None else rows_per_seq[s]
        res.append(prefill(q[a:b], k[a:b], v[a:b], qbar, B, float(alphas[s]),
                           gamma, sigma, enable_gqa, to_bf16, scale, rows,
                           num_slots=num_slots, estimate_diagonal=estimate_diagonal))
    return res


def decode(q_new, k_cache, v_cache, kbar_cache, L, B, alpha, gamma, sigma,
           enable_gqa=True, scale=None, kdiag=None):
    """One decode step: the row i = L - 1 of a sequence of length L.

    q_new [Hq, D]; k_cache / v_cache [>= L, Hkv, D] hold the L tokens
    (the new token's key and value at position L - 1); kbar_cache
    [>= floor((L-1)/B), Hkv, D] holds the cached summaries of the complete
    chunks.  ``kdiag`` [Hkv, D], when given, is the estimated summary of the
    row's own chunk (``summarize_diagonal`` of the cached keys at its last
    position), which then enters the routing (``route_position``).
    Returns dict(out [Hq, D], lse [Hq], mask [Hkv, n], log_prior [Hkv, n],
    tau_hat [Hq]) with n = floor((L-1)/B).
    """
    q_new = np.asarray(q_new, dtype=F64)
    Hq, D = q_new.shape
    Hkv = k_cache.shape[1]
    G = _group_size(Hq, Hkv, enable_gqa)
    s = _default_scale(D, scale)
    i = L - 1
    n = i // B
    kb = np.asarray(kbar_cache[:n], dtype=F64)
    mask = np.zeros((Hkv, n), dtype=bool)
    logp = np.full((Hkv, n), -np.inf, dtype=F64)
    tau_hat = np.zeros(Hq, dtype=F64)
    for h in range(Hkv):
        r = route_position(q_new[h * G:(h + 1) * G], kb[:, h, :], alpha, gamma, s,
                           None if kdiag is None else kdiag[h])
        mask[h] = r["mask"]
        tau_hat[h * G:(h + 1) * G] = r["tau_hat"]
        with np.errstate(divide="ignore"):
            logp[h][r["mask"]] = sigma * np.log(r["wbar"][r["mask"]])
    # attend: reuse the row-sparse form on a one-row view of the sequence
    k_seq = np.asarray(k_cache[:L], dtype=F64)
    v_seq = np.asarray(v_cache[:L], dtype=F64)
    qfull = np.zeros((L, Hq, D), dtype=F64)
    qfull[i] = q_new
    mfull = np.zeros((Hkv, L, n + 1), dtype=bool)
    lfull = np.full((Hkv, L, n + 1), -np.inf, dtype=F64)
    mfull[:, i, :n] = mask
    lfull[:, i, :n] = logp
    out, lse = attention_rows(qfull, k_seq, v_seq, mfull, lfull, B, s, G, [i])
    return dict(out=out[0], lse=lse[:, 0], mask=mask, log_prior=logp,
                tau_hat=tau_hat)
