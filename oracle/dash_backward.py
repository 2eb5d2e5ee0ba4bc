"""CPU oracle for the backward pass of the DashAttention forward path.

Test infrastructure only, like ``dash_oracle`` (plain NumPy, float64).  The
pages make differentiability the method's central claim: alpha-entmax lets
gradients flow from the second-stage attention back through the routing to
the phase-0 summaries ([NL] "Technische Samenvatting: DashAttention", Fase 1,
Differentieerbaarheid bullet; Belangrijkste Bijdragen, item 1).  They print
no backward formulas; each step below is the derivative of the matching
forward step in ``dash_oracle``, taken in reverse order:

  phase 2  o = sum_j P_j v_j, P = softmax(s <q, k_j> + b_j):
           dv_j += P_j do;  dP_j = <do, v_j>;  D = <do, o>;
           dS_j = P_j (dP_j - D);  dq += s sum_j dS_j k_j;  dk_j += s dS_j q;
           db_c  = sum over the chunk's keys (and the group's heads) of dS
  prior    b_c = sigma log w_bar_c on the active chunks: dw_bar_c = sigma db_c / w_bar_c
  GQA      w_bar = mean over the G heads of p:  dp_q = dw_bar / G
  entmax   the Jacobian of p = alpha-entmax(u) on the support (Peters,
           Niculae & Martins 2019): dp/du = diag(r) - r r^T / sum(r),
           r = p^(2 - alpha) on the support, 0 off it (alpha = 1: r = p)
  logits   u_c = gamma s <q, k_bar_c>:  dq += gamma s sum_c du_c k_bar_c;
           dk_bar_c += gamma s du_c q
  phase 0  k_bar = sum_t pi_t k_t, pi = softmax(s <q_bar, k_t>):
           dpi_t = <dk_bar, k_t>;  dz = pi (dpi - <pi, dpi>);
           dk_t += pi_t dk_bar + s dz_t q_bar;  dq_bar += s sum_t dz_t k_t

The support (the mask) is piecewise constant in the inputs, so it carries no
gradient of its own: it enters only through p.  Rounding of summaries to the
storage dtype is passed through as the identity.  Packed sequences are
independent: each is the one-sequence case.

With estimate_diagonal (reading E1) each routed row's entmax has one more
entry, u_d = gamma s <q, k_hat_i>, whose probability feeds no prior: its dp
is 0, so du_d = -r_d rho, and rho's denominator includes r_d.  Then
dq += gamma s du_d k_hat_i, dk_hat_i = gamma s sum over the group's heads of
du_d q, and k_hat_i = sum_{t = cB..i} pi_t k_t (the running summary of the
row's own chunk) passes it back like a summary:
dk_t += pi_t dk_hat_i + s dz_t q_bar, dq_bar += s sum_t dz_t k_t.
"""

from __future__ import annotations

import math

import numpy as np

from .dash_oracle import (F64, _default_scale, _group_size, _row_keys_and_bias,
                          route_position, route_sequence, softmax, summarize,
                          summarize_diagonal)


def attention_backward_rows(q, k, v, mask, log_prior, B, scale, G, dout, rows=None):
    """Backward of phase 2 (``attention_rows``) for a given routing.

    q/dout [L, Hq, D], k/v [L, Hkv, D], mask/log_prior [Hkv, L, S].
    Returns dict(dq, dk, dv, dbias [Hkv, L, S] (the gradient of each active
    routed chunk's bias, 0 elsewhere), delta [Hq, L] = <do, o>).  With
    ``rows`` only those query rows are taken: their dq, dbias and delta are
    complete, while dk and dv hold just those rows' contributions.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    dout = np.asarray(dout, dtype=F64)
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    S = mask.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbias = np.zeros((Hkv, L, S), dtype=F64)
    delta = np.zeros((Hq, L), dtype=F64)
    for i in (range(L) if rows is None else rows):
        for h in range(Hkv):
            idx, bias = _row_keys_and_bias(i, B, mask[h, i], log_prior[h, i])
            chunk = idx // B
            for qh in range(h * G, (h + 1) * G):
                p = softmax(scale * (k[idx, h, :] @ q[i, qh]) + bias)
                o = p @ v[idx, h, :]
                dp = v[idx, h, :] @ dout[i, qh]
                dlt = float(dout[i, qh] @ o)
                ds = p * (dp - dlt)
                dq[i, qh] += scale * (ds @ k[idx, h, :])
                dk[idx, h, :] += scale * np.outer(ds, q[i, qh])
                dv[idx, h, :] += np.outer(p, dout[i, qh])
                delta[qh, i] = dlt
                routed = chunk < i // B
                np.add.at(dbias[h, i], chunk[routed], ds[routed])
    return dict(dq=dq, dk=dk, dv=dv, dbias=dbias, delta=delta)


def attention_backward_keys(q, k, v, mask, log_prior, B, scale, G, dout, lse, out, keys):
    """dk and dv of the given key positions from phase 2's backward, taken
    column by column: for key j, every query row i that sees it (rows of j's
    own chunk at or after j, bias 0; later rows with j's chunk active, bias
    log_prior), with P_ij = exp(s <q_i, k_j> + b_ij - lse_i) and
    dS_ij = P_ij (<do_i, v_j> - <do_i, o_i>), from the forward's lse [Hq, L]
    (natural log) and output o [L, Hq, D].

    Returns dict(dk [len(keys), Hkv, D], dv [len(keys), Hkv, D]); the same
    quantities as ``attention_backward_rows`` summed the other way round.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    dout = np.asarray(dout, dtype=F64)
    lse = np.asarray(lse, dtype=F64)
    out = np.asarray(out, dtype=F64)
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    dk = np.zeros((len(keys), Hkv, D), dtype=F64)
    dv = np.zeros((len(keys), Hkv, D), dtype=F64)
    for h in range(Hkv):
        # the rows that see each key, with their bias
        seen = []
        for j in keys:
            c = j // B
            own = np.arange(j, min((c + 1) * B, L))
            later = np.arange((c + 1) * B, L)
            later = later[mask[h, later, c]] if later.size else later
            seen.append((np.concatenate([own, later]).astype(np.int64),
                         np.concatenate([np.zeros(own.size), log_prior[h, later, c]])))
        for qh in range(h * G, (h + 1) * G):
            qh_q = np.ascontiguousarray(q[:, qh, :])
            qh_do = np.ascontiguousarray(dout[:, qh, :])
            dlt = np.einsum("rd,rd->r", qh_do, out[:, qh, :])   # <do_i, o_i>
            for n, j in enumerate(keys):
                rows, bias = seen[n]
                qi, doi = qh_q[rows], qh_do[rows]
                p = np.exp(scale * (qi @ k[j, h]) + bias - lse[qh, rows])
                ds = p * (doi @ v[j, h] - dlt[rows])
                dv[n, h] += p @ doi
                dk[n, h] += scale * (ds @ qi)
    return dict(dk=dk, dv=dv)


def entmax_backward(p, dp, alpha):
    """du for p = alpha-entmax(u) (one row): J^T dp with the symmetric
    Jacobian diag(r) - r r^T / sum(r), r = p^(2 - alpha) on the support."""
    p = np.asarray(p, dtype=F64)
    dp = np.asarray(dp, dtype=F64)
    r = np.where(p > 0, p ** (2.0 - alpha), 0.0)
    sr = r.sum()
    if sr == 0.0:
        return np.zeros_like(p)
    return r * dp - r * (r @ dp) / sr


def routing_backward(q, kbar, B, alpha, gamma, sigma, G, scale, dbias, rows=None, kdiag=None):
    """Backward of the log-prior of ``route_sequence`` (b = sigma log w_bar on
    the active chunks) to the queries and the summaries.

    dbias [Hkv, L, S].  Returns dict(dq [L, Hq, D], dkbar [C, Hkv, D],
    du [Hq, L, S] (zero past each row's routable chunks), dkdiag [L, Hkv, D]
    (the gradient of each row's own-chunk estimate when ``kdiag`` is given,
    else None)).  With ``rows`` only those rows are taken (their dq, du and
    dkdiag complete, dkbar partial).
    """
    q = np.asarray(q, dtype=F64)
    kbar = np.asarray(kbar, dtype=F64)
    L, Hq, D = q.shape
    Hkv = kbar.shape[1]
    S = dbias.shape[2]
    dq = np.zeros_like(q)
    dkbar = np.zeros_like(kbar)
    du = np.zeros((Hq, L, S), dtype=F64)
    dkdiag = None if kdiag is None else np.zeros((L, Hkv, q.shape[2]), dtype=F64)
    gs = gamma * scale
    for i in (range(L) if rows is None else rows):
        n = i // B
        if n == 0:
            continue
        for h in range(Hkv):
            kd = None if kdiag is None else np.asarray(kdiag[i, h], dtype=F64)
            r = route_position(q[i, h * G:(h + 1) * G], kbar[:n, h, :], alpha, gamma, scale,
                               kdiag_h=kd)
            m = r["mask"]
            dw = np.zeros(n, dtype=F64)
            dw[m] = sigma * dbias[h, i, :n][m] / r["wbar"][m]
            dp = dw / G
            for g in range(G):
                qh = h * G + g
                if kd is None:
                    d = entmax_backward(r["p"][g], dp, alpha)
                    dq[i, qh] += gs * (d @ kbar[:n, h, :])
                else:
                    # the own-chunk entry: in the entmax, no prior (dp 0)
                    d = entmax_backward(np.append(r["p"][g], r["p_diag"][g]),
                                        np.append(dp, 0.0), alpha)
                    dq[i, qh] += gs * (d[:n] @ kbar[:n, h, :] + d[n] * kd)
                    dkdiag[i, h] += gs * d[n] * q[i, qh]
                    d = d[:n]
                du[qh, i, :n] = d
                dkbar[:n, h, :] += gs * np.outer(d, q[i, qh])
    return dict(dq=dq, dkbar=dkbar, du=du, dkdiag=dkdiag)


def summarize_backward(k, qbar, B, dkbar):
    """Backward of ``summarize`` (complete chunks only).

    Returns dict(dk [L, Hkv, D], dqbar [Hkv, D])."""
    k = np.asarray(k, dtype=F64)
    qbar = np.asarray(qbar, dtype=F64)
    dkbar = np.asarray(dkbar, dtype=F64)
    L, Hkv, D = k.shape
    s = 1.0 / math.sqrt(D)
    dk = np.zeros_like(k)
    dqbar = np.zeros_like(qbar)
    for c in range(L // B):
        for h in range(Hkv):
            keys = k[c * B:(c + 1) * B, h, :]
            pi = softmax(s * (keys @ qbar[h]))
            dpi = keys @ dkbar[c, h]
            dz = pi * (dpi - pi @ dpi)
            dk[c * B:(c + 1) * B, h, :] += np.outer(pi, dkbar[c, h]) + s * np.outer(dz, qbar[h])
            dqbar[h] += s * (dz @ keys)
    return dict(dk=dk, dqbar=dqbar)


def summarize_diagonal_backward(k, qbar, B, dkdiag):
    """Backward of ``summarize_diagonal``: every row i's estimate of its own
    chunk, k_hat_i = sum_{t = cB..i} pi_t k_t, pi = softmax(s <q_bar, k_t>).

    Returns dict(dk [L, Hkv, D], dqbar [Hkv, D])."""
    k = np.asarray(k, dtype=F64)
    qbar = np.asarray(qbar, dtype=F64)
    dkdiag = np.asarray(dkdiag, dtype=F64)
    L, Hkv, D = k.shape
    s = 1.0 / math.sqrt(D)
    dk = np.zeros_like(k)
    dqbar = np.zeros_like(qbar)
    for i in range(L):
        c0 = (i // B) * B
        for h in range(Hkv):
            keys = k[c0:i + 1, h, :]
            pi = softmax(s * (keys @ qbar[h]))
            dpi = keys @ dkdiag[i, h]
            dz = pi * (dpi - pi @ dpi)
            dk[c0:i + 1, h, :] += np.outer(pi, dkdiag[i, h]) + s * np.outer(dz, qbar[h])
            dqbar[h] += s * (dz @ keys)
    return dict(dk=dk, dqbar=dqbar)


def prefill_backward(q, k, v, qbar, B, alpha, gamma, sigma, dout, enable_gqa=True,
                     scale=None, estimate_diagonal=False):
    """Gradients of sum(dout * o) for the causal prefill of one sequence
    (``dash_oracle.prefill`` without storage rounding) with respect to q, k,
    v and q_bar, plus the intermediate gradients of the stages.

    Returns dict(dq, dk, dv, dqbar, dbias, dkbar, du, delta, out, lse, mask,
    log_prior)."""
    from .dash_oracle import attention_rows

    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    G = _group_size(Hq, Hkv, enable_gqa)
    s = _default_scale(D, scale)
    kbar = summarize(k, qbar, B)
    kdiag = summarize_diagonal(k, qbar, B) if estimate_diagonal else None
    mask, logp, _ = route_sequence(q, kbar, B, alpha, gamma, sigma, G, s, kdiag=kdiag)
    out, lse = attention_rows(q, k, v, mask, logp, B, s, G, list(range(L)))
    a = attention_backward_rows(q, k, v, mask, logp, B, s, G, dout)
    r = routing_backward(q, kbar, B, alpha, gamma, sigma, G, s, a["dbias"], kdiag=kdiag)
    m = summarize_backward(k, qbar, B, r["dkbar"])
    dk, dqbar = a["dk"] + m["dk"], m["dqbar"]
    if kdiag is not None:
        md = summarize_diagonal_backward(k, qbar, B, r["dkdiag"])
        dk, dqbar = dk + md["dk"], dqbar + md["dqbar"]
    return dict(dq=a["dq"] + r["dq"], dk=dk, dv=a["dv"], dqbar=dqbar,
                dbias=a["dbias"], dkbar=r["dkbar"], du=r["du"], dkdiag=r["dkdiag"],
                delta=a["delta"], out=out, lse=lse, mask=mask, log_prior=logp)
