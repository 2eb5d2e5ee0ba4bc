"""Pins of the backward oracle (oracle/dash_backward.py) against facts fixed
outside it: central finite differences of the forward oracle (itself pinned
in test_oracle.py), torch autograd on the dense attention form, and the
sigma = 0 case where the routing carries no gradient."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import dash_backward as OB


def _inputs(seed, L=20, Hq=4, Hkv=2, D=6):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((L, Hq, D)), k=rng.standard_normal((L, Hkv, D)),
                v=rng.standard_normal((L, Hkv, D)), qbar=0.5 * rng.standard_normal((Hkv, D)),
                dout=rng.standard_normal((L, Hq, D)))


def _loss(x, B, alpha, gamma, sigma, diag=False):
    r = O.prefill(x["q"], x["k"], x["v"], x["qbar"], B, alpha, gamma, sigma,
                  estimate_diagonal=diag)
    return float(np.sum(x["dout"] * r["out"]))


@pytest.mark.parametrize("alpha,gamma,sigma", [(1.5, 4.0, 1.0), (2.0, 5.0, 0.5),
                                               (1.25, 4.0, 1.0), (1.0, 2.0, 0.7)])
def test_backward_matches_finite_differences(alpha, gamma, sigma):
    B = 4
    x = _inputs(31)
    G = 2
    s = 1.0 / math.sqrt(6)
    # no routing decision may sit near its threshold: a step of eps must not
    # change any support
    kbar = O.summarize(x["k"], x["qbar"], B)
    _, _, th = O.route_sequence(x["q"], kbar, B, alpha, gamma, sigma, G, s)
    if alpha > 1.0:
        mg = O.routing_margin(x["q"], kbar, B, gamma, s, G, th, list(range(20)), 5)
        assert np.min(mg) > 1e-4
    g = OB.prefill_backward(x["q"], x["k"], x["v"], x["qbar"], B, alpha, gamma, sigma,
                            x["dout"])
    rng = np.random.default_rng(7)
    eps = 1e-6
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"]), ("qbar", g["dqbar"])):
        arr = x[name]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(x, B, alpha, gamma, sigma)
            arr[idx] = old - eps
            lm = _loss(x, B, alpha, gamma, sigma)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 + 1e-5 * abs(fd), (name, idx, fd, grad[idx])


def test_attention_backward_matches_torch_autograd():
    # dense form with the bias matrix of the routing, differentiated by torch
    B, L = 4, 20
    x = _inputs(32)
    G, s = 2, 1.0 / math.sqrt(6)
    kbar = O.summarize(x["k"], x["qbar"], B)
    mask, logp, _ = O.route_sequence(x["q"], kbar, B, 1.5, 4.0, 1.0, G, s)
    a = OB.attention_backward_rows(x["q"], x["k"], x["v"], mask, logp, B, s, G, x["dout"])
    tq = torch.tensor(x["q"], requires_grad=True)
    tk = torch.tensor(x["k"], requires_grad=True)
    tv = torch.tensor(x["v"], requires_grad=True)
    tb = torch.zeros((2, L, 5), dtype=torch.float64, requires_grad=True)  # per routed chunk
    outs = []
    for qh in range(4):
        h = qh // G
        bias = torch.full((L, L), -math.inf, dtype=torch.float64)
        for i in range(L):
            for c in range(i // B):
                if mask[h, i, c]:
                    bias[i, c * B:(c + 1) * B] = float(logp[h, i, c])
            bias[i, (i // B) * B:i + 1] = 0.0
        # the bias of routed keys through the learnable per-chunk offsets
        cidx = torch.arange(L) // B
        add = tb[h][:, cidx]                                   # [L, L]
        routed = torch.isfinite(bias) & (cidx[None, :] < (torch.arange(L) // B)[:, None])
        full = bias + torch.where(routed, add, torch.zeros_like(add))
        sc = s * tq[:, qh, :] @ tk[:, h, :].T + full
        outs.append(torch.softmax(sc, dim=1) @ tv[:, h, :])
    out = torch.stack(outs, dim=1)
    (out * torch.tensor(x["dout"])).sum().backward()
    np.testing.assert_allclose(a["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(a["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(a["dv"], tv.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(a["dbias"], tb.grad.numpy(), atol=1e-12)
    assert np.all(a["dbias"][~mask] == 0.0)


@pytest.mark.parametrize("alpha", [1.0, 1.25, 1.5, 2.0])
def test_entmax_jacobian_matches_finite_differences(alpha):
    rng = np.random.default_rng(33)
    u = 3.0 * rng.standard_normal(9)
    dp = rng.standard_normal(9)
    p = O.entmax(u, alpha)[0]
    du = OB.entmax_backward(p, dp, alpha)
    eps = 1e-6
    for c in range(9):
        e = np.zeros(9)
        e[c] = eps
        fd = (O.entmax(u + e, alpha)[0] - O.entmax(u - e, alpha)[0]) @ dp / (2 * eps)
        assert abs(fd - du[c]) <= 1e-7, (c, fd, du[c])
    # the gradient is orthogonal to shifts of u (entmax is shift invariant)
    assert abs(du.sum()) < 1e-12


def test_sigma_zero_routing_carries_no_gradient():
    # sigma = 0: the bias is 0 wherever it is finite, so q_bar gets nothing and
    # q's gradient is the attention part alone
    B = 4
    x = _inputs(34)
    g = OB.prefill_backward(x["q"], x["k"], x["v"], x["qbar"], B, 1.5, 4.0, 0.0, x["dout"])
    assert np.all(g["dqbar"] == 0.0) and np.all(g["dkbar"] == 0.0)
    s = 1.0 / math.sqrt(6)
    a = OB.attention_backward_rows(x["q"], x["k"], x["v"], g["mask"], g["log_prior"], B, s, 2,
                                   x["dout"])
    np.testing.assert_allclose(g["dq"], a["dq"], atol=0)
    np.testing.assert_allclose(g["dk"], a["dk"], atol=0)


def test_row_subsets_match_the_full_pass():
    # the rows option of the stage functions takes exactly those rows
    B = 4
    x = _inputs(35)
    s = 1.0 / math.sqrt(6)
    kbar = O.summarize(x["k"], x["qbar"], B)
    mask, logp, _ = O.route_sequence(x["q"], kbar, B, 1.5, 4.0, 1.0, 2, s)
    full = OB.attention_backward_rows(x["q"], x["k"], x["v"], mask, logp, B, s, 2, x["dout"])
    rows = [0, 5, 13, 19]
    part = OB.attention_backward_rows(x["q"], x["k"], x["v"], mask, logp, B, s, 2, x["dout"],
                                      rows=rows)
    for key in ("dq", "delta"):
        ax = 0 if key == "dq" else 1
        np.testing.assert_array_equal(np.take(part[key], rows, axis=ax),
                                      np.take(full[key], rows, axis=ax))
    np.testing.assert_array_equal(part["dbias"][:, rows], full["dbias"][:, rows])
    rf = OB.routing_backward(x["q"], kbar, B, 1.5, 4.0, 1.0, 2, s, full["dbias"])
    rp = OB.routing_backward(x["q"], kbar, B, 1.5, 4.0, 1.0, 2, s, full["dbias"], rows=rows)
    np.testing.assert_array_equal(rp["dq"][rows], rf["dq"][rows])


def test_key_columns_match_the_row_pass():
    # the column form (per key, from the forward's lse and output) against the
    # row form; the ragged tail and both bias kinds are in range
    B = 4
    x = _inputs(36, L=22)
    s = 1.0 / math.sqrt(6)
    kbar = O.summarize(x["k"], x["qbar"], B)
    mask, logp, _ = O.route_sequence(x["q"], kbar, B, 1.5, 4.0, 1.0, 2, s)
    out, lse = O.attention_rows(x["q"], x["k"], x["v"], mask, logp, B, s, 2, list(range(22)))
    rows = OB.attention_backward_rows(x["q"], x["k"], x["v"], mask, logp, B, s, 2, x["dout"])
    keys = [0, 3, 4, 9, 15, 19, 21]
    cols = OB.attention_backward_keys(x["q"], x["k"], x["v"], mask, logp, B, s, 2, x["dout"],
                                      lse, out, keys)
    np.testing.assert_allclose(cols["dk"], rows["dk"][keys], atol=1e-12)
    np.testing.assert_allclose(cols["dv"], rows["dv"][keys], atol=1e-12)


@pytest.mark.parametrize("alpha,gamma,sigma", [(1.5, 4.0, 1.0), (2.0, 5.0, 1.0), (1.0, 2.0, 0.7)])
def test_estimate_diagonal_backward_matches_finite_differences(alpha, gamma, sigma):
    # the own-chunk entry of every routed row (reading E1) and its running
    # summary are differentiated too
    B = 4
    x = _inputs(37)
    s = 1.0 / math.sqrt(6)
    kbar = O.summarize(x["k"], x["qbar"], B)
    kd = O.summarize_diagonal(x["k"], x["qbar"], B)
    _, _, th = O.route_sequence(x["q"], kbar, B, alpha, gamma, sigma, 2, s, kdiag=kd)
    if alpha > 1.0:
        # no routing decision (routed chunks or the own-chunk entry) near a threshold
        mg = O.routing_margin(x["q"], kbar, B, gamma, s, 2, th, list(range(20)), 5)
        assert np.min(mg) > 1e-4
        ud = gamma * s * np.einsum("lgd,lgd->gl", x["q"], np.repeat(kd, 2, axis=1))
        assert np.min(np.abs(ud - th)[:, B:]) > 1e-4
    g = OB.prefill_backward(x["q"], x["k"], x["v"], x["qbar"], B, alpha, gamma, sigma,
                            x["dout"], estimate_diagonal=True)
    assert np.max(np.abs(g["dkdiag"])) > 0.0
    rng = np.random.default_rng(8)
    eps = 1e-6
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("qbar", g["dqbar"])):
        arr = x[name]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(x, B, alpha, gamma, sigma, True)
            arr[idx] = old - eps
            lm = _loss(x, B, alpha, gamma, sigma, True)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 + 1e-5 * abs(fd), (name, idx, fd, grad[idx])


def test_diagonal_summary_backward_is_the_summary_backward_on_full_chunks():
    # at a chunk's last row the running estimate is the chunk's summary, so
    # a gradient placed only on those rows back-propagates as the summary's
    B = 4
    x = _inputs(38)
    dkd = np.zeros((20, 2, 6))
    dkb = np.random.default_rng(9).standard_normal((5, 2, 6))
    for c in range(5):
        dkd[c * B + B - 1] = dkb[c]
    a = OB.summarize_diagonal_backward(x["k"], x["qbar"], B, dkd)
    b = OB.summarize_backward(x["k"], x["qbar"], B, dkb)
    np.testing.assert_allclose(a["dk"], b["dk"], atol=1e-12)
    np.testing.assert_allclose(a["dqbar"], b["dqbar"], atol=1e-12)
