"""Shared helpers of the GPU parity tests (imported by test modules only)."""

import math

import numpy as np
import torch

import oracle as O
from sparse_hierarchical_attention_dash_amd import ops

BAND = 1e-4          # mask bits may differ only this close to the threshold
TOL = {"bf16": 2e-2, "f32": 1e-4}
# LSE: the bf16 kernels normalise by the sum of the bf16-rounded attention
# weights (the same weights that multiply V), each within 2^-8 relative of its
# fp32 value, so log(sum) moves by at most 2^-8 = 3.9e-3; fp32 score and
# accumulation errors add < 1e-4.  fp32 kernels keep fp32 weights.
LSE_TOL = {"bf16": 2.0 ** -8 + 1e-4, "f32": 1e-4}


def to_dev(a, dtype):
    """float32 numpy -> (device tensor in dtype, float64 numpy of its exact values)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda(), t.to(torch.float64).numpy()


def unpack_bits(ab, slots):
    """int64 [..., W] words (chunk c = bit c%64 of word c//64) -> bool [..., slots]."""
    a = np.ascontiguousarray(ab.detach().cpu().numpy()).view(np.uint64)
    b = np.unpackbits(a.view(np.uint8), bitorder="little")
    return b.reshape(a.shape[:-1] + (a.shape[-1] * 64,))[..., :slots].astype(bool)


def pack_bits(mask):
    """bool [..., S] -> int64 [..., W] words, chunk c in bit c%64 of word c//64."""
    S = mask.shape[-1]
    Wd = -(-S // 64)
    full = np.zeros(mask.shape[:-1] + (Wd * 64,), dtype=bool)
    full[..., :S] = mask
    by = np.packbits(full, axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view(np.uint64).view(np.int64)


def flush(msg):
    print(msg, flush=True)


def compare_masks(gpu_bits, ora_mask, margin, what=""):
    """gpu_bits/ora_mask/margin: [Hkv, R, S].  Flips are allowed only inside the
    threshold band: where some head of the group has |u - tau_hat| < BAND."""
    mism = gpu_bits != ora_mask
    bad = mism & ~(margin < BAND)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} mask bits differ outside the band, "
                             f"first at {idx.tolist()} (margins {margin[tuple(idx.T)]})")
    return int(mism.sum())


def oracle_mask_on(qx, kbg, B, alpha, gamma, sigma, G, s, rows, S, kdiag=None):
    """The oracle's routing of the given rows run on the GPU's own summaries.

    The summaries are checked against the oracle's by themselves
    (``check_summaries``).  Routing both sides on the same summary values
    keeps a last-place difference of a summary from moving a logit, so the
    band rule holds for every bit with no exemption.  Returns
    (mask [Hkv, R, S], margin [Hkv, R, S], tau_hat [Hq, R])."""
    mask, _, th = O.route_sequence(qx, kbg, B, alpha, gamma, sigma, G, s, rows=rows,
                                   num_slots=S, kdiag=kdiag)
    margin = O.routing_margin(qx, kbg, B, gamma, s, G, th, rows, S)
    return mask[:, rows], margin, th[:, rows]


def summary_bound(k, B):
    """Per (chunk, head, dim) bound on the fp32 error of a summary: the
    weights sum to 1, so the weighted sum of B keys carries at most about
    B * 2^-24 (accumulation) + 1e-6 (weights) times the largest |key|."""
    L, Hkv, D = k.shape
    C = L // B
    kk = np.abs(k[:C * B]).reshape(C, B, Hkv, D).max(axis=1)
    return (B * 2.0 ** -24 + 1e-6) * kk


def check_summaries(kbar_gpu, kbar_ora, dtype, k=None, B=64):
    fp = summary_bound(k, B) if k is not None else 2e-6
    if dtype == "f32":
        assert np.all(np.abs(kbar_gpu - kbar_ora) <= fp + 1e-5 * np.abs(kbar_ora))
        return 0
    # bf16: the fp32 result, within the bound above of the exact value, is
    # rounded once; it can land one unit in the last place (2^-7 relative at
    # most) away from the rounded exact value, or more where cancellation
    # makes the value small next to the fp32 error
    d = np.abs(kbar_gpu - kbar_ora)
    if d.size == 0:
        return 0.0
    ulp = np.abs(kbar_ora) * 2.0 ** -7 + 2 * fp
    assert np.all(d <= ulp), float(np.max(d / ulp))
    frac = float(np.mean(d > 0))
    assert frac < 1e-3, frac
    return frac


def prefill_case(d, B, alpha, gamma, sigma, dtype, gqa=True, rows=None, scale=0.0):
    """Run one prefill sequence on the GPU and through the oracle; compare."""
    q, qx = to_dev(d["q"], dtype)
    k, kx = to_dev(d["k"], dtype)
    v, vx = to_dev(d["v"], dtype)
    qbar = torch.from_numpy(d["qbar"]).cuda()
    L, Hq, D = d["q"].shape
    Hkv = d["k"].shape[1]
    G = Hq // Hkv
    out, lse, ab = ops.attn_prefill(q, k, v, qbar, B, alpha=alpha, gamma=gamma, sigma=sigma,
                                    softmax_scale=scale, enable_gqa=gqa, return_lse=True,
                                    return_active_blocks=True)
    kb = ops.summarize(k, qbar, B)
    torch.cuda.synchronize()
    S = -(-L // B)
    rows = list(range(L)) if rows is None else sorted(set(int(r) for r in rows))
    ref = O.prefill(qx, kx, vx, d["qbar"].astype(np.float64), B, alpha, gamma, sigma, gqa,
                    to_bf16=(dtype == "bf16"), scale=(scale if scale > 0 else None), rows=rows,
                    num_slots=S)
    kb_gpu = kb.to(torch.float64).cpu().numpy()
    check_summaries(kb_gpu, ref["kbar"], dtype, kx, B)
    s = scale if scale > 0 else 1.0 / math.sqrt(D)
    om, margin, _ = oracle_mask_on(qx, kb_gpu, B, alpha, gamma, sigma, G, s, rows, S)
    bits = unpack_bits(ab, S)[:, rows, :]
    flips = compare_masks(bits, om, margin, "prefill")
    o = out.to(torch.float64).cpu().numpy()[rows]
    err = float(np.max(np.abs(o - ref["out"])))
    assert err <= TOL[dtype], f"out max-abs {err}"
    le = lse.cpu().numpy().astype(np.float64)[:, rows]
    lerr = float(np.max(np.abs(le - ref["lse"])))
    assert lerr <= LSE_TOL[dtype], f"lse max-abs {lerr}"
    return dict(err=err, lse_err=lerr, flips=flips, bits=bits, ref=ref, out=out, ab=ab)
