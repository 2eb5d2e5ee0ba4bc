"""GPU parity of the backward pass against the CPU backward oracle.

Phase 2 alone (dash_attn_sparse_backward) is compared on the GPU's own
routing (mask and log-prior) with the oracle's attention backward.  The GPU
recomputes P from the forward's LSE and rounds P and dS to bf16 for its
products, as the forward rounds P, so each gradient is held to 2e-2 of its
largest magnitude (bf16: 2^-8 relative per rounding, accumulated over up to
a few thousand keys with random signs).
"""

import math

import numpy as np
import pytest
import torch

from oracle import dash_backward as OB
from sparse_hierarchical_attention_dash_amd import ops
from sparse_hierarchical_attention_dash_amd import workloads as W

from gpu_helpers import flush, to_dev, unpack_bits

pytestmark = pytest.mark.gpu

REL = 2e-2


def rel_err(g, o):
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


CASES = [
    # name, L, Hq, Hkv, D, B, alpha, gamma, sigma
    ("g16-d128-b64", 600, 32, 2, 128, 64, 1.5, 30.0, 1.0),
    ("g16-d64-b128", 500, 16, 1, 64, 128, 1.5, 20.0, 1.0),
    ("g32-d128", 400, 32, 1, 128, 64, 2.0, 30.0, 0.5),
    ("g16-ragged", 333, 32, 2, 128, 64, 1.25, 20.0, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_attention_backward(case):
    name, L, Hq, Hkv, D, B, alpha, gamma, sigma = case
    flush(f"attention backward {name}")
    d = W.gen_prefill(L, Hq, Hkv, D, seed=61)
    q, qx = to_dev(d["q"], "bf16")
    k, kx = to_dev(d["k"], "bf16")
    v, vx = to_dev(d["v"], "bf16")
    rng = np.random.default_rng(62)
    do, dox = to_dev(rng.standard_normal((L, Hq, D)).astype(np.float32), "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    kb = ops.summarize(k, qb, B)
    mask, lp, _ = ops.route(q, kb, Hkv, B, alpha=alpha, gamma=gamma, sigma=sigma,
                            log_prior=True)
    out, lse = ops.attn_sparse(q, k, v, mask, lp, B, return_lse=True)
    dq, dk, dv, dbias = ops.attn_sparse_backward(q, k, v, out, do, lse, mask, lp, B)
    torch.cuda.synchronize()
    S = -(-L // B)
    bits = unpack_bits(mask, S)
    lpx = lp.cpu().numpy().astype(np.float64)
    lpx = np.where(bits, lpx, -np.inf)
    ref = OB.attention_backward_rows(qx, kx, vx, bits, lpx, B, 1 / math.sqrt(D), Hq // Hkv, dox)
    errs = {}
    for nm, gt, rt in (("dq", dq, ref["dq"]), ("dk", dk, ref["dk"]), ("dv", dv, ref["dv"])):
        errs[nm] = rel_err(gt.to(torch.float64).cpu().numpy(), rt)
        assert errs[nm] <= REL, (nm, errs[nm])
    gb = dbias.cpu().numpy().astype(np.float64)
    assert np.all(gb[~bits] == 0.0)
    errs["dbias"] = rel_err(gb[bits], ref["dbias"][bits]) if bits.any() else 0.0
    assert errs["dbias"] <= REL, errs["dbias"]
    flush(f"  backward {name}: " + " ".join(f"{k_} {v_:.2e}" for k_, v_ in errs.items()))
