"""Pick the routing temperature gamma of each synthetic workload.

Test infrastructure: run by hand (``python -m oracle.calibrate_gamma``); it
prints the gamma that gives the target mean block support on the GQA-shared
mask, measured through the oracle's routing on a seeded sample of rows.  The
printed values are copied into the workload table as workload parameters
(they are not expected results of anything).

Sparsity is 1 - sum_{h,i} |M_{h,i}| / sum_{h,i} n_i over the sampled rows,
n_i = floor(i / B) routable chunks, the diagonal chunk excluded.
"""

from __future__ import annotations

import argparse
import math

import numpy as np

from . import dash_oracle as O


def calibrate(name, target=0.25, nrows=96, seed=123, lo=1.0, hi=200.0, iters=14):
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from sparse_hierarchical_attention_dash_amd import workloads as W

    d = W.make(name)
    w = d["workload"]
    G = w.Hq // w.Hkv
    scale = 1.0 / math.sqrt(w.D)
    rng = np.random.default_rng(seed)
    if w.kind == "prefill":
        q = d["q"].astype(np.float64)
        kbar = O.summarize(d["k"], d["qbar"], w.B, to_bf16=(w.dtype == "bf16"))
        rows = [(int(i), 0, w.alpha) for i in rng.integers(w.B, w.seqlen, nrows)]
        kb = {0: kbar}
        getkb = lambda base: kb[0]
    elif w.kind == "decode":
        # one query row per sequence; rows are keyed by their sequence
        nb = min(w.batch, 4)
        kbs = {b: O.summarize(d["k_cache"][b], d["qbar"], w.B, to_bf16=True)
               for b in range(nb)}
        q = np.zeros((nb, w.Hq, w.D))
        q[:] = d["q"][:nb]
        rows = [(w.seqlen - 1, b, w.alpha) for b in range(nb)]
        getkb = lambda base: kbs[base]
    else:
        cu = d["cu_seqlens"]
        q = d["q"].astype(np.float64)
        kbs = {}
        rows = []
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            kbs[a] = O.summarize(d["k"][a:b], d["qbar"], w.B, to_bf16=True)
            for i in rng.integers(a + w.B, b, max(4, nrows // (len(cu) - 1))):
                rows.append((int(i), a, float(d["alphas"][s])))
        getkb = lambda base: kbs[base]

    def frac(gamma):
        on = tot = 0
        for i, base, al in rows:
            local = i if w.kind == "decode" else i - base
            n = local // w.B
            if n == 0:
                continue
            kb = getkb(base)
            qi = q[base] if w.kind == "decode" else q[i]
            for h in range(w.Hkv):
                r = O.route_position(qi[h * G:(h + 1) * G], kb[:n, h], al,
                                     gamma, scale)
                on += int(r["mask"].sum())
                tot += n
        return on / max(tot, 1)

    a, b = math.log(lo), math.log(hi)
    for _ in range(iters):
        m = 0.5 * (a + b)
        f = frac(math.exp(m))
        if f > target:
            a = m
        else:
            b = m
    g = math.exp(0.5 * (a + b))
    return g, frac(g)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("names", nargs="*", default=["prefill_16k", "prefill_64k_needles",
                                                 "decode_128k", "varlen_mixed"])
    ap.add_argument("--target", type=float, default=0.25)
    args = ap.parse_args()
    for n in args.names:
        g, f = calibrate(n, args.target)
        print(f"{n}: gamma={g:.4f} support={f:.4f}", flush=True)


if __name__ == "__main__":
    main()
