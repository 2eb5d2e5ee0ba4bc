"""Seeded synthetic inputs for the DashAttention forward path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  The tests, the benchmark and the oracle checks all
take their inputs from here, so the HIP library and the oracle always see the
same bits.  Arrays are float32 NumPy; callers that run in bfloat16 round them
once (round to nearest even) and hand the rounded values to both sides.

The shapes follow an 8B-class long-context setting: 32 query heads sharing
2 KV heads (GQA group of 16), head dim 128, chunk size 64 or 128, and about
75% block sparsity.  The pages evaluate on RULER/HELMET with MiniCPM-4
weights, which are not available here; these synthetic inputs stand in for
them and reproduce no item of those suites.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One named synthetic configuration."""

    name: str
    kind: str                  # "prefill" | "varlen" | "decode"
    dtype: str                 # "f32" | "bf16"
    Hq: int
    Hkv: int
    D: int
    B: int
    alpha: float
    gamma: float
    sigma: float
    seed: int
    seqlen: int = 0            # prefill: sequence length; decode: cache length
    batch: int = 1
    needles: int = 0           # planted chunks per KV head
    needle_mag: float = 3.0
    varlen_n: int = 0
    varlen_lo: int = 0
    varlen_hi: int = 0
    varlen_alphas: tuple = field(default_factory=tuple)
    cluster_frac: float = 0.0
    n_centroids: int = 0
    qbar_std: float = 0.1


# gamma is a workload parameter: it was chosen (by sampling rows through the
# oracle routing, see oracle/calibrate_gamma.py) so that the mean block
# support on the GQA-shared mask is about 25% of the routable chunks.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "prefill", "f32", 1, 1, 64, 64, 1.5, 1.0,
                         1.0, seed=1, seqlen=512),
    "prefill_16k": Workload("prefill_16k", "prefill", "bf16", 32, 2, 128, 64,
                            1.5, 35.33, 1.0, seed=2, seqlen=16384),
    "prefill_64k_needles": Workload("prefill_64k_needles", "prefill", "bf16",
                                    32, 2, 128, 64, 1.5, 6.290, 1.0, seed=3,
                                    seqlen=65536, needles=32, needle_mag=3.0),
    "decode_128k": Workload("decode_128k", "decode", "bf16", 32, 2, 128, 64,
                            1.5, 5.588, 1.0, seed=4, seqlen=131072, batch=16),
    "varlen_mixed": Workload("varlen_mixed", "varlen", "bf16", 32, 2, 128, 128,
                             1.5, 6.046, 1.0, seed=5, varlen_n=8,
                             varlen_lo=4096, varlen_hi=131072,
                             varlen_alphas=(1.25, 1.5, 2.0), cluster_frac=0.2,
                             n_centroids=16),
}


def normal(rng, shape, std=1.0):
    """float32 N(0, std^2) draws."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def gen_prefill(L, Hq, Hkv, D, seed, B=64, needles=0, needle_mag=3.0,
                qbar_std=0.1):
    """One sequence: Q, K, V ~ N(0, 1), q_bar ~ N(0, qbar_std^2).

    ``needles`` > 0 plants that many chunks per KV head whose keys are all
    shifted by needle_mag times a unit vector pointing along a randomly
    chosen later query (a query row after the chunk, a query head of the
    group), so that some queries concentrate their routing on few chunks.
    Returns dict(q [L,Hq,D], k [L,Hkv,D], v [L,Hkv,D], qbar [Hkv,D]).
    """
    rng = np.random.default_rng(seed)
    q = normal(rng, (L, Hq, D))
    k = normal(rng, (L, Hkv, D))
    v = normal(rng, (L, Hkv, D))
    qbar = normal(rng, (Hkv, D), qbar_std)
    G = Hq // Hkv
    C = L // B
    planted = []
    if needles and C >= 2:
        for h in range(Hkv):
            for _ in range(needles):
                c = int(rng.integers(0, C - 1))
                lo = (c + 1) * B + 1
                if lo >= L:
                    continue
                r = int(rng.integers(lo, L))
                qh = h * G + int(rng.integers(0, G))
                d = q[r, qh].astype(np.float64)
                d = d / np.linalg.norm(d)
                k[c * B:(c + 1) * B, h, :] += np.float32(needle_mag) * d.astype(np.float32)
                planted.append((h, c, r, qh))
    return dict(q=q, k=k, v=v, qbar=qbar, planted=planted)


def varlen_lengths(n, lo, hi, seed):
    """n lengths drawn log-uniform in [lo, hi] (floored)."""
    rng = np.random.default_rng(seed)
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), n))).astype(np.int64)


def gen_varlen(lengths, Hq, Hkv, D, seed, B=128, cluster_frac=0.2,
               n_centroids=16, qbar_std=0.1):
    """Packed sequences.  Keys: a fraction ``cluster_frac`` of the chunks are
    'clustered' (every key = one of ``n_centroids`` N(0, I) centroids plus
    0.5 * N(0, I)), the rest N(0, I); Q, V ~ N(0, I).
    Returns dict(q, k, v [T, H, D], qbar, cu_seqlens int32 [n+1]).
    """
    rng = np.random.default_rng(seed + 1000)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = normal(rng, (T, Hq, D))
    k = normal(rng, (T, Hkv, D))
    v = normal(rng, (T, Hkv, D))
    qbar = normal(rng, (Hkv, D), qbar_std)
    cents = normal(rng, (Hkv, n_centroids, D))
    for s in range(len(lengths)):
        a, L = int(cu[s]), int(lengths[s])
        for c in range(L // B):
            if rng.random() < cluster_frac:
                for h in range(Hkv):
                    j = int(rng.integers(0, n_centroids))
                    k[a + c * B:a + (c + 1) * B, h, :] = (
                        cents[h, j][None, :] + normal(rng, (B, D), 0.5))
    return dict(q=q, k=k, v=v, qbar=qbar, cu_seqlens=cu)


def gen_decode(batch, cap, Hq, Hkv, D, seed, qbar_std=0.1):
    """Decode inputs: one new query per sequence, a contiguous K/V cache of
    ``cap`` tokens per sequence (the new token's key/value already written at
    position seqlen - 1), all ~ N(0, 1).
    Returns dict(q [batch,Hq,D], k_cache/v_cache [batch,cap,Hkv,D], qbar).
    """
    rng = np.random.default_rng(seed)
    q = normal(rng, (batch, Hq, D))
    qbar = normal(rng, (Hkv, D), qbar_std)
    k = np.empty((batch, cap, Hkv, D), dtype=np.float32)
    v = np.empty((batch, cap, Hkv, D), dtype=np.float32)
    for b in range(batch):
        k[b] = normal(rng, (cap, Hkv, D))
        v[b] = normal(rng, (cap, Hkv, D))
    return dict(q=q, k_cache=k, v_cache=v, qbar=qbar)


def gen_summaries(C, Hkv, D, seed, std=0.125):
    """Stand-alone summary tensors [C, Hkv, D] ~ N(0, std^2), used to drive
    the routing stage on its own (std 1/8 is the spread of a mean of 64
    unit-variance keys)."""
    rng = np.random.default_rng(seed + 2000)
    return normal(rng, (C, Hkv, D), std)


def make(name, **overrides):
    """Materialise a named workload's inputs (float32 NumPy)."""
    w = WORKLOADS[name]
    if overrides:
        w = Workload(**{**w.__dict__, **overrides})
    if w.kind == "prefill":
        d = gen_prefill(w.seqlen, w.Hq, w.Hkv, w.D, w.seed, w.B, w.needles,
                        w.needle_mag, w.qbar_std)
    elif w.kind == "varlen":
        lens = varlen_lengths(w.varlen_n, w.varlen_lo, w.varlen_hi, w.seed)
        d = gen_varlen(lens, w.Hq, w.Hkv, w.D, w.seed, w.B, w.cluster_frac,
                       w.n_centroids, w.qbar_std)
        d["alphas"] = np.array([w.varlen_alphas[i % len(w.varlen_alphas)]
                                for i in range(w.varlen_n)], dtype=np.float32)
    else:
        d = gen_decode(w.batch, w.seqlen, w.Hq, w.Hkv, w.D, w.seed, w.qbar_std)
        d["seqlens"] = np.full(w.batch, w.seqlen, dtype=np.int32)
    d["workload"] = w
    return d


def gen_routing(Hkv, L, B, density, seed, lo=-6.0):
    """A synthetic routing for driving the attention stage on its own: each
    routable chunk c < floor(i/B) of each (KV head, position) is active with
    probability ``density``; active chunks get a bias drawn uniformly in
    [lo, 0], inactive ones -inf.  Returns (mask bool [Hkv, L, S],
    log_prior float32 [Hkv, L, S]) with S = ceil(L / B)."""
    rng = np.random.default_rng(seed + 3000)
    S = -(-L // B)
    n = (np.arange(L) // B)[None, :, None]
    mask = (rng.random((Hkv, L, S)) < density) & (np.arange(S)[None, None, :] < n)
    lp = rng.uniform(lo, 0.0, (Hkv, L, S)).astype(np.float32)
    lp[~mask] = -np.inf
    return mask, lp
