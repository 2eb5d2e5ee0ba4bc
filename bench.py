#!/usr/bin/env python3
"""Benchmark of the DashAttention forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  prefill of the 64K-token planted-needle sequence (32 query / 2 KV heads,
  D = 128, B = 64, bf16, ~75% block sparsity): chunk summaries, alpha-entmax
  routing, sparse attention -- the three launches dash_attn_prefill makes,
  issued here as dash_summarize, dash_route and dash_attn_sparse so that each
  kernel is timed with its own HIP events on the stream it runs on;
  then one decode step for 16 sequences with 128K-token caches (cached
  summaries, ~75% sparsity, split-K): dash_attn_decode.

value  = prefill active TFLOP/s: 4 * D * sum over query heads and rows of
         (B * active routed chunks + diagonal length), counted from the mask
         the step produced, over the whole prefill (all three launches).
decode = microseconds per decode step and per token, and active K/V GB/s.
roofline: the sparse-attention kernel (the dominant one) against the bf16
         MFMA peak; decode against HBM.
cpu_baseline: the float64 NumPy oracle on a sample of the same prefill rows.
Inputs are resident in HBM before the timed region starts.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("prefill TFLOP/s (active) + decode µs/token at 64K–128K, 75% sparsity; "
          "% roofline")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector
PMC_FILE = os.path.join(ROOT, "profiles", "prefill_attn_pmc.json")
KERNEL_SOURCES = ["attn_prefill.hip", "attn_stage.h", "dash_device.h"]
DEC_PMC_FILE = os.path.join(ROOT, "profiles", "decode_attn_pmc.json")
DEC_KERNEL_SOURCES = ["attn_decode.hip", "attn_stage.h", "dash_device.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash(sources=KERNEL_SOURCES):
    """Hash of a kernel's sources with comments and blank space removed: a
    change of code invalidates the stored counters, a comment does not."""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "sparse_hierarchical_attention_dash_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def popcounts(mask_i64):
    """[..., W] int64 words -> [...] number of set bits."""
    a = np.ascontiguousarray(mask_i64).view(np.uint8)
    return np.unpackbits(a, axis=-1).reshape(mask_i64.shape[:-1] + (-1,)).sum(-1)


def prefill_active_flops(pop, B, D, G):
    """pop [Hkv, T] active routed chunks per (KV head, row) of one sequence."""
    T = pop.shape[1]
    diag = (np.arange(T) % B) + 1
    per = B * pop.astype(np.int64) + diag[None, :]
    return 4.0 * D * G * float(per.sum())


def local_positions(cu, T):
    """Position of every packed row inside its own sequence."""
    pos = np.empty(T, dtype=np.int64)
    for a, b in zip(cu[:-1], cu[1:]):
        pos[a:b] = np.arange(b - a)
    return pos


def active_flops_at(pop, pos, B, D, G):
    """pop [Hkv, T] active routed chunks; pos [T] local positions."""
    per = B * pop.astype(np.int64) + ((pos % B) + 1)[None, :]
    return 4.0 * D * G * float(per.sum())


def decode_kv_bytes(popd, seqlens, B, D):
    """Algorithmic bytes of one bf16 decode step: every key and value row the
    new query of each (KV head, sequence) reads, once: the B keys of each
    active chunk (popd [Hkv, batch]) and its own chunk's keys up to itself."""
    diag = ((np.asarray(seqlens, dtype=np.int64) - 1) % B) + 1
    return float(np.sum(B * popd.astype(np.int64) + diag[None, :])) * D * 2 * 2


FULL_CPU_BUDGET_S = 45.0  # a configuration's oracle runs on every row if that fits


def extra_config(name, stream, reps, cpu_rows, do_cpu, full_cpu=False):
    """One more configuration timed as a whole fused dash_attn_prefill
    (summaries, routing and attention), with its active FLOPs, its roofline
    fraction and the oracle timed on a sample of its rows (on every row with
    full_cpu, when the sample's time extrapolates to FULL_CPU_BUDGET_S or
    less)."""
    import torch
    import oracle as O
    from sparse_hierarchical_attention_dash_amd import ops
    from sparse_hierarchical_attention_dash_amd import workloads as W
    d = W.make(name)
    w = d["workload"]
    bf = w.dtype == "bf16"
    conv = (lambda a: torch.from_numpy(a).to(torch.bfloat16)) if bf else torch.from_numpy
    qh, kh, vh = conv(d["q"]), conv(d["k"]), conv(d["v"])
    q, k, v = qh.cuda(), kh.cuda(), vh.cuda()
    qbar = torch.from_numpy(d["qbar"]).cuda()
    T = q.shape[0]
    G = w.Hq // w.Hkv
    kw = {}
    if w.kind == "varlen":
        cu = d["cu_seqlens"]
        kw = dict(cu_seqlens=torch.from_numpy(cu).cuda(), max_seqlen=int(np.diff(cu).max()),
                  alpha_per_seq=torch.from_numpy(d["alphas"]).cuda())
    else:
        cu = np.array([0, T], dtype=np.int64)
    lens = np.diff(cu)
    pos = local_positions(cu, T)
    shp = ops._seq_shape(q, w.Hq, w.Hkv, w.B, kw.get("cu_seqlens"), kw.get("max_seqlen"))
    from sparse_hierarchical_attention_dash_amd import _lib as L
    ws = torch.empty(L.workspace_size(L.DASH_OP_PREFILL, shp), dtype=torch.uint8, device="cuda")
    _, _, ab = ops.attn_prefill(q, k, v, qbar, w.B, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma,
                                return_active_blocks=True, workspace=ws, **kw)
    torch.cuda.synchronize()
    pop = popcounts(ab.cpu().numpy())
    flops = active_flops_at(pop, pos, w.B, w.D, G)
    t = stats(time_reps(stream, lambda: ops.attn_prefill(
        q, k, v, qbar, w.B, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma, workspace=ws, **kw),
        reps, warm=3))
    routable = float(np.sum(pos // w.B)) * w.Hkv
    tfl = flops / (t["median"] * 1e-3) / 1e12
    peak, bound = (PEAK_BF16_TFLOPS, "mfma") if bf else (PEAK_F32_VALU_TFLOPS, "alu")
    r = {"workload": name, "tokens": T, "sequences": int(len(lens)), "dtype": w.dtype,
         "B": w.B, "ms": t, "active_flops": flops, "tflops_at_median": tfl,
         "roofline": {"bound": bound, "peak": peak, "frac": tfl / peak},
         "block_support": float(pop.sum()) / max(routable, 1.0),
         "support_histogram": support_histogram(pop, w.B, pos)}
    if do_cpu:
        # oracle: a stratified sample of rows of every sequence (all of them
        # when the sequence is short), summaries prorated per row; with
        # full_cpu, every row when the sample says that takes at most
        # FULL_CPU_BUDGET_S seconds
        qx = qh.to(torch.float64).numpy()
        kx = kh.to(torch.float64).numpy()
        vx = vh.to(torch.float64).numpy()
        rng = np.random.default_rng(0)
        s = 1.0 / math.sqrt(w.D)
        alphas = d.get("alphas", np.full(len(lens), w.alpha))

        def oracle_pass(all_rows):
            tot_rows, secs, fl = 0, 0.0, 0.0
            per_seq = max(1, cpu_rows // len(lens))
            full = all_rows or T <= cpu_rows
            for si, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
                Ls = int(b - a)
                if full or Ls <= per_seq:
                    rows = list(range(Ls))
                else:
                    edges = np.linspace(0, Ls, per_seq + 1).astype(int)
                    rows = sorted(int(rng.integers(x, max(x + 1, y)))
                                  for x, y in zip(edges[:-1], edges[1:]))
                t0 = time.perf_counter()
                kbar = O.summarize(kx[a:b], d["qbar"], w.B, to_bf16=bf)
                t_sum = time.perf_counter() - t0
                t0 = time.perf_counter()
                m_, lp_, _ = O.route_sequence(qx[a:b], kbar, w.B, float(alphas[si]), w.gamma,
                                              w.sigma, G, s, rows=rows)
                O.attention_rows(qx[a:b], kx[a:b], vx[a:b], m_, lp_, w.B, s, G, rows)
                secs += time.perf_counter() - t0 + t_sum * len(rows) / Ls
                tot_rows += len(rows)
                for i in rows:
                    for h in range(w.Hkv):
                        fl += 4.0 * w.D * G * (w.B * int(m_[h, i].sum()) + (i % w.B) + 1)
            return tot_rows, secs, fl

        tot_rows, secs, fl = oracle_pass(False)
        est_full = secs * flops / max(fl, 1.0)
        if full_cpu and tot_rows < T and est_full <= FULL_CPU_BUDGET_S:
            tot_rows, secs, fl = oracle_pass(True)
        r["cpu"] = {"value": fl / secs / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                    "cpu_model": cpu_model(), "kind": "oracle", "seconds": secs,
                    "extrapolated_full_seconds": secs * flops / max(fl, 1.0),
                    "sample": ("every row (routing + attention in float64 NumPy, and the "
                               "summaries)" if tot_rows == T else
                               f"{tot_rows} stratified rows of {T} (routing + attention in "
                               "float64 NumPy, summaries prorated per row); the full time is "
                               "extrapolated by active FLOPs")}
    return r


def decode_oracle_time(dd, wd):
    """The oracle's decode step (routing of each new token against the cached
    summaries, then attention over its active blocks) for every sequence of
    the batch, in float64 NumPy; the summary cache is built beforehand, as it
    is cached in decode."""
    import torch
    import oracle as O
    secs = 0.0
    for b in range(wd.batch):
        L = int(dd["seqlens"][b])
        kx = torch.from_numpy(dd["k_cache"][b, :L]).to(torch.bfloat16).to(torch.float64).numpy()
        vx = torch.from_numpy(dd["v_cache"][b, :L]).to(torch.bfloat16).to(torch.float64).numpy()
        qx = torch.from_numpy(dd["q"][b]).to(torch.bfloat16).to(torch.float64).numpy()
        kb = O.summarize(kx, dd["qbar"], wd.B, to_bf16=True)
        t0 = time.perf_counter()
        O.decode(qx, kx, vx, kb, L, wd.B, wd.alpha, wd.gamma, wd.sigma)
        secs += time.perf_counter() - t0
    return {"us_per_step": secs * 1e6, "unit": "us/step", "cores": blas_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the whole step: all {wd.batch} sequences (routing + attention, "
                      "float64 NumPy; summary cache built beforehand, untimed)"}


def to_bf16_dev(a):
    import torch
    return torch.from_numpy(a).to(torch.bfloat16).cuda()


def matched_topk(n_rows, target_blocks, copies):
    """The k whose top-k routing activates as many blocks as the entmax
    routing did: copies * sum_i min(k, n_i) closest to target_blocks."""
    n_rows = np.asarray(n_rows, dtype=np.int64)
    best, best_err = 1, None
    for k in range(1, int(n_rows.max(initial=1)) + 1):
        err = abs(copies * float(np.minimum(n_rows, k).sum()) - target_blocks)
        if best_err is None or err < best_err:
            best, best_err = k, err
    return best


def time_it(stream, fn, reps):
    """Mean milliseconds of fn() over reps runs after one warm-up, from HIP
    events on the stream the work is launched on."""
    import torch
    fn()
    a = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    a[0].record(stream)
    for r in range(reps):
        fn()
        a[r + 1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a[r].elapsed_time(a[r + 1]) for r in range(reps)]))


def stats(ms):
    """mean / median / min of a list of milliseconds."""
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min())}


def time_reps(stream, fn, reps, warm=2, before=None):
    """Per-rep milliseconds of fn() from HIP events on its stream; before(),
    when given, runs ahead of every rep outside the timed interval."""
    import torch
    for _ in range(warm):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def measured_peaks(stream):
    """Achievable peaks on this GPU, next to the spec values: the library's
    probes (an MFMA issue loop of the attention kernels' 16x16x32 bf16
    instruction; an HBM read stream of 1 GiB) and, for scale, a large bf16
    GEMM through torch (the vendor BLAS) and a 1 GiB device copy."""
    import ctypes
    import torch
    from sparse_hierarchical_attention_dash_amd import _lib as L
    lib = L.lib()
    sink = torch.empty(256, dtype=torch.float32, device="cuda")
    work = ctypes.c_double(0.0)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def probe(kind, src, nbytes, iters):
        L.check("dash_probe_peak", lib.dash_probe_peak(
            kind, ctypes.c_void_p(0 if src is None else src.data_ptr()), nbytes, iters,
            ctypes.c_void_p(sink.data_ptr()), 1024, ctypes.byref(work), sp))

    probe(0, None, 0, 20000)
    t_m = stats(time_reps(stream, lambda: probe(0, None, 0, 20000), 5, warm=1))
    mfma = work.value / (t_m["min"] * 1e-3) / 1e12
    nb = 1 << 30
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
    t_r = stats(time_reps(stream, lambda: probe(1, buf, nb, 0), 10, warm=2))
    rd = work.value / (t_r["min"] * 1e-3) / 1e9
    dst = torch.empty_like(buf)
    t2 = stats(time_reps(stream, lambda: dst.copy_(buf), 10, warm=3))
    copy = 2.0 * nb / (t2["min"] * 1e-3) / 1e9
    del buf, dst
    n = 8192
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    t = stats(time_reps(stream, lambda: torch.matmul(a, b, out=c), 10, warm=3))
    gemm = 2.0 * n ** 3 / (t["min"] * 1e-3) / 1e12
    del a, b, c
    return {"mfma_bf16_tflops": mfma,
            "mfma_bf16": "dash_probe_peak kind 0: 16x16x32 bf16 MFMA, two chains per wave, "
                         "two waves per SIMD, best of 5",
            "hbm_read_GB_per_s": rd,
            "hbm_read": "dash_probe_peak kind 1: 1 GiB read with 16-byte loads, best of 10",
            "torch_gemm_bf16_tflops": gemm, "torch_gemm": f"torch.matmul {n}x{n}x{n}, best of 10",
            "copy_GB_per_s": copy, "copy": "1 GiB device copy (read + write bytes), best of 10"}


def support_histogram(pop, B, starts=None):
    """Per-(KV head, row) active routed chunks over the rows that have at
    least one routable chunk: percentiles and a log2-binned histogram."""
    T = pop.shape[1]
    pos = np.arange(T) if starts is None else starts
    n = pos // B
    vals = pop[:, n >= 1].ravel()
    if vals.size == 0:
        return None
    edges = [0, 1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048]
    hist, _ = np.histogram(vals, bins=edges)
    rel = (pop[:, n >= 1] / n[None, n >= 1]).ravel()
    return {"bins": edges, "counts": hist.tolist(),
            "percentiles": {str(p): float(np.percentile(vals, p)) for p in (1, 10, 50, 90, 99)},
            "min": int(vals.min()), "max": int(vals.max()), "mean": float(vals.mean()),
            "relative_percentiles": {str(p): float(np.percentile(rel, p))
                                     for p in (1, 10, 50, 90, 99)}}


def graph_time(stream, fn, outs, reps):
    """Mean milliseconds of one replay of fn() captured as a HIP graph (GPU
    time without Python launch gaps).  Two replays are first checked to give
    the eager result bit for bit (outs: the tensors fn writes)."""
    import torch
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(2):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), "graph replay differs from the eager run"
    a = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    a[0].record(stream)
    for r in range(reps):
        g.replay()
        a[r + 1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a[r].elapsed_time(a[r + 1]) for r in range(reps)]))


def cpu_baseline(d, w, gamma, rows_n, seed=0):
    """Time the oracle on a stratified sample of prefill rows; returns the
    oracle's active TFLOP/s on that sample (summaries prorated per row)."""
    import oracle as O
    import torch
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    qx = torch.from_numpy(d["q"]).to(torch.bfloat16).to(torch.float64).numpy()
    kx = torch.from_numpy(d["k"]).to(torch.bfloat16).to(torch.float64).numpy()
    vx = torch.from_numpy(d["v"]).to(torch.bfloat16).to(torch.float64).numpy()
    L = qx.shape[0]
    rng = np.random.default_rng(seed)
    edges = np.linspace(w.B, L, rows_n + 1).astype(int)
    rows = sorted(int(rng.integers(a, max(a + 1, b))) for a, b in zip(edges[:-1], edges[1:]))
    t0 = time.perf_counter()
    kbar = O.summarize(kx, d["qbar"], w.B, to_bf16=True)
    t_sum = time.perf_counter() - t0
    G = w.Hq // w.Hkv
    s = 1.0 / math.sqrt(w.D)
    t0 = time.perf_counter()
    mask, logp, _ = O.route_sequence(qx, kbar, w.B, w.alpha, gamma, w.sigma, G, s, rows=rows)
    O.attention_rows(qx, kx, vx, mask, logp, w.B, s, G, rows)
    t_rows = time.perf_counter() - t0
    t = t_rows + t_sum * len(rows) / L
    flops = 0.0
    for i in rows:
        for h in range(w.Hkv):
            flops += 4.0 * w.D * G * (w.B * int(mask[h, i].sum()) + (i % w.B) + 1)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"{len(rows)} stratified rows of the {L}-token prefill (routing + "
                       f"attention, float64 NumPy) plus their {len(rows)}/{L} share of the "
                       f"chunk summaries; {t:.1f} s of CPU time"),
            "seconds": t}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--prefill", default="prefill_64k_needles")
    ap.add_argument("--decode", default="decode_128k")
    ap.add_argument("--only", choices=["both", "prefill", "decode"], default="both")
    ap.add_argument("--cpu-rows", type=int, default=1536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the dense and top-k comparison timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timings of the other configurations (16K, varlen, tiny)")
    ap.add_argument("--configs", default="tiny_f32,prefill_16k,varlen_mixed")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the "
                         "reference for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: this build has no multi-GPU path, so "
              "--gpus must be 1 (sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_hierarchical_attention_dash_amd import _lib as L
    from sparse_hierarchical_attention_dash_amd import ops
    from sparse_hierarchical_attention_dash_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_ref:
        n = args.copy_ref * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_ref_bytes": n * 4, "reps": 5}))
        return
    L.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    do_pre = args.only in ("both", "prefill")
    do_dec = args.only in ("both", "decode")

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    if do_pre:
        dp = W.make(args.prefill)
        wp = dp["workload"]
        q = to_bf16_dev(dp["q"])
        k = to_bf16_dev(dp["k"])
        v = to_bf16_dev(dp["v"])
        qbar = torch.from_numpy(dp["qbar"]).cuda()
        T = q.shape[0]
        G = wp.Hq // wp.Hkv
        shp = ops._seq_shape(q, wp.Hq, wp.Hkv, wp.B, None, None)
        lay = L.layout(shp)
        kbar = torch.empty((lay.summary_rows, wp.Hkv, wp.D), dtype=torch.bfloat16, device=dev)
        mask = torch.empty((wp.Hkv, T, lay.mask_words), dtype=torch.int64, device=dev)
        logp = torch.empty((wp.Hkv, T, lay.chunk_slots), dtype=torch.float32, device=dev)
        out = torch.empty_like(q)
        ws_route = torch.empty(max(256, L.workspace_size(L.DASH_OP_ROUTE, shp)),
                               dtype=torch.uint8, device=dev)
        ws_sparse = ops.sparse_workspace(q, k, wp.B)
        log(f"prefill inputs {wp.name}: T={T} Hq={wp.Hq} Hkv={wp.Hkv} D={wp.D} B={wp.B} "
            f"({time.time() - t0:.1f}s)")
    if do_dec:
        dd = W.make(args.decode)
        wd = dd["workload"]
        qd = to_bf16_dev(dd["q"])
        kc = to_bf16_dev(dd["k_cache"])
        vc = to_bf16_dev(dd["v_cache"])
        seqlens = torch.from_numpy(dd["seqlens"]).cuda()
        cap = kc.shape[1]
        # the summary cache is built once (summaries of complete chunks are fixed)
        kbar_c = ops.summarize(kc.view(-1, wd.Hkv, wd.D), torch.from_numpy(dd["qbar"]).cuda(),
                               wd.B, max_seqlen=cap).view(wd.batch, cap // wd.B, wd.Hkv, wd.D)
        ws_dec = ops.decode_workspace(qd, kc, wd.B)
        out_d = torch.empty_like(qd)
        ab_d = torch.empty((wd.Hkv, wd.batch, (cap // wd.B + 63) // 64), dtype=torch.int64,
                           device=dev)
        log(f"decode inputs {wd.name}: batch={wd.batch} cache={cap} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    def step(ev):
        if do_pre:
            ev[0].record(stream)
            ops.summarize(k, qbar, wp.B, out=kbar, workspace=ws_route)
            ev[1].record(stream)
            ops.route(q, kbar, wp.Hkv, wp.B, alpha=wp.alpha, gamma=wp.gamma, sigma=wp.sigma,
                      mask_out=mask, log_prior_out=logp, log_prior=True, workspace=ws_route)
            ev[2].record(stream)
            ops.attn_sparse(q, k, v, mask, logp, wp.B, out=out, workspace=ws_sparse)
            ev[3].record(stream)
        if do_dec:
            ev[4].record(stream)
            ops.attn_decode(qd, kc, vc, seqlens, kbar_c, wd.B, alpha=wd.alpha, gamma=wd.gamma,
                            sigma=wd.sigma, workspace=ws_dec, out=out_d)
            ev[5].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    wall0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for e in evs:
        step(e)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop) / args.steps

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": total_ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    config = {"workload": " + ".join(x for x in (args.prefill if do_pre else None,
                                                args.decode if do_dec else None) if x)}
    if do_pre:
        s_sum = stats([e[0].elapsed_time(e[1]) for e in evs])
        s_route = stats([e[1].elapsed_time(e[2]) for e in evs])
        s_attn = stats([e[2].elapsed_time(e[3]) for e in evs])
        s_pre = stats([e[0].elapsed_time(e[3]) for e in evs])
        t_sum, t_route, t_attn = s_sum["mean"], s_route["mean"], s_attn["mean"]
        t_pre = t_sum + t_route + t_attn
        # parity of the staged launches with the fused entry point (untimed)
        out2, _, ab2 = ops.attn_prefill(q, k, v, qbar, wp.B, alpha=wp.alpha, gamma=wp.gamma,
                                        sigma=wp.sigma, return_active_blocks=True)
        torch.cuda.synchronize()
        assert torch.equal(ab2, mask) and torch.equal(out2, out), "staged != fused prefill"
        pop = popcounts(mask.cpu().numpy())
        flops = prefill_active_flops(pop, wp.B, wp.D, G)
        routable = float(np.sum(np.arange(T) // wp.B)) * wp.Hkv
        support = float(pop.sum()) / routable
        tflops = flops / (t_pre * 1e-3) / 1e12
        attn_tflops = flops / (t_attn * 1e-3) / 1e12
        res.update(value=tflops, unit="TFLOP/s")
        traffic = None
        if os.path.exists(PMC_FILE):
            pmc = json.load(open(PMC_FILE))
            if pmc.get("kernel_hash") == kernel_hash() and pmc.get("workload") == wp.name:
                traffic = pmc.get("hbm_bytes_per_launch")
        res["roofline"] = {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                           "traffic": traffic, "kernel": "prefill_attn_ring_kernel<128>",
                           "algorithmic_flops_per_launch": flops,
                           "avg_launch_ms": t_attn}
        config["prefill"] = {"workload": wp.name, "tokens": T, "q_heads": wp.Hq,
                             "kv_heads": wp.Hkv, "head_dim": wp.D, "chunk": wp.B,
                             "alpha": wp.alpha, "gamma": wp.gamma, "sigma": wp.sigma,
                             "needles": wp.needles}
        res["prefill"] = {"ms": t_pre, "summarize_ms": t_sum, "route_ms": t_route,
                          "attention_ms": t_attn, "active_flops": flops,
                          "block_support": support, "block_sparsity": 1.0 - support,
                          "dense_causal_flops": 4.0 * wp.D * wp.Hq * T * (T + 1) / 2,
                          "attention_tflops": attn_tflops,
                          "ms_stats": s_pre, "summarize_ms_stats": s_sum,
                          "route_ms_stats": s_route, "attention_ms_stats": s_attn,
                          "support_histogram": support_histogram(pop, wp.B)}
    if do_dec:
        s_dec = stats([e[4].elapsed_time(e[5]) for e in evs])
        t_dec = s_dec["mean"]
        ops.attn_decode(qd, kc, vc, seqlens, kbar_c, wd.B, alpha=wd.alpha, gamma=wd.gamma,
                        sigma=wd.sigma, workspace=ws_dec, out=out_d)
        # active blocks of the decode step (untimed run returning the mask)
        _, _, abd = ops.attn_decode(qd, kc, vc, seqlens, kbar_c, wd.B, alpha=wd.alpha,
                                    gamma=wd.gamma, sigma=wd.sigma, workspace=ws_dec,
                                    return_active_blocks=True)
        torch.cuda.synchronize()
        popd = popcounts(abd.cpu().numpy())                  # [Hkv, batch]
        sl = dd["seqlens"].astype(np.int64)
        kv_bytes = decode_kv_bytes(popd, sl, wd.B, wd.D)
        gbs = kv_bytes / (t_dec * 1e-3) / 1e9
        routable = float(np.sum((sl - 1) // wd.B)) * wd.Hkv
        dec_traffic = None
        if os.path.exists(DEC_PMC_FILE):
            pmc = json.load(open(DEC_PMC_FILE))
            if (pmc.get("kernel_hash") == kernel_hash(DEC_KERNEL_SOURCES)
                    and pmc.get("workload") == wd.name):
                dec_traffic = pmc.get("hbm_bytes_per_launch")
        # the decode step alone with the last-level cache flushed before every
        # rep: a 512 MiB buffer is read between reps (outside the timed
        # interval), which leaves only its clean lines in the cache (a written
        # buffer would leave dirty lines whose write-back lands in the step)
        flush_buf = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        flush_out = torch.empty((), dtype=torch.int64, device=dev)
        s_fl = stats(time_reps(stream, lambda: ops.attn_decode(
            qd, kc, vc, seqlens, kbar_c, wd.B, alpha=wd.alpha, gamma=wd.gamma, sigma=wd.sigma,
            workspace=ws_dec, out=out_d), 20, warm=3,
            before=lambda: flush_out.copy_(flush_buf.sum(dtype=torch.int64))))
        del flush_buf, flush_out
        res["decode"] = {"us_per_step": t_dec * 1e3, "us_per_token": t_dec * 1e3 / wd.batch,
                         "us_stats": {k_: v_ * 1e3 for k_, v_ in s_dec.items()},
                         "us_stats_flushed": {k_: v_ * 1e3 for k_, v_ in s_fl.items()},
                         "active_kv_bytes": kv_bytes, "GB_per_s": gbs,
                         "block_support": float(popd.sum()) / routable,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                      "traffic": dec_traffic,
                                      "traffic_kernel": "decode_attn_kernel<128, 1>"}}
        config["decode"] = {"workload": wd.name, "batch": wd.batch, "cache_tokens": cap,
                            "q_heads": wd.Hq, "kv_heads": wd.Hkv, "head_dim": wd.D,
                            "chunk": wd.B, "alpha": wd.alpha, "gamma": wd.gamma}
        if not do_pre:
            res.update(value=t_dec * 1e3 / wd.batch, unit="us/token", higher_is_better=False)
    res["config"] = config
    res["wall_s"] = wall
    if not args.no_compare:
        # Comparison modes on the same kernels (untimed for value): dense
        # causal attention -- the attention kernel alone over every chunk with
        # bias 0 (the routing of alpha = 1, sigma = 0, made once, untimed), as a
        # flash-style dense kernel would run -- and top-k routing with k
        # matched to the entmax routing's active block count, as a whole step
        # (summaries, routing, attention).
        log("comparison modes ...")
        cmp = {}
        reps = 3
        if do_pre:
            n_i = np.arange(T) // wp.B
            kp = matched_topk(n_i, float(pop.sum()), wp.Hkv)
            m2 = torch.empty_like(mask)
            l2 = torch.empty_like(logp)
            ops.route(q, kbar, wp.Hkv, wp.B, alpha=1.0, gamma=wp.gamma, sigma=0.0,
                      mask_out=m2, log_prior_out=l2, log_prior=True, workspace=ws_route)

            def dense_pre():
                ops.attn_sparse(q, k, v, m2, l2, wp.B, out=out, workspace=ws_sparse)

            def topk_pre():
                ops.summarize(k, qbar, wp.B, out=kbar, workspace=ws_route)
                ops.route_topk(q, kbar, wp.Hkv, wp.B, kp, gamma=wp.gamma, mask_out=m2,
                               log_prior_out=l2, workspace=ws_route)
                ops.attn_sparse(q, k, v, m2, l2, wp.B, out=out, workspace=ws_sparse)

            pop_dense = popcounts(m2.cpu().numpy())
            t_dense = time_it(stream, dense_pre, reps)
            assert np.array_equal(pop_dense, np.broadcast_to(n_i, pop_dense.shape))
            dense_flops = prefill_active_flops(pop_dense, wp.B, wp.D, G)
            t_topk = time_it(stream, topk_pre, reps)
            pop_k = popcounts(m2.cpu().numpy())
            t_topk_route = time_it(stream, lambda: ops.route_topk(
                q, kbar, wp.Hkv, wp.B, kp, gamma=wp.gamma, mask_out=m2, log_prior_out=l2,
                workspace=ws_route), reps)
            # estimate_diagonal: the own-chunk estimates join every row's routing
            kd = torch.empty_like(k)

            def diag_pre():
                ops.summarize(k, qbar, wp.B, out=kbar, workspace=ws_route)
                ops.summarize_diagonal(k, qbar, wp.B, out=kd)
                ops.route(q, kbar, wp.Hkv, wp.B, alpha=wp.alpha, gamma=wp.gamma, sigma=wp.sigma,
                          mask_out=m2, log_prior_out=l2, log_prior=True, workspace=ws_route,
                          kdiag=kd)
                ops.attn_sparse(q, k, v, m2, l2, wp.B, out=out, workspace=ws_sparse)

            t_diag = time_it(stream, diag_pre, reps)
            pop_dg = popcounts(m2.cpu().numpy())
            flops_dg = prefill_active_flops(pop_dg, wp.B, wp.D, G)
            t_dsum = time_it(stream, lambda: ops.summarize_diagonal(k, qbar, wp.B, out=kd), reps)
            t_droute = time_it(stream, lambda: ops.route(
                q, kbar, wp.Hkv, wp.B, alpha=wp.alpha, gamma=wp.gamma, sigma=wp.sigma,
                mask_out=m2, log_prior_out=l2, log_prior=True, workspace=ws_route, kdiag=kd), reps)
            # backward: the whole prefill backward (routing recomputed, attention,
            # prior, entmax routing and summaries), and, for scale, phase 2's
            # backward alone over every chunk (dense causal attention backward)
            dout = torch.randn_like(q)
            o_b, lse_b, _ = ops.attn_prefill(q, k, v, qbar, wp.B, alpha=wp.alpha, gamma=wp.gamma,
                                             sigma=wp.sigma, return_lse=True)
            ws_pb = torch.empty(L.workspace_size(L.DASH_OP_PREFILL_BACKWARD, shp),
                                dtype=torch.uint8, device=dev)
            t_bwd = time_it(stream, lambda: ops.attn_prefill_backward(
                q, k, v, qbar, o_b, dout, lse_b, wp.B, alpha=wp.alpha, gamma=wp.gamma,
                sigma=wp.sigma, workspace=ws_pb), reps)
            # with estimate_diagonal: its own forward's output and LSE
            o_g, lse_g, _ = ops.attn_prefill(q, k, v, qbar, wp.B, alpha=wp.alpha, gamma=wp.gamma,
                                             sigma=wp.sigma, return_lse=True,
                                             estimate_diagonal=True)
            t_bwd_diag = time_it(stream, lambda: ops.attn_prefill_backward(
                q, k, v, qbar, o_g, dout, lse_g, wp.B, alpha=wp.alpha, gamma=wp.gamma,
                sigma=wp.sigma, estimate_diagonal=True, workspace=ws_pb), reps)
            del o_g, lse_g
            ops.route(q, kbar, wp.Hkv, wp.B, alpha=1.0, gamma=wp.gamma, sigma=0.0,
                      mask_out=m2, log_prior_out=l2, log_prior=True, workspace=ws_route)
            o_d, lse_d = ops.attn_sparse(q, k, v, m2, l2, wp.B, return_lse=True)
            t_dbwd = time_it(stream, lambda: ops.attn_sparse_backward(
                q, k, v, o_d, dout, lse_d, m2, l2, wp.B), reps)
            del ws_pb, o_b, lse_b, o_d, lse_d, dout
            # the usual count of an attention backward: 2.5 times the forward's
            # products (S, dP, dV, dQ, dK; S is recomputed)
            cmp["backward"] = {
                "dash_ms": t_bwd, "dash_estimate_diagonal_ms": t_bwd_diag,
                "dense_attention_ms": t_dbwd,
                "dash_tflops": 2.5 * flops / (t_bwd * 1e-3) / 1e12,
                "dense_tflops": 2.5 * dense_flops / (t_dbwd * 1e-3) / 1e12,
                "speedup_vs_dense": t_dbwd / t_bwd}
            cmp["estimate_diagonal"] = {
                "prefill_ms": t_diag, "diag_summary_ms": t_dsum, "route_ms": t_droute,
                "active_blocks": int(pop_dg.sum()), "tflops": flops_dg / (t_diag * 1e-3) / 1e12}
            cmp["prefill"] = {
                "dash_ms": t_pre,
                "dense_ms": t_dense, "dense_flops": dense_flops,
                "dense_tflops": dense_flops / (t_dense * 1e-3) / 1e12,
                "speedup_vs_dense": t_dense / t_pre,
                "topk_k": kp, "topk_ms": t_topk, "topk_route_ms": t_topk_route,
                "topk_active_blocks": int(pop_k.sum()), "dash_active_blocks": int(pop.sum()),
                "speedup_vs_topk": t_topk / t_pre}
        if do_dec:
            n_b = (dd["seqlens"].astype(np.int64) - 1) // wd.B
            kd = matched_topk(n_b, float(popd.sum()), wd.Hkv)
            ws_ds = ops.decode_sparse_workspace(qd, kc, wd.B)
            ws_rd = ops.route_topk_decode_workspace(qd, wd.Hkv, wd.B, cap)
            md = torch.empty_like(abd)
            ld = torch.empty((wd.Hkv, wd.batch, cap // wd.B), dtype=torch.float32, device=dev)
            # k at least n: every routable chunk, bias 0
            md_all, ld_all = ops.route_topk(qd, kbar_c, wd.Hkv, wd.B, cap // wd.B,
                                            gamma=wd.gamma, decode_seqlens=seqlens,
                                            cache_len=cap, workspace=ws_rd)
            torch.cuda.synchronize()
            assert np.array_equal(popcounts(md_all.cpu().numpy()),
                                  np.broadcast_to(n_b, (wd.Hkv, wd.batch)))

            def dense_dec():
                ops.attn_decode_sparse(qd, kc, vc, seqlens, md_all, ld_all, wd.B,
                                       workspace=ws_ds, out=out_d)

            def topk_dec():
                ops.route_topk(qd, kbar_c, wd.Hkv, wd.B, kd, gamma=wd.gamma,
                               decode_seqlens=seqlens, cache_len=cap, mask_out=md,
                               log_prior_out=ld, workspace=ws_rd)
                ops.attn_decode_sparse(qd, kc, vc, seqlens, md, ld, wd.B, workspace=ws_ds,
                                       out=out_d)

            def dash_dec():
                ops.attn_decode(qd, kc, vc, seqlens, kbar_c, wd.B, alpha=wd.alpha,
                                gamma=wd.gamma, sigma=wd.sigma, workspace=ws_dec, out=out_d)

            t_dd = time_it(stream, dense_dec, 5)
            t_kd = time_it(stream, topk_dec, 5)
            # the same three steps as graph replays: GPU time alone
            g_dash = graph_time(stream, dash_dec, [out_d], 10)
            g_dense = graph_time(stream, dense_dec, [out_d], 10)
            g_topk = graph_time(stream, topk_dec, [out_d, md], 10)
            # decode-cache upkeep: append each sequence's token at seqlens-1 (its
            # own row again, so the caches keep their contents) before the step
            ar = torch.arange(wd.batch, device=dev)
            last = (seqlens.long() - 1)
            kn = kc[ar, last].contiguous()
            vn = vc[ar, last].contiguous()
            qbar_d = torch.from_numpy(dd["qbar"]).cuda()

            def append():
                ops.cache_append(kn, vn, seqlens, qbar_d, kc, vc, kbar_c, wd.B)

            def append_dec():
                append()
                dash_dec()

            t_app = time_it(stream, append, 10)
            g_app = graph_time(stream, append_dec, [out_d], 10)

            # the same append + step as one fused call (dash_attn_decode_append)
            def fused_dec():
                ops.attn_decode_append(qd, kn, vn, kc, vc, seqlens, kbar_c, qbar_d, wd.B,
                                       alpha=wd.alpha, gamma=wd.gamma, sigma=wd.sigma,
                                       workspace=ws_dec, out=out_d)

            t_app_dec = time_it(stream, append_dec, 10)
            t_fused = time_it(stream, fused_dec, 10)
            g_fused = graph_time(stream, fused_dec, [out_d], 10)

            def diag_dec():
                ops.attn_decode(qd, kc, vc, seqlens, kbar_c, wd.B, alpha=wd.alpha,
                                gamma=wd.gamma, sigma=wd.sigma, workspace=ws_dec, out=out_d,
                                estimate_diagonal=True, qbar=qbar_d)

            t_ddiag = time_it(stream, diag_dec, 5)
            g_ddiag = graph_time(stream, diag_dec, [out_d], 10)
            cmp.setdefault("estimate_diagonal", {}).update(
                decode_us=t_ddiag * 1e3, decode_graph_us=g_ddiag * 1e3)
            dense_bytes = float(np.sum(wd.B * n_b + ((dd["seqlens"] - 1) % wd.B) + 1)) \
                * wd.Hkv * wd.D * 2 * 2
            cmp["decode"] = {
                "dash_us": t_dec * 1e3, "dense_us": t_dd * 1e3,
                "dense_GB_per_s": dense_bytes / (t_dd * 1e-3) / 1e9,
                "speedup_vs_dense": t_dd / t_dec,
                "topk_k": kd, "topk_us": t_kd * 1e3,
                "topk_active_blocks": int(popcounts(md.cpu().numpy()).sum()),
                "dash_active_blocks": int(popd.sum()),
                "speedup_vs_topk": t_kd / t_dec,
                "graph_us": {"dash": g_dash * 1e3, "dense": g_dense * 1e3,
                             "topk": g_topk * 1e3},
                "append_us": t_app * 1e3, "graph_us_append_and_step": g_app * 1e3,
                "append_then_step_us": t_app_dec * 1e3, "fused_append_step_us": t_fused * 1e3,
                "graph_us_fused_append_step": g_fused * 1e3,
                "graph_speedup_vs_dense": g_dense / g_dash,
                "graph_speedup_vs_topk": g_topk / g_dash}
        res["compare"] = cmp
    if not args.no_configs and do_pre:
        log("other configurations ...")
        res["configs"] = {}
        for name in [x for x in args.configs.split(",") if x]:
            log(f"  {name}")
            # the small fixed-length configurations' oracle in full, the
            # varlen pack's on a sample
            res["configs"][name] = extra_config(name, stream, 20, 256,
                                                not args.no_cpu_baseline,
                                                full_cpu=name in ("tiny_f32", "prefill_16k"))
    log("measured peaks ...")
    res["peaks_measured"] = measured_peaks(stream)
    if "roofline" in res:
        res["roofline"]["frac_of_measured_peak"] = (
            res["roofline"]["achieved"] / res["peaks_measured"]["mfma_bf16_tflops"])
    if do_dec:
        res["decode"]["roofline"]["frac_of_measured_peak"] = (
            res["decode"]["roofline"]["achieved"] / res["peaks_measured"]["hbm_read_GB_per_s"])
    if do_pre and not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(dp, wp, wp.gamma, args.cpu_rows)
        res["cpu_baseline"]["cpu_model"] = cpu_model()
    else:
        res["cpu_baseline"] = None
    if do_dec and not args.no_cpu_baseline:
        log("cpu baseline, decode (oracle) ...")
        res["cpu_baseline_decode"] = decode_oracle_time(dd, wd)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
