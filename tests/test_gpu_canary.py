"""Every entry point writes its outputs and nothing else, and repeats itself.

Through the C ABI, on buffers of our own: each output and the workspace sit
inside a larger allocation whose guard bytes before and after hold a
sentinel pattern, which must be unchanged after the call, and the inputs must
equal their copies.  Shapes have ragged tails (a partial last chunk, decode
lengths of 1, B + 1 and the capacity) so that the boundary tiles run.  Then
run-twice determinism, bit for bit, of the paths that use no atomics: the
decode step, a packed varlen prefill (its work list) and decode top-k
routing.  (The backward adds the dK/dV slices, the bias gradients and dq̄ by
fp32 atomics, whose order the hardware picks; its repeat may differ by one
bf16 unit where a sum lands on a rounding boundary, and dq̄ within 1e-5 of
its largest magnitude.)
"""

import ctypes

import numpy as np
import pytest
import torch

from sparse_hierarchical_attention_dash_amd import _lib as L
from sparse_hierarchical_attention_dash_amd import ops
from sparse_hierarchical_attention_dash_amd import workloads as W

from gpu_helpers import flush, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side; keeps the 256-byte alignment
SENT = 0xA5


class Guarded:
    """An nbytes region inside an allocation with sentinel guard bands."""

    def __init__(self, nbytes, dtype=torch.uint8, shape=None):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * GUARD,), SENT, dtype=torch.uint8, device="cuda")
        raw = self.buf[GUARD:GUARD + self.n]
        self.t = raw.view(dtype).view(shape) if shape is not None else raw

    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:GUARD] == SENT) and np.all(b[GUARD + self.n:] == SENT))


def tensor_out(shape, dtype):
    el = torch.empty((), dtype=dtype).element_size()
    return Guarded(int(np.prod(shape)) * el, dtype, shape)


def assert_guards(what, **bufs):
    torch.cuda.synchronize()
    bad = [k for k, g in bufs.items() if not g.intact()]
    assert not bad, f"{what}: writes outside {bad}"


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def prefill_inputs(L_, Hq=32, Hkv=2, D=128, seed=91):
    d = W.gen_prefill(L_, Hq, Hkv, D, seed=seed)
    q, _ = to_dev(d["q"], "bf16")
    k, _ = to_dev(d["k"], "bf16")
    v, _ = to_dev(d["v"], "bf16")
    qb = torch.from_numpy(d["qbar"]).cuda()
    return q, k, v, qb


def test_prefill_writes_only_outputs():
    flush("canary: prefill")
    T, Hq, Hkv, D, B = 333, 32, 2, 128, 64
    q, k, v, qb = prefill_inputs(T)
    keep = [x.clone() for x in (q, k, v, qb)]
    shape = ops._seq_shape(q, Hq, Hkv, B, None, None)
    lay = L.layout(shape, True)
    out = tensor_out((T, Hq, D), torch.bfloat16)
    lse = tensor_out((Hq, T), torch.float32)
    ab = tensor_out((Hkv, T, lay.mask_words), torch.int64)
    n = L.workspace_size(L.DASH_OP_PREFILL, shape)
    ws = Guarded(n)
    L.check("dash_attn_prefill", L.lib().dash_attn_prefill(
        ctypes.byref(shape), ops._ptr(q), ops._ptr(k), ops._ptr(v), ops._ptr(qb), 1.5, None,
        30.0, 1.0, 0.0, 1, 0, out.ptr(), lse.ptr(), ab.ptr(), ws.ptr(), n, stream()))
    assert_guards("dash_attn_prefill", out=out, lse=lse, active_blocks=ab, workspace=ws)
    for a, b in zip((q, k, v, qb), keep):
        assert torch.equal(a, b)
    # the same results as through the binding (its own buffers)
    o2, l2, a2 = ops.attn_prefill(q, k, v, qb, B, gamma=30.0, return_lse=True,
                                  return_active_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(out.t, o2) and torch.equal(lse.t, l2) and torch.equal(ab.t, a2)


def test_decode_writes_only_outputs_and_repeats():
    flush("canary: decode")
    batch, cap, Hq, Hkv, D, B = 3, 1024, 32, 2, 128, 64
    d = W.gen_decode(batch, cap, Hq, Hkv, D, seed=92)
    q, _ = to_dev(d["q"], "bf16")
    kc = torch.from_numpy(d["k_cache"]).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(d["v_cache"]).to(torch.bfloat16).cuda()
    qbt = torch.from_numpy(d["qbar"]).cuda()
    kb = ops.summarize(kc.view(-1, Hkv, D), qbt, B, max_seqlen=cap).view(batch, cap // B, Hkv, D)
    seq = torch.tensor([1, B + 1, cap], dtype=torch.int32, device="cuda")
    keep = [x.clone() for x in (q, kc, vc, kb, seq)]
    shape = ops.decode_shape(q, kc, B)
    lay = L.layout(L.make_shape(batch, cap, batch * cap, None, Hq, Hkv, D, B, L.DASH_BF16), True)
    n = L.workspace_size(L.DASH_OP_DECODE, shape)
    runs = []
    for _ in range(2):
        out = tensor_out((batch, Hq, D), torch.bfloat16)
        lse = tensor_out((Hq, batch), torch.float32)
        ab = tensor_out((Hkv, batch, lay.mask_words), torch.int64)
        ws = Guarded(n)
        L.check("dash_attn_decode", L.lib().dash_attn_decode(
            ctypes.byref(shape), ops._ptr(q), ops._ptr(kc), ops._ptr(vc), ops._ptr(seq),
            ops._ptr(kb), None, 1.5, 20.0, 1.0, 0.0, 1, 0, out.ptr(), lse.ptr(), ab.ptr(),
            ws.ptr(), n, stream()))
        assert_guards("dash_attn_decode", out=out, lse=lse, active_blocks=ab, workspace=ws)
        runs.append((out.t.clone(), lse.t.clone(), ab.t.clone()))
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b), "decode differs between two runs"
    for a, b in zip((q, kc, vc, kb, seq), keep):
        assert torch.equal(a, b)


def test_prefill_backward_writes_only_outputs():
    flush("canary: prefill backward")
    T, Hq, Hkv, D, B = 333, 32, 2, 128, 64
    q, k, v, qb = prefill_inputs(T, seed=93)
    rng = np.random.default_rng(94)
    do, _ = to_dev(rng.standard_normal((T, Hq, D)).astype(np.float32), "bf16")
    out, lse, _ = ops.attn_prefill(q, k, v, qb, B, gamma=20.0, return_lse=True)
    keep = [x.clone() for x in (q, k, v, qb, out, do, lse)]
    shape = ops._seq_shape(q, Hq, Hkv, B, None, None)
    n = L.workspace_size(L.DASH_OP_PREFILL_BACKWARD, shape)
    runs = []
    for _ in range(2):
        dq = tensor_out((T, Hq, D), torch.bfloat16)
        dk = tensor_out((T, Hkv, D), torch.bfloat16)
        dv = tensor_out((T, Hkv, D), torch.bfloat16)
        dqb = tensor_out((Hkv, D), torch.float32)
        ws = Guarded(n)
        L.check("dash_attn_prefill_backward", L.lib().dash_attn_prefill_backward(
            ctypes.byref(shape), ops._ptr(q), ops._ptr(k), ops._ptr(v), ops._ptr(qb), 1.5, None,
            20.0, 1.0, 0.0, 1, 0, ops._ptr(out), ops._ptr(do), ops._ptr(lse), dq.ptr(),
            dk.ptr(), dv.ptr(), dqb.ptr(), ws.ptr(), n, stream()))
        assert_guards("dash_attn_prefill_backward", dq=dq, dk=dk, dv=dv, dqbar=dqb, workspace=ws)
        runs.append([x.t.float().clone() for x in (dq, dk, dv, dqb)])
    for nm, a, b in zip(("dq", "dk", "dv", "dqbar"), runs[0], runs[1]):
        scale = max(float(a.abs().max()), 1e-30)
        if nm == "dqbar":   # fp32, summed by atomics
            assert float((a - b).abs().max()) <= 1e-5 * scale, (nm, "repeat")
        else:               # bf16: a sum that lands on a rounding boundary may flip one unit
            assert bool(((a - b).abs() <= 2.0 ** -7 * a.abs() + 1e-6 * scale).all()), (nm, "repeat")
    for a, b in zip((q, k, v, qb, out, do, lse), keep):
        assert torch.equal(a, b)


def test_varlen_prefill_and_topk_decode_repeat():
    flush("determinism: varlen prefill, top-k decode routing")
    lens = [300, 64, 1, 517, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, qb = prefill_inputs(int(cu[-1]), seed=95)
    cut = torch.from_numpy(cu).cuda()
    alphas = torch.tensor([1.5, 2.0, 1.25, 1.5, 2.0], dtype=torch.float32, device="cuda")
    kw = dict(gamma=25.0, alpha_per_seq=alphas, cu_seqlens=cut, max_seqlen=max(lens),
              return_lse=True, return_active_blocks=True)
    a = ops.attn_prefill(q, k, v, qb, 64, **kw)
    b = ops.attn_prefill(q, k, v, qb, 64, **kw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), "varlen prefill differs between two runs"
    batch, cap, Hkv, D, B = 3, 1024, 2, 128, 64
    d = W.gen_decode(batch, cap, 32, Hkv, D, seed=96)
    qd, _ = to_dev(d["q"], "bf16")
    kb32 = W.gen_summaries(batch * cap // B, Hkv, D, seed=96).reshape(batch, cap // B, Hkv, D)
    kbd, _ = to_dev(kb32, "bf16")
    seq = torch.tensor([cap, 200, 65], dtype=torch.int32, device="cuda")
    ws = ops.route_topk_decode_workspace(qd, Hkv, B, cap)
    kw = dict(gamma=10.0, decode_seqlens=seq, cache_len=cap, workspace=ws)
    r1 = ops.route_topk(qd, kbd, Hkv, B, 5, **kw)
    r2 = ops.route_topk(qd, kbd, Hkv, B, 5, **kw)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        # bit patterns: the prior's unwritten slots keep the binding's NaN fill
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), "top-k decode routing differs between two runs"
