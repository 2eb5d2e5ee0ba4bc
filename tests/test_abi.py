"""C ABI checks that need no GPU: the library loads, exports every function
include/dash.h declares, and rejects every invalid argument with the right
status before any HIP call (nothing is launched on these paths)."""

import ctypes
import math
import os
import re

import pytest

from sparse_hierarchical_attention_dash_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash.h")

A = 0x10000          # a 256-byte aligned stand-in address, never dereferenced
BF16, F32 = L.DASH_BF16, L.DASH_F32


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:dash_status|size_t|const char\*|int)\s+(dash_\w+)\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libdash.so is not built (run __graft_entry__.build())")
    return L.lib()


def shape(T=256, Hq=32, Hkv=2, D=128, B=64, dtype=BF16, num_seqs=1, max_seqlen=None, cu=None):
    return L.make_shape(num_seqs, T if max_seqlen is None else max_seqlen, T, cu, Hq, Hkv, D,
                        B, dtype)


_DEFAULT = object()


def prefill(lib, s, *, q=A, k=A, v=A, qbar=A, out=A, alpha=1.5, gamma=1.0, sigma=1.0,
            scale=0.0, gqa=1, diag=0, ws=_DEFAULT, ws_bytes=None):
    need = L.workspace_size(L.DASH_OP_PREFILL, s)
    ws = A if ws is _DEFAULT else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    return lib.dash_attn_prefill(ctypes.byref(s), q, k, v, qbar, alpha, None, gamma, sigma,
                                 scale, gqa, diag, out, None, None, ws, ws_bytes, None)


def test_header_declares_the_four_operations():
    names = declared_functions()
    for f in ("dash_summarize", "dash_route", "dash_attn_prefill", "dash_attn_decode"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(L.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.dash_abi_version() == 3
    for code, text in ((0, "ok"), (1, "invalid argument"), (2, "unsupported configuration"),
                       (3, "workspace too small"), (4, "HIP launch error")):
        assert L.status_string(code) == text
    assert L.status_string(99) == "unknown status"


def test_layout_and_workspace_sizes(lib):
    s = shape(T=1000, B=64)
    lay = L.layout(s)
    assert (lay.summary_rows, lay.chunk_slots, lay.mask_words, lay.group_size) == (15, 16, 1, 16)
    s = shape(T=131072, B=64)
    lay = L.layout(s)
    assert (lay.chunk_slots, lay.mask_words) == (2048, 32)
    # prefill workspace holds summaries, a mask, the dense log-prior, (bf16,
    # group >= 16) V transposed into 64-padded columns, the own-chunk
    # estimates of estimate_diagonal, and (bf16, group 16 or 32) one flag per
    # row and KV head of the streaming routing (each head's row of flags
    # padded to 16 bytes)
    T, Hkv, D, W, C = 1000, 2, 128, 1, 16
    need = L.workspace_size(L.DASH_OP_PREFILL, shape(T=T))
    flags = (T + 15) // 16 * 16 * Hkv
    parts = [(T // 64) * Hkv * D * 2, Hkv * T * W * 8, Hkv * T * C * 4, Hkv * D * (T + 64) * 2,
             T * Hkv * D * 2, flags]
    assert need == sum((p + 255) // 256 * 256 for p in parts)
    assert L.workspace_size(L.DASH_OP_SUMMARIZE, shape()) == 0
    # route: the varlen prefix arrays, then the row flags (256 rows x 2 heads)
    assert L.workspace_size(L.DASH_OP_ROUTE, shape(cu=A, num_seqs=3)) == 512 + 512
    assert L.workspace_size(L.DASH_OP_ROUTE, shape(Hq=8)) == 0   # group of 4: one row per workgroup
    assert L.workspace_size(L.DASH_OP_DECODE, shape(T=4, num_seqs=4, max_seqlen=4096)) > 0
    assert L.workspace_size(L.DASH_OP_PREFILL, shape(D=96)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), L.DASH_ERR_UNSUPPORTED),
    (dict(B=32), L.DASH_ERR_UNSUPPORTED),
    (dict(dtype=7), L.DASH_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=2), L.DASH_ERR_UNSUPPORTED),          # bf16 group of 3
    (dict(Hq=48, Hkv=1), L.DASH_ERR_UNSUPPORTED),         # bf16 group of 48
    (dict(Hq=64, Hkv=1), L.DASH_ERR_UNSUPPORTED),         # bf16 groups above 32
    (dict(Hq=256, Hkv=1), L.DASH_ERR_UNSUPPORTED),
    (dict(Hq=5, Hkv=2), L.DASH_ERR_INVALID_ARGUMENT),
    (dict(T=200000, B=64), L.DASH_ERR_UNSUPPORTED),       # more than 2048 chunk slots
])
def test_prefill_rejects_bad_shapes(lib, kw, status):
    assert prefill(lib, shape(**kw)) == status


def test_prefill_rejects_bad_arguments(lib):
    s = shape()
    assert lib.dash_attn_prefill(None, A, A, A, A, 1.5, None, 1.0, 1.0, 0.0, 1, 0, A, None,
                                 None, A, 1 << 30, None) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, q=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, out=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, qbar=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, k=A + 2) == L.DASH_ERR_INVALID_ARGUMENT      # misaligned
    assert prefill(lib, s, alpha=0.5) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, alpha=3.0) == L.DASH_ERR_UNSUPPORTED
    assert prefill(lib, s, alpha=math.nan) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, gamma=0.0) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, gamma=math.inf) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, sigma=-1.0) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, scale=math.nan) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, gqa=0) == L.DASH_ERR_INVALID_ARGUMENT       # Hq != Hkv
    need = L.workspace_size(L.DASH_OP_PREFILL, s)
    assert prefill(lib, s, ws_bytes=need - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert prefill(lib, s, ws=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert prefill(lib, s, ws=A + 16) == L.DASH_ERR_INVALID_ARGUMENT   # not 256-aligned
    bad = shape(T=100, num_seqs=2, max_seqlen=64)                       # T != num_seqs*max
    assert prefill(lib, bad) == L.DASH_ERR_INVALID_ARGUMENT


def test_empty_input_is_a_no_op(lib):
    # zero tokens: valid, nothing to do, no HIP call is made
    assert prefill(lib, shape(T=0, num_seqs=0, max_seqlen=0)) == L.DASH_OK
    s = shape(T=0, num_seqs=0, max_seqlen=0)
    assert lib.dash_summarize(ctypes.byref(s), A, A, A, None, 0, None) == L.DASH_OK
    assert lib.dash_route(ctypes.byref(s), A, A, None, 1.5, None, 1.0, 1.0, 0.0, 1, A, None,
                          None, None, 0, None) == L.DASH_OK
    assert lib.dash_summarize_diagonal(ctypes.byref(s), A, A, A, None) == L.DASH_OK


def test_route_and_summarize_checks(lib):
    s = shape()
    n = L.workspace_size(L.DASH_OP_ROUTE, s)   # the streaming routing's row flags
    assert n == 512
    assert lib.dash_route(ctypes.byref(s), A, A, None, 1.5, None, 1.0, 1.0, 0.0, 1, None, None,
                          None, A, n, None) == L.DASH_ERR_INVALID_ARGUMENT   # mask is required
    assert lib.dash_route(ctypes.byref(s), A, A, None, 2.5, None, 1.0, 1.0, 0.0, 1, A, None,
                          None, A, n, None) == L.DASH_ERR_UNSUPPORTED
    assert lib.dash_route(ctypes.byref(s), A, A, A + 4, 1.5, None, 1.0, 1.0, 0.0, 1, A, None,
                          None, A, n, None) == L.DASH_ERR_INVALID_ARGUMENT  # kdiag misaligned
    assert lib.dash_route(ctypes.byref(s), A, A, None, 1.5, None, 1.0, 1.0, 0.0, 1, A, None,
                          None, A, n - 1, None) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    for args in ((None, A, A), (A, None, A), (A, A, None), (A + 2, A, A)):
        assert lib.dash_summarize_diagonal(ctypes.byref(s), *args, None) == \
            L.DASH_ERR_INVALID_ARGUMENT
    assert lib.dash_summarize_diagonal(ctypes.byref(shape(D=96)), A, A, A, None) == \
        L.DASH_ERR_UNSUPPORTED
    assert lib.dash_summarize(ctypes.byref(s), None, A, A, None, 0, None) == \
        L.DASH_ERR_INVALID_ARGUMENT
    v = shape(cu=A, num_seqs=3)
    assert lib.dash_summarize(ctypes.byref(v), A, A, A, None, 0, None) == \
        L.DASH_ERR_WORKSPACE_TOO_SMALL


def test_decode_checks(lib):
    s = L.make_shape(4, 4096, 4, None, 32, 2, 128, 64, BF16)
    need = L.workspace_size(L.DASH_OP_DECODE, s)

    def dec(sh, **kw):
        a = dict(q=A, k=A, v=A, sl=A, kb=A, qb=None, diag=0, out=A, ws=A, n=need, alpha=1.5)
        a.update(kw)
        return lib.dash_attn_decode(ctypes.byref(sh), a["q"], a["k"], a["v"], a["sl"], a["kb"],
                                    a["qb"], a["alpha"], 1.0, 1.0, 0.0, 1, a["diag"], a["out"],
                                    None, None, a["ws"], a["n"], None)

    assert dec(s, diag=1) == L.DASH_ERR_INVALID_ARGUMENT            # q_bar needed
    assert dec(s, diag=1, qb=A + 4) == L.DASH_ERR_INVALID_ARGUMENT  # misaligned

    assert dec(s, sl=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert dec(s, kb=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert dec(s, n=need - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert dec(s, alpha=0.9) == L.DASH_ERR_INVALID_ARGUMENT
    assert dec(L.make_shape(4, 4000, 4, None, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                   # capacity % B
    assert dec(L.make_shape(4, 4096, 4, A, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                   # no cu_seqlens
    assert dec(L.make_shape(4, 4096, 4, None, 128, 1, 128, 64, BF16)) == \
        L.DASH_ERR_UNSUPPORTED                                        # group > 64


def test_decode_append_checks(lib):
    # the fused append + decode step: the decode checks, plus k_new, v_new and
    # qbar required and aligned (no compute: every call here is refused)
    s = L.make_shape(4, 4096, 4, None, 32, 2, 128, 64, BF16)
    need = L.workspace_size(L.DASH_OP_DECODE, s)

    def dap(sh, **kw):
        a = dict(q=A, kn=A, vn=A, k=A, v=A, sl=A, kb=A, qb=A, out=A, ws=A, n=need)
        a.update(kw)
        return lib.dash_attn_decode_append(ctypes.byref(sh), a["q"], a["kn"], a["vn"], a["k"],
                                           a["v"], a["sl"], a["kb"], a["qb"], 1.5, 1.0, 1.0,
                                           0.0, 1, 0, a["out"], None, None, a["ws"], a["n"],
                                           None)

    assert dap(s, kn=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert dap(s, vn=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert dap(s, qb=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert dap(s, kn=A + 4) == L.DASH_ERR_INVALID_ARGUMENT
    assert dap(s, sl=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert dap(s, n=need - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert dap(L.make_shape(4, 4000, 4, None, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                   # capacity % B
    # an empty batch does nothing
    assert dap(L.make_shape(0, 4096, 0, None, 32, 2, 128, 64, BF16), kn=None) == L.DASH_OK


def test_topk_route_checks(lib):
    s = shape()
    need = L.workspace_size(L.DASH_OP_ROUTE, s)

    def rt(sh, **kw):
        a = dict(q=A, kb=A, k=8, gamma=1.0, scale=0.0, gqa=1, sl=None, m=A, lp=None, ws=A,
                 n=need)
        a.update(kw)
        return lib.dash_route_topk(ctypes.byref(sh), a["q"], a["kb"], a["k"], a["gamma"],
                                   a["scale"], a["gqa"], a["sl"], a["m"], a["lp"], a["ws"],
                                   a["n"], None)

    assert rt(s, k=0) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, k=-3) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, m=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, q=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, q=A + 4) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, gamma=0.0) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, scale=math.nan) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(s, gqa=0) == L.DASH_ERR_INVALID_ARGUMENT
    assert rt(shape(D=96)) == L.DASH_ERR_UNSUPPORTED
    v = shape(cu=A, num_seqs=3)
    assert rt(v, n=0, ws=None) == L.DASH_ERR_WORKSPACE_TOO_SMALL     # varlen needs metadata
    z = shape(T=0, num_seqs=0, max_seqlen=0)
    assert rt(z) == L.DASH_OK                                        # empty: no HIP call
    d = L.make_shape(4, 4096, 4, None, 32, 2, 128, 64, BF16)
    nd = L.workspace_size(L.DASH_OP_ROUTE_DECODE, d)
    # logits [4, 2, 16, 64] + softmax statistics [4, 2, 16, 2] + scores [4, 2, 64], fp32
    assert nd == 4 * 2 * 16 * 64 * 4 + 256 * -(-(4 * 2 * 16 * 2 * 4) // 256) + 4 * 2 * 64 * 4
    assert rt(d, sl=A, n=nd - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert rt(d, sl=A, kb=None, n=nd) == L.DASH_ERR_INVALID_ARGUMENT
    assert L.workspace_size(L.DASH_OP_ROUTE_DECODE,
                            L.make_shape(4, 4096, 4, None, 4, 2, 64, 64, F32)) == 0


def test_sparse_decode_checks(lib):
    s = L.make_shape(4, 4096, 4, None, 32, 2, 128, 64, BF16)
    need = L.workspace_size(L.DASH_OP_DECODE_SPARSE, s)
    assert 0 < need < L.workspace_size(L.DASH_OP_DECODE, s)   # no routing buffers

    def ds(sh, **kw):
        a = dict(q=A, k=A, v=A, sl=A, m=A, lp=A, scale=0.0, gqa=1, out=A, ws=A, n=need)
        a.update(kw)
        return lib.dash_attn_decode_sparse(ctypes.byref(sh), a["q"], a["k"], a["v"], a["sl"],
                                           a["m"], a["lp"], a["scale"], a["gqa"], a["out"],
                                           None, a["ws"], a["n"], None)

    for key in ("q", "k", "v", "sl", "m", "lp", "out"):
        assert ds(s, **{key: None}) == L.DASH_ERR_INVALID_ARGUMENT, key
    assert ds(s, v=A + 8) == L.DASH_ERR_INVALID_ARGUMENT
    assert ds(s, scale=math.nan) == L.DASH_ERR_INVALID_ARGUMENT
    assert ds(s, n=need - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert ds(s, ws=A + 16) == L.DASH_ERR_INVALID_ARGUMENT
    assert ds(L.make_shape(4, 4000, 4, None, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                   # capacity % B
    assert ds(L.make_shape(0, 4096, 0, None, 32, 2, 128, 64, BF16)) == L.DASH_OK


def test_cache_append_checks(lib):
    s = L.make_shape(4, 4096, 4, None, 32, 2, 128, 64, BF16)

    def ap(sh, **kw):
        a = dict(kn=A, vn=A, sl=A, qb=A, kc=A, vc=A, kb=A)
        a.update(kw)
        return lib.dash_cache_append(ctypes.byref(sh), a["kn"], a["vn"], a["sl"], a["qb"],
                                     a["kc"], a["vc"], a["kb"], None)

    for key in ("kn", "vn", "sl", "qb", "kc", "vc", "kb"):
        assert ap(s, **{key: None}) == L.DASH_ERR_INVALID_ARGUMENT, key
    assert ap(s, kc=A + 8) == L.DASH_ERR_INVALID_ARGUMENT
    assert ap(L.make_shape(4, 4000, 4, None, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                   # capacity % B
    assert ap(L.make_shape(4, 4096, 4, A, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                   # no cu_seqlens
    assert ap(L.make_shape(4, 4096, 4, None, 32, 2, 96, 64, BF16)) == L.DASH_ERR_UNSUPPORTED
    assert ap(L.make_shape(0, 4096, 0, None, 32, 2, 128, 64, BF16)) == L.DASH_OK


def test_sparse_backward_checks(lib):
    s = shape()
    need = L.workspace_size(L.DASH_OP_BACKWARD, s)
    assert need > 0

    def bw(sh, **kw):
        a = dict(q=A, k=A, v=A, o=A, do=A, lse=A, m=A, lp=A, dq=A, dk=A, dv=A, db=A, ws=A,
                 n=need, gqa=1)
        a.update(kw)
        return lib.dash_attn_sparse_backward(ctypes.byref(sh), a["q"], a["k"], a["v"], a["o"],
                                             a["do"], a["lse"], a["m"], a["lp"], 0.0, a["gqa"],
                                             a["dq"], a["dk"], a["dv"], a["db"], a["ws"], a["n"],
                                             None)

    for key in ("q", "k", "v", "o", "do", "lse", "m", "lp", "dq", "dk", "dv", "db"):
        assert bw(s, **{key: None}) == L.DASH_ERR_INVALID_ARGUMENT, key
    assert bw(s, dk=A + 8) == L.DASH_ERR_INVALID_ARGUMENT
    assert bw(s, n=need - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert bw(shape(Hq=8, Hkv=2)) == L.DASH_ERR_UNSUPPORTED            # group of 4
    assert bw(shape(dtype=F32, Hq=32, Hkv=2)) == L.DASH_ERR_UNSUPPORTED
    vs = shape(cu=A, num_seqs=3)                                       # varlen: metadata
    assert bw(vs, n=L.workspace_size(L.DASH_OP_BACKWARD, vs) - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert bw(shape(T=0, num_seqs=0, max_seqlen=0)) == L.DASH_OK


def test_prefill_backward_checks(lib):
    s = shape()
    need = L.workspace_size(L.DASH_OP_PREFILL_BACKWARD, s)
    assert need > L.workspace_size(L.DASH_OP_BACKWARD, s)

    def bw(sh, alpha=1.5, gamma=1.0, sigma=1.0, **kw):
        a = dict(q=A, k=A, v=A, qb=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, dqb=A, ws=A,
                 n=need, gqa=1)
        a.update(kw)
        return lib.dash_attn_prefill_backward(ctypes.byref(sh), a["q"], a["k"], a["v"], a["qb"],
                                              alpha, None, gamma, sigma, 0.0, a["gqa"], 0, a["o"],
                                              a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                              a["dqb"], a["ws"], a["n"], None)

    for key in ("q", "k", "v", "qb", "o", "do", "lse", "dq", "dk", "dv", "dqb"):
        assert bw(s, **{key: None}) == L.DASH_ERR_INVALID_ARGUMENT, key
    assert bw(s, dqb=A + 8) == L.DASH_ERR_INVALID_ARGUMENT
    assert bw(s, n=need - 1) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert bw(s, alpha=0.5) == L.DASH_ERR_INVALID_ARGUMENT
    assert bw(shape(Hq=8, Hkv=2)) == L.DASH_ERR_UNSUPPORTED            # group of 4
    assert bw(shape(dtype=F32, Hq=32, Hkv=2)) == L.DASH_ERR_UNSUPPORTED
    vs = shape(cu=A, num_seqs=3)                                       # varlen: metadata
    assert bw(vs, n=L.workspace_size(L.DASH_OP_PREFILL_BACKWARD, vs) - 1) == \
        L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert bw(shape(T=0, num_seqs=0, max_seqlen=0)) == L.DASH_OK


def test_noalloc_decode_checks(lib):
    # everything is checked on the host before the scratch is looked up
    m = re.search(r"#define DASH_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == L.DASH_NOALLOC_SCRATCH_BYTES
    s = L.make_shape(4, 4096, 4, None, 32, 2, 128, 64, BF16)
    need = lib.dash_noalloc_scratch_need(ctypes.byref(s))
    assert 0 < need <= L.DASH_NOALLOC_SCRATCH_BYTES
    assert need == L.workspace_size(L.DASH_OP_DECODE, s)

    def na(shape, **kw):
        a = dict(q=A, k=A, v=A, sl=A, kb=A, qbar=None, alpha=1.5, gamma=1.0, sigma=1.0,
                 scale=0.0, gqa=1, diag=0, out=A, lse=None, ab=None)
        a.update(kw)
        return lib.dash_attn_decode_noalloc(ctypes.byref(shape), a["q"], a["k"], a["v"],
                                            a["sl"], a["kb"], a["qbar"], a["alpha"],
                                            a["gamma"], a["sigma"], a["scale"], a["gqa"],
                                            a["diag"], a["out"], a["lse"], a["ab"], None)
    assert na(s, q=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert na(s, out=None) == L.DASH_ERR_INVALID_ARGUMENT
    assert na(s, diag=1) == L.DASH_ERR_INVALID_ARGUMENT          # estimate_diagonal, no qbar
    assert na(s, alpha=3.0) == L.DASH_ERR_UNSUPPORTED
    assert na(L.make_shape(4, 4000, 4, None, 32, 2, 128, 64, BF16)) == \
        L.DASH_ERR_INVALID_ARGUMENT                                # capacity not whole chunks
    # a shape whose workspace exceeds the fixed scratch is refused
    big = L.make_shape(512, 131072, 512, None, 32, 2, 128, 64, BF16)
    assert lib.dash_noalloc_scratch_need(ctypes.byref(big)) > L.DASH_NOALLOC_SCRATCH_BYTES
    assert na(big) == L.DASH_ERR_UNSUPPORTED
    assert na(L.make_shape(0, 4096, 0, None, 32, 2, 128, 64, BF16)) == L.DASH_OK


def test_prefill_schedule_checks(lib):
    P = ctypes.c_int(0)
    # fixed-length shapes have no work list
    assert lib.dash_prefill_schedule(ctypes.byref(shape()), 1, A, 1 << 20, ctypes.byref(P),
                                     None) == L.DASH_ERR_UNSUPPORTED
    v = shape(T=5000, cu=A, num_seqs=3, max_seqlen=4000)
    need = -(-5000 // 8) + 3
    assert lib.dash_prefill_schedule(ctypes.byref(v), 1, A, need - 1, ctypes.byref(P),
                                     None) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert lib.dash_prefill_schedule(ctypes.byref(v), 1, None, need, ctypes.byref(P),
                                     None) == L.DASH_ERR_INVALID_ARGUMENT
    assert lib.dash_prefill_schedule(ctypes.byref(v), 1, A, need, None,
                                     None) == L.DASH_ERR_INVALID_ARGUMENT
    # more sequences than the list is built for
    many = shape(T=5000, cu=A, num_seqs=2000, max_seqlen=4000)
    assert lib.dash_prefill_schedule(ctypes.byref(many), 1, A, 1 << 20, ctypes.byref(P),
                                     None) == L.DASH_ERR_UNSUPPORTED
    # the prefill workspaces hold the list for varlen packs
    base = L.workspace_size(L.DASH_OP_SPARSE, shape(T=5000, num_seqs=1, max_seqlen=5000))
    assert L.workspace_size(L.DASH_OP_SPARSE, v) >= need * 4
