"""DashAttention forward path on MI355X (gfx950): HIP kernels behind a C ABI.

The four operations (chunk summaries, alpha-entmax routing, prefill
attention, decode attention) live in ``libdash.so`` (include/dash.h); the
functions here only marshal torch tensors and the current stream into it.
The library is loaded on first use and its absence is an error.
"""

from ._lib import DashError  # noqa: F401


def __getattr__(name):
    # the torch-facing ops are imported lazily so that the seeded input
    # generators (``workloads``) are usable without torch or the library
    if name in ("summarize", "route", "attn_prefill", "attn_sparse", "attn_decode",
                "prefill_workspace",
                "decode_workspace", "layout"):
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
