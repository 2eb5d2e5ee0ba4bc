"""CPU oracle for the DashAttention forward path (test infrastructure only).

This package is the checker, not the product.  Only the test-suite, the
``smoke()`` check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The HIP library never imports, links or calls
anything in here, and nothing in here imports the HIP library.

Every function is plain NumPy in float64.  See ``dash_oracle`` for the
definitions and for which pages and sections each step follows.
"""

from .dash_oracle import (  # noqa: F401
    round_to_bf16,
    softmax,
    summarize,
    summarize_varlen,
    summarize_diagonal,
    routing_logits,
    entmax_threshold_bisect,
    sparsemax_sort,
    entmax15_sort,
    entmax,
    entmax_rows,
    route_position,
    routing_margin,
    route_sequence,
    route_topk_sequence,
    attention_dense,
    attention_rows,
    prefill,
    prefill_varlen,
    decode,
)

from . import dash_backward  # noqa: F401,E402
