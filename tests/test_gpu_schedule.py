"""The cost-sorted work list of packed (varlen) prefill, integer-exact.

The list (dash_prefill_schedule) is the order in which the G >= 16 prefill
attention kernel takes its tiles of P positions: the sequences longest first
(by tile count, ties by index), each sequence's tiles from its last (a tile's
rows see more keys the later it starts) down to its first.  The reference
here restates that rule in plain Python from the lengths alone.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

from sparse_hierarchical_attention_dash_amd import _lib as L

from gpu_helpers import flush

pytestmark = pytest.mark.gpu


def reference(lens, P, cap):
    n = [-(-L // P) for L in lens]
    order = sorted(range(len(lens)), key=lambda s: (-n[s], s))
    items = [(s << 16) | t for s in order for t in range(n[s] - 1, -1, -1)]
    assert len(items) <= cap
    return np.array(items + [0xFFFFFFFF] * (cap - len(items)), dtype=np.uint32)


@pytest.mark.parametrize("lens,G", [
    ([4791, 4937, 11028, 15466, 16872, 24434, 66682, 67364], 16),   # the varlen workload's draw
    ([1, 15, 16, 17, 0, 33, 64, 65, 1000], 16),                    # ragged, one empty sequence
    ([300, 300, 300, 2, 5000], 32),                                 # G = 32: 16 positions a tile
    (list(np.random.default_rng(3).integers(1, 3000, 600)), 16),    # many sequences
])
def test_schedule_is_cost_sorted(lens, G):
    flush(f"schedule: {len(lens)} sequences, G = {G}")
    lens = [int(x) for x in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    cut = torch.from_numpy(cu).cuda()
    shape = L.make_shape(len(lens), max(lens), T, cut.data_ptr(), 2 * G, 2, 128, 64, 1)
    cap = -(-T // 8) + len(lens)
    items = torch.empty(cap, dtype=torch.int32, device="cuda")
    P = ctypes.c_int(0)
    st = L.lib().dash_prefill_schedule(ctypes.byref(shape), 1, ctypes.c_void_p(items.data_ptr()),
                                       cap, ctypes.byref(P), None)
    assert st == L.DASH_OK, L.status_string(st) if hasattr(L, "status_string") else st
    torch.cuda.synchronize()
    got = items.cpu().numpy().view(np.uint32)
    assert P.value == 16 * 16 // G     # 16 tiles of 16 rows: 16 heads of 16 or 8 positions
    ref = reference(lens, P.value, cap)
    assert np.array_equal(got, ref)
    # every tile of every sequence exactly once
    live = got[got != 0xFFFFFFFF]
    pairs = sorted((int(x) >> 16, int(x) & 0xFFFF) for x in live)
    want = sorted((s, t) for s, L_ in enumerate(lens) for t in range(-(-L_ // P.value)))
    assert pairs == want
    flush(f"  {len(live)} tiles of {P.value} positions")
