"""The benchmark's algorithmic counts against brute force (CPU).

bench.py prices the attention kernel by active FLOPs counted from the mask
the step produced: 4 D G (B |M_i| + (i mod B) + 1) per row and KV head, i.e.
2 FLOPs for each (query head, key) product of QK^T and 2 for PV over every
key a row attends (its active chunks' keys and its own chunk's keys up to
itself).  Here that count is checked against an explicit boolean matrix of
attended (row, key) pairs built from the same mask, for a fixed-length
sequence and a packed batch, and the popcount of the mask words against a
per-bit count.  The decode step's algorithmic bytes likewise: every key and
value row (D bf16 values each) the new query of a (KV head, sequence) reads.
"""

import numpy as np
import pytest

import bench


def attended_pairs(mask_rows, L, B):
    """mask_rows [Hkv, L, C] bool (chunk c of row i active) -> number of
    attended (KV head, row, key) triples, counted key by key."""
    Hkv = mask_rows.shape[0]
    total = 0
    for h in range(Hkv):
        att = np.zeros((L, L), dtype=bool)
        for i in range(L):
            for c in np.nonzero(mask_rows[h, i])[0]:
                assert c < i // B, "only chunks before the row's own are routable"
                att[i, c * B:(c + 1) * B] = True
            att[i, (i // B) * B:i + 1] = True          # own chunk, causal
        total += int(att.sum())
    return total


def random_routing(rng, Hkv, L, B, density):
    C = -(-L // B)
    m = rng.random((Hkv, L, C)) < density
    n = np.arange(L) // B
    m &= np.arange(C)[None, None, :] < n[None, :, None]
    return m


def to_words(m):
    C = m.shape[-1]
    W = -(-C // 64)
    full = np.zeros(m.shape[:-1] + (W * 64,), dtype=bool)
    full[..., :C] = m
    by = np.packbits(full, axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view(np.uint64).view(np.int64)


def test_popcounts_match_bitwise_count():
    rng = np.random.default_rng(3)
    words = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=(2, 9, 3),
                         dtype=np.int64)
    words[0, 0, 0] = -1                      # every bit set
    words[1, 1, 2] = 0
    got = bench.popcounts(words)
    want = np.zeros(words.shape[:-1], dtype=np.int64)
    for idx in np.ndindex(words.shape[:-1]):
        want[idx] = sum(bin(int(w) & (2 ** 64 - 1)).count("1") for w in words[idx])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("L,B,density", [(200, 16, 0.3), (129, 32, 1.0), (70, 64, 0.5)])
def test_prefill_active_flops_is_four_d_g_per_attended_pair(L, B, density):
    rng = np.random.default_rng(L)
    Hkv, D, G = 2, 8, 3
    m = random_routing(rng, Hkv, L, B, density)
    pop = bench.popcounts(to_words(m))
    assert np.array_equal(pop, m.sum(-1))
    want = 4.0 * D * G * attended_pairs(m, L, B)
    assert bench.prefill_active_flops(pop, B, D, G) == want
    assert bench.active_flops_at(pop, np.arange(L), B, D, G) == want


def test_packed_sequences_count_each_sequence_from_its_start():
    rng = np.random.default_rng(11)
    Hkv, D, G, B = 1, 4, 2, 16
    lens = [37, 16, 1, 80]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    C = -(-max(lens) // B)
    packed = np.zeros((Hkv, T, C), dtype=bool)
    want = 0.0
    for a, b in zip(cu[:-1], cu[1:]):
        m = random_routing(rng, Hkv, int(b - a), B, 0.4)
        packed[:, a:b, :m.shape[-1]] = m
        want += 4.0 * D * G * attended_pairs(m, int(b - a), B)
    pos = bench.local_positions(cu, T)
    assert np.array_equal(pos[cu[1]:cu[2]], np.arange(lens[1]))
    pop = bench.popcounts(to_words(packed))
    assert bench.active_flops_at(pop, pos, B, D, G) == want


def test_decode_kv_bytes_count_every_row_read_once():
    rng = np.random.default_rng(5)
    Hkv, B, D = 2, 16, 8
    seqlens = np.array([1, 16, 17, 95, 160], dtype=np.int64)
    C = -(-int(seqlens.max()) // B)
    m = np.zeros((Hkv, len(seqlens), C), dtype=bool)
    rows = 0
    for b, L in enumerate(seqlens):
        n = (int(L) - 1) // B
        m[:, b, :n] = rng.random((Hkv, n)) < 0.4
        for h in range(Hkv):
            keys = set(range(n * B, int(L)))              # own chunk, up to the query
            for c in np.nonzero(m[h, b])[0]:
                keys |= set(range(c * B, (c + 1) * B))
            rows += len(keys)
    pop = bench.popcounts(to_words(m))
    assert bench.decode_kv_bytes(pop, seqlens, B, D) == rows * D * 2 * 2   # K and V, bf16
