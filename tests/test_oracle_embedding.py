"""Pins of the oracle's embedding gather (oracle/embedding.py): over the whole
vocabulary it is row indexing (a brute-force loop on a tiny table); over a
partition of the vocabulary into shards the shards' outputs add up to the
whole table's gather, every id landing in exactly one shard; ids outside a
shard give zero rows; rows are copied bit for bit."""

import numpy as np

from oracle import embedding_gather


def test_full_range_is_row_indexing():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((11, 6))
    ids = np.array([0, 10, 3, 3, 7])
    got = embedding_gather(W, ids, 0, 11)
    for i, t in enumerate(ids):           # brute force, row by row
        for j in range(6):
            assert got[i, j] == W[t, j]


def test_shards_add_up_to_the_whole_table():
    rng = np.random.default_rng(2)
    V, H = 103, 8
    W = rng.standard_normal((V, H))
    ids = rng.integers(0, V, 40)
    cuts = [0, 17, 50, 51, 103]                  # uneven shards, one of a single row
    parts = [embedding_gather(W[a:b], ids, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.array_equal(sum(parts), embedding_gather(W, ids, 0, V))
    hits = sum((p != 0).any(axis=1).astype(int) for p in parts)
    assert np.array_equal(hits, np.ones(len(ids), int))


def test_out_of_range_ids_give_zero_rows():
    W = np.arange(20, dtype=np.float32).reshape(5, 4) + 1
    got = embedding_gather(W, [-1, 4, 5, 9, 6], 5, 10)   # shard of ids 5..9 holds rows 0..4
    assert np.array_equal(got[0], np.zeros(4)) and np.array_equal(got[1], np.zeros(4))
    assert np.array_equal(got[2], W[0]) and np.array_equal(got[3], W[4]) and np.array_equal(got[4], W[1])


def test_bit_patterns_are_kept():
    bits = np.array([[0x7FC0, 0x8000, 0x0001, 0xFF80]], dtype=np.uint16)   # NaN, -0, denormal, -inf
    got = embedding_gather(bits, [0, 0], 0, 1)
    assert got.dtype == np.uint16 and np.array_equal(got, np.repeat(bits, 2, axis=0))
