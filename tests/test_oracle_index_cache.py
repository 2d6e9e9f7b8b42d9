"""Pins of the oracle's index-cache insert (CPU only).

[SPA] minimax_m3_insert_index_cache scatters N index keys into a [B, T, D]
key cache through a slot mapping and does nothing on empty input; the
oracle's reading is that slot s names block s // T, position s % T, and that
negative slots are padding.
"""

import numpy as np

import oracle


def test_hand_built_example():
    # B = 3 blocks of T = 4 positions, D = 2
    cache = np.zeros((3, 4, 2))
    keys = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    slots = np.array([5, -1, 0, 11])
    want = np.zeros((3, 4, 2))
    want[1, 1] = [1.0, 2.0]      # slot 5 = block 1, position 1
    want[0, 0] = [5.0, 6.0]      # slot 0
    want[2, 3] = [7.0, 8.0]      # slot 11 = the last position; key 1 is padding
    got = oracle.insert_index_cache(keys, cache, slots)
    assert got is cache
    assert np.array_equal(got, want)


def test_matches_flat_indexed_assignment():
    # the same scatter as numpy's indexed assignment on the cache viewed as
    # B * T rows (slots distinct, a quarter of them padding)
    rng = np.random.default_rng(7)
    B, T, D, N = 9, 16, 32, 100
    keys = rng.standard_normal((N, D))
    slots = rng.permutation(B * T)[:N]
    slots[rng.random(N) < 0.25] = -1
    base = rng.standard_normal((B, T, D))
    want = base.copy().reshape(B * T, D)
    ok = slots >= 0
    want[slots[ok]] = keys[ok]
    got = oracle.insert_index_cache(keys, base.copy(), slots)
    assert np.array_equal(got, want.reshape(B, T, D))


def test_empty_input_leaves_the_cache():
    base = np.arange(24, dtype=np.float64).reshape(2, 3, 4)
    got = oracle.insert_index_cache(np.zeros((0, 4)), base.copy(), np.zeros(0, np.int64))
    assert np.array_equal(got, base)
