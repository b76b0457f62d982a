"""Pins of the oracle's KV commit (the step after the accepted path): moves checked by
hand on small caches, in both layouts, against the reading that node j sits at
position ctx + j and path node i lands at ctx + i."""
import numpy as np

import oracle


def _cache(B, cap, hkv, d, dtype=np.float32):
    """Distinct values: element (b, t, g, e) of K = 1000 b + 10 t + g + e / 10, V = -K."""
    b, t, g, e = np.meshgrid(np.arange(B), np.arange(cap), np.arange(hkv), np.arange(d), indexing="ij")
    k = (1000 * b + 10 * t + g + e / 10).astype(np.float32)
    v = -k
    if dtype == np.uint16:  # bf16 bit patterns: the moves are byte copies either way
        k = (k.view(np.uint32) >> 16).astype(np.uint16)
        v = (v.view(np.uint32) >> 16).astype(np.uint16)
    return k, v


def test_moves_by_hand_contiguous():
    k, v = _cache(1, 10, 2, 3)
    # ctx 3, tree of 5 nodes at positions 3..7; accepted path 0 -> 2 -> 4
    nk, nv, new_len, freed, _ = oracle.kv_commit(k, v, [3], [5], [[0, 2, 4, -1, -1]], [2])
    assert new_len.tolist() == [6]
    exp_k = k.copy()
    exp_k[0, 4] = k[0, 5]  # path node 2 (position 3 + 2) -> position 3 + 1
    exp_k[0, 5] = k[0, 7]  # path node 4 (position 3 + 4) -> position 3 + 2
    assert np.array_equal(nk, exp_k) and np.array_equal(nv, -exp_k)
    assert (freed == -1).all()


def test_destination_that_is_another_source():
    # path 0 -> 2 -> 3: position 5 (node 2) is read for slot 1 and written by slot 2
    k, v = _cache(1, 8, 1, 2)
    nk, nv, new_len, _, _ = oracle.kv_commit(k, v, [1], [6], [[0, 2, 3, -1, -1, -1]], [2])
    assert new_len.tolist() == [4]
    assert np.array_equal(nk[0, 2], k[0, 3]) and np.array_equal(nk[0, 3], k[0, 4])
    assert np.array_equal(nk[0, :2], k[0, :2]) and np.array_equal(nk[0, 4:], k[0, 4:])


def test_full_chain_is_the_identity_and_nothing_accepted_keeps_the_root():
    k, v = _cache(2, 12, 2, 4, np.uint16)
    nk, nv, new_len, _, _ = oracle.kv_commit(k, v, [2, 5], [6, 3], [[0, 1, 2, 3, 4, 5], [0, -1, -1, -1, -1, -1]],
                                             [5, 0])
    assert new_len.tolist() == [2 + 6, 5 + 1]
    assert np.array_equal(nk, k) and np.array_equal(nv, v)


def test_bad_requests_are_untouched():
    k, v = _cache(3, 10, 1, 2)
    paths = [[0, 1, -1, -1], [0, 2, 1, -1], [0, 1, 2, 3]]
    nk, nv, new_len, _, _ = oracle.kv_commit(k, v, [2, 2, 8], [4, 4, 4], paths, [-1, 2, 3])
    # accept_len < 0; a path that is not increasing; a tree past the cache end (8 + 4 > 10)
    assert new_len.tolist() == [-1, -1, -1]
    assert np.array_equal(nk, k) and np.array_equal(nv, v)


def test_paged_moves_and_page_release():
    page, hkv, d = 2, 1, 2
    # request 0: ctx 3, 5 nodes at positions 3..7 -> slots 1..3; pool pages permuted
    pool_k, pool_v = _cache(1, 6 * page, hkv, d)
    pool_k = pool_k.reshape(6, page, hkv, d)
    pool_v = pool_v.reshape(6, page, hkv, d)
    table = np.array([[4, 0, 5, 2]], np.int32)  # logical slot -> page
    nk, nv, new_len, freed, nt = oracle.kv_commit(pool_k, pool_v, [3], [5], [[0, 3, -1, -1, -1]], [1],
                                                  block_table=table, page_size=page, n_pages=6)

    def at(pool, t):  # logical position -> stored vector under the original table
        return pool[table[0, t // page], t % page]

    assert new_len.tolist() == [5]
    assert np.array_equal(nk[table[0, 2], 0], at(pool_k, 6))  # position 4 <- node 3 (position 6)
    # positions 0..3 and the rest of the pool are unchanged
    changed = np.zeros(pool_k.shape[:2], bool)
    changed[table[0, 2], 0] = True
    assert np.array_equal(nk[~changed], pool_k[~changed])
    # new_len 5 -> slots 0..2 stay; slot 3 (positions 6, 7) is released
    assert nt.tolist() == [[4, 0, 5, -1]]
    assert freed[0, 0] == 2 and (freed[0, 1:] == -1).all()


def test_every_layer_takes_the_same_moves():
    # three layers stacked on a leading axis, each with distinct values (layer l adds 1e5 l)
    k1, _ = _cache(1, 10, 2, 3)
    k = np.stack([k1 + 1e5 * l for l in range(3)]).astype(np.float32)
    v = -k
    nk, nv, new_len, _, _ = oracle.kv_commit(k, v, [3], [5], [[0, 2, 4, -1, -1]], [2])
    assert new_len.tolist() == [6]
    exp = k.copy()
    for l in range(3):
        exp[l, 0, 4] = k[l, 0, 5]
        exp[l, 0, 5] = k[l, 0, 7]
    assert np.array_equal(nk, exp) and np.array_equal(nv, -exp)


def test_layers_share_one_page_release():
    page, hkv, d = 2, 1, 2
    pool, _ = _cache(1, 6 * page, hkv, d)
    pool = pool.reshape(6, page, hkv, d)
    k = np.stack([pool, pool + 1e5]).astype(np.float32)  # two layers
    table = np.array([[4, 0, 5, 2]], np.int32)
    nk, nv, new_len, freed, nt = oracle.kv_commit(k, -k, [3], [5], [[0, 3, -1, -1, -1]], [1],
                                                  block_table=table, page_size=page, n_pages=6)
    assert new_len.tolist() == [5]
    for l in range(2):  # position 4 <- node 3 (position 6) in both layers, under the original table
        assert np.array_equal(nk[l, table[0, 2], 0], k[l, table[0, 3], 0])
    changed = np.zeros(k.shape[:3], bool)
    changed[:, table[0, 2], 0] = True
    assert np.array_equal(nk[~changed], k[~changed]) and np.array_equal(nv, -nk)
    assert nt.tolist() == [[4, 0, 5, -1]]  # slot 3 released once, not once per layer
    assert freed[0, 0] == 2 and (freed[0, 1:] == -1).all()
