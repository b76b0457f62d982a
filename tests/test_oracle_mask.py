"""Pins of the oracle's ancestor-mask step against facts fixed by the pages and by
elementary tree properties (no implementation is compared against)."""
import json
import os

import numpy as np

import oracle


def test_seven_node_tree_by_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "mask_7node.json")))
    parent = np.array([g["parent"]], np.int32)
    anc, child, depth, valid = oracle.mask(parent, [7])
    assert valid[0] == 1
    assert [int(x) for x in anc[0]] == [int(h, 16) for h in g["anc_rows_hex"]]
    assert [int(x) for x in child[0]] == [int(h, 16) for h in g["child_rows_hex"]]
    assert depth[0].tolist() == g["depth"]


def test_chain_is_the_causal_mask():
    for n in (1, 2, 16, 63, 64):
        parent = np.arange(-1, n - 1, dtype=np.int32)[None]
        anc, child, depth, valid = oracle.mask(parent, [n])
        assert valid[0] == 1
        for i in range(n):
            assert int(anc[0, i]) == (1 << (i + 1)) - 1  # lower-triangular row
            assert depth[0, i] == i


def test_star():
    n = 40
    parent = np.array([[-1] + [0] * (n - 1)], np.int32)
    anc, child, depth, valid = oracle.mask(parent, [n])
    assert int(anc[0, 0]) == 1
    for i in range(1, n):
        assert int(anc[0, i]) == 1 | (1 << i)
        assert depth[0, i] == 1
    assert int(child[0, 0]) == ((1 << n) - 1) & ~1


def test_siblings_and_cousins_are_hidden():
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(2, 65))
        parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], np.int32)
        anc, _, depth, valid = oracle.mask(parent[None], [n])
        assert valid[0] == 1
        for i in range(n):
            # walk up the parent links by hand
            walk, j = set(), i
            while j >= 0:
                walk.add(j)
                j = parent[j]
            bits = {j for j in range(n) if (int(anc[0, i]) >> j) & 1}
            assert bits == walk
            assert depth[0, i] == len(walk) - 1


def test_padding_and_invalid_trees():
    n_max = 8
    parent = np.full((5, n_max), -1, np.int32)
    parent[0, :4] = [-1, 0, 0, 1]          # valid, padded
    parent[1, :3] = [0, 0, 1]              # root has a parent
    parent[2, :3] = [-1, 0, 2]             # self loop
    parent[3, :3] = [-1, 2, 0]             # forward reference
    parent[4, :3] = [-1, 0, 1]             # n_nodes out of range below
    anc, child, depth, valid = oracle.mask(parent, [4, 3, 3, 3, 9])
    assert valid.tolist() == [1, 0, 0, 0, 0]
    assert int(anc[0, 3]) == 0b1011 and all(int(a) == 0 for a in anc[0, 4:])
    assert (depth[0, 4:] == -1).all()
    for b in range(1, 5):
        assert all(int(a) == 0 for a in anc[b]) and (depth[b] == -1).all()
