"""Pins of the oracle's EAGLE-2 tree construction (expand, rerank, flatten) against
the pages' worked expansion step, a hand-derived two-round build, library routines
and the properties the pages state (connected rerank, values non-increasing along a
path, breadth-first order)."""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import tree_build as tb


def _golden(name):
    return json.load(open(os.path.join(os.path.dirname(__file__), "golden", name)))


def test_worked_expansion_step():
    # tree notes part E.3: frontier {0.95, 0.6, 0.3, 0.05}, k = 2
    g = _golden("expand_step.json")
    kept, vals, par = tb.expand_values(g["frontier_values"], g["k"], g["child_confidences_of_kept"])
    assert kept == g["kept_frontier_indices"]
    assert np.allclose(sorted(vals, reverse=True), g["new_frontier_values_sorted"], rtol=0, atol=1e-12)
    assert par.tolist() == [0, 0, 1, 1]
    # the weaker parent's strong child outranks the stronger parent's weak child
    assert vals[2] > vals[1]


def test_hand_derived_two_round_build():
    g = _golden("eagle2_build_small.json")
    rows = {tuple(int(x) for x in k.split(",")): np.log(np.array(v, np.float64)).astype(np.float32)
            for k, v in g["rows"].items()}
    for n_final, exp in g["expected"].items():
        t, parent, tokens, ids = tb.build_tree(lambda path: rows[path], g["root_token"], g["T_d"], g["top_k"],
                                               g["depth"], int(n_final), select_k=g["select_k"])
        assert parent.tolist() == exp["parent"] and tokens.tolist() == exp["tokens"] and ids.tolist() == exp["ids"]
        if "values_by_id" in exp:
            assert np.allclose(t.value, exp["values_by_id"], rtol=1e-6, atol=0)
        assert t.ties == []


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_confidences_are_the_library_softmax(T):
    row = np.random.default_rng(1).normal(0, 3, 5000).astype(np.float32)
    assert np.allclose(tb.softmax_f64(row, T), sp_softmax(row.astype(np.float64) / T), rtol=1e-12, atol=0)


def test_topk_order_and_ties_by_hand():
    assert tb.topk_tokens(np.array([1, 3, 3, 2, 3], np.float32), 3).tolist() == [1, 2, 4]
    assert tb.topk_tokens(np.array([-np.inf, 0, -1, 0], np.float32), 4).tolist() == [1, 3, 2, 0]
    assert tb.topk_tokens(np.zeros(6, np.float32), 2).tolist() == [0, 1]


def _rows_from_seed(seed, V, scale=3.0):
    cache = {}

    def row_of(path):
        if path not in cache:
            r = np.random.default_rng([seed] + list(path))
            cache[path] = r.normal(0, scale, V).astype(np.float32)
        return cache[path]

    return row_of


def test_top1_is_the_greedy_draft_chain():
    V, depth = 50, 7
    row_of = _rows_from_seed(3, V)
    t, parent, tokens, ids = tb.build_tree(row_of, 5, 1.0, 1, depth, 64)
    assert parent.tolist() == [-1] + list(range(depth))
    path, val = (5,), 1.0
    for d in range(depth):  # each token is the argmax of the previous node's row
        row = row_of(path)
        nxt = int(np.argmax(row))
        assert tokens[d + 1] == nxt
        val *= float(sp_softmax(row.astype(np.float64))[nxt])
        path = path + (nxt,)
    assert t.value[ids[-1]] == pytest.approx(val, rel=1e-12)


def test_depth_one_is_the_top_tokens_of_the_root():
    V = 40
    row_of = _rows_from_seed(4, V)
    t, parent, tokens, ids = tb.build_tree(row_of, 2, 1.0, 10, 1, 8)
    assert parent.tolist() == [-1] + [0] * 7
    assert tokens[1:].tolist() == np.argsort(-row_of((2,)).astype(np.float64), kind="stable")[:7].tolist()


@pytest.mark.parametrize("seed,k,depth,n", [(0, 10, 6, 60), (1, 8, 8, 64), (2, 3, 5, 20), (3, 4, 3, 64)])
def test_rerank_properties(seed, k, depth, n):
    V = 300
    t, parent, tokens, ids = tb.build_tree(_rows_from_seed(seed, V), 1, 1.0, k, depth, n)
    total = 1 + k + (depth - 1) * k * k
    assert len(t.parent) == total
    m = len(ids)
    assert m == min(n, total)
    kept = set(ids.tolist())
    dropped = [i for i in range(1, total) if i not in kept]
    if dropped:  # every kept node is worth at least every dropped one
        assert min(t.value[i] for i in kept if i) >= max(t.value[i] for i in dropped)
    d = np.array([t.depth[i] for i in ids])
    assert parent[0] == -1 and np.all(parent[1:] < np.arange(1, m)) and np.all(parent[1:] >= 0)
    assert np.all(np.diff(d) >= 0) and np.all(np.diff(parent[1:]) >= 0)  # breadth-first
    for i in range(1, m):  # parent links agree with the candidate tree; value never grows
        assert ids[parent[i]] == t.parent[ids[i]]
        assert t.value[ids[i]] <= t.value[ids[parent[i]]]
        assert tokens[i] == t.token[ids[i]]
    for i in range(1, m - 1):  # siblings in descending confidence
        if parent[i] == parent[i + 1]:
            assert t.conf[ids[i]] >= t.conf[ids[i + 1]]


def test_certain_token_ties_its_parent_and_the_parent_wins():
    # a row with one finite logit has confidence exactly 1: the child's value equals its
    # parent's, and the shallower node is kept first
    V = 6

    def row_of(path):
        r = np.full(V, -np.inf, np.float32)
        if len(path) == 1:
            r[:] = np.log(np.array([0.4, 0.3, 0.2, 0.05, 0.03, 0.02], np.float32))
        else:
            r[len(path)] = 0.0
        return r

    t, parent, tokens, ids = tb.build_tree(row_of, 0, 1.0, 1, 3, 3)
    assert t.value[1] == t.value[2] == t.value[3] == pytest.approx(0.4, rel=1e-6)
    assert ids.tolist() == [0, 1, 2] and parent.tolist() == [-1, 0, 1]


def test_near_ties_are_recorded():
    tr = tb.TreeBuild(0)
    a = np.log(np.array([0.5, 0.5 * (1 - 3e-6), 0.0 + 1e-30], np.float64)).astype(np.float32)
    tr.expand([a], 1.0, 2, 1)
    assert ("frontier", 0) in tr.ties
    tr2 = tb.TreeBuild(0)
    tr2.expand([np.log(np.array([0.6, 0.3, 0.1])).astype(np.float32)], 1.0, 2, 1)
    assert tr2.ties == []


def _prob_rows(table):
    return {k: np.log(np.array(v, np.float64)).astype(np.float32) for k, v in table.items()}


def test_best_first_returns_to_a_shallower_leaf_by_hand():
    # root children 0.6, 0.4; the 0.6 node's children 0.5 x 0.6 = 0.3 each.  The next
    # frontier (select_k 1): EAGLE-2 picks among the new children (a 0.3 node); the
    # best-first heap picks the older 0.4 leaf at depth 1
    rows = _prob_rows({(7,): [0.6, 0.4, 1e-12, 1e-12], (7, 0): [0.5, 0.5, 1e-12, 1e-12],
                       (7, 1): [0.9, 0.1, 1e-12, 1e-12]})
    lay, bf = tb.TreeBuild(7), tb.TreeBuild(7)
    for t, pol in ((lay, "layer"), (bf, "best_first")):
        t.expand([rows[(7,)]], 1.0, 2, 1, pol)
        assert t.frontier == [1]  # the 0.6 child
        t.expand([rows[(7, 0)]], 1.0, 2, 1, pol)
    assert lay.frontier == [3] and bf.frontier == [2]  # ids: 3 = first 0.3 child, 2 = the 0.4 leaf
    bf.expand([rows[(7, 1)]], 1.0, 2, 1, "best_first")
    assert bf.value[5] == pytest.approx(0.4 * 0.9, rel=1e-6) and bf.frontier == [5]  # 0.36 > 0.3


def _full_values(row_of, root, top_k, depth):
    """Every node of the candidate tree to ``depth`` (brute force): path -> value."""
    out, level = {}, [((root,), 1.0)]
    for _ in range(depth):
        nxt = []
        for path, v in level:
            p = tb.softmax_f64(row_of(path), 1.0)
            for t in tb.topk_tokens(row_of(path), top_k):
                nxt.append((path + (int(t),), v * float(p[t])))
        out.update(nxt)
        level = nxt
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_best_first_pops_the_best_nodes_of_the_whole_candidate_tree(seed):
    # one pop per round: the expanded nodes are the r most valuable nodes of the full
    # candidate tree (values never grow along a path), popped in non-increasing order
    V, k, r = 12, 3, 9
    row_of = _rows_from_seed(seed, V, scale=2.0)
    t = tb.TreeBuild(0)
    popped = []
    for _ in range(r):
        popped.append(t.frontier[0])
        t.expand([row_of(tb.path_tokens(t, t.frontier[0]))], 1.0, k, 1, "best_first")
    vals = [t.value[i] for i in popped]
    assert all(a >= b for a, b in zip(vals, vals[1:]))
    full = _full_values(row_of, 0, k, r)
    best = sorted(full.values(), reverse=True)[: r - 1]  # the root (value 1) is the first pop
    assert np.allclose(sorted(vals[1:], reverse=True), best, rtol=1e-12)
    assert t.ties == []


def test_worked_example_values_follow_the_product_rule():
    # tree notes part G: node values are products of the draft confidences on the root path
    g = _golden("worked_example.json")["printed_by_the_page"]
    conf = g["draft_confidence"]
    _, lvl1, _ = tb.expand_values([1.0], 1, [[conf["1"], conf["2"]]])
    _, lvl2, _ = tb.expand_values(list(lvl1), 2, [[conf["3"], conf["4"]], [conf["5"], conf["6"]]])
    np.testing.assert_allclose([1.0] + list(lvl1) + list(lvl2), g["node_values"], rtol=0, atol=1e-12)
