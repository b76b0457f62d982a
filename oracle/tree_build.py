"""EAGLE-2 draft-tree construction, the oracle (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use this module; it shares no code with the GPU path.  Plain numpy
in double precision; the only library steps are a softmax written out and a sort.

Sources.  "EAGLE 演化史 (1 → 2 → 3) 与 DFlash 的回答" (zhangshuibai.github.io paper
notes), "Tree Verification 详解" part E.2 (expand and rerank), E.3 (worked
expansion step); the EAGLE-2 section of the same notes (value of a node = product of
the draft confidences on its root path, the rerank lemma); "The EAGLE Family:
Speculating in Feature Space" (consciousengines.com), "EAGLE-2: context-aware dynamic
trees" (expand from the highest path values, rerank to the top m, flatten with a tree
mask).

The pages leave these steps open; the readings taken here:

* Expand.  The tree starts as the root (value 1).  Each round expands the nodes of
  the current frontier: round 1 the root, later rounds the ``select_k`` nodes of the
  previous round's children with the largest value (ties to the earlier node).  An
  expanded node's children are the ``top_k`` tokens of its draft row by logit (ties
  to the lower token id), each with confidence c = softmax(row / T_d)[token] and
  value = value(parent) * c.
* Node ids.  Children get consecutive ids as they are created: expanded nodes in
  frontier order, each node's children in top-k order.
* Best-first (the DDTree variant of the same notes, part E.4).  The frontier is kept
  as a max-heap over every node not yet expanded, whatever its depth, and the node of
  largest value is expanded next.  Reading: a round expands the ``select_k`` best
  nodes of that frontier (``select_k`` = 1 is the one-pop heap); since every expanded
  node gets children, the unexpanded nodes are exactly the leaves of the candidate
  tree.  Leaves at depth ``MAX_DEPTH`` are not expanded (the GPU's path key holds 15
  levels).
* Rerank.  Keep the root and the ``n_final - 1`` other nodes of largest value (ties
  to the shallower node, then the lower id).  Value never increases along a path and
  a parent precedes its child on ties, so the kept set is a connected subtree.
* Flatten.  Breadth-first: by depth, then the parent's flattened index, then
  siblings in descending confidence (which is their top-k order).
* Near ties.  The GPU computes confidences with an fp32 exponential inside the
  vocabulary sum, so values agree with these to about 1e-6 relative.  A ranking
  decision between two values closer than ``TIE_REL`` (1e-5 relative, the
  probability tolerance) is recorded; such a decision may legitimately differ.
"""
from __future__ import annotations

import numpy as np

TIE_REL = 1e-5
MAX_DEPTH = 15


def softmax_f64(row, T):
    """softmax(row / T) in double precision (the definition written out)."""
    z = np.asarray(row, np.float64) / float(T)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def topk_tokens(row, k):
    """The k tokens of largest logit, largest first, ties to the lower token id."""
    row = np.asarray(row)
    order = np.lexsort((np.arange(row.shape[0]), -row.astype(np.float64)))
    return order[:k]


def _near(a, b):
    return abs(a - b) <= TIE_REL * max(abs(a), abs(b))


class TreeBuild:
    """One request's tree under construction (candidate arrays indexed by node id)."""

    def __init__(self, root_token: int):
        self.parent = [-1]
        self.token = [int(root_token)]
        self.depth = [0]
        self.value = [1.0]
        self.conf = [1.0]
        self.rank = [0]  # position among its siblings (top-k order)
        self.frontier = [0]
        self.ties = []  # (stage, round) of every decision inside the near-tie band
        self.rounds = 0

    def expand(self, rows, T_d: float, top_k: int, select_k: int, policy: str = "layer"):
        """One round.  ``rows[j]`` is the draft row (logits) at ``frontier[j]``.
        policy "layer": the next frontier is chosen among this round's children (EAGLE-2);
        "best_first": among every leaf of the candidate tree (DDTree)."""
        assert len(rows) == len(self.frontier)
        new = []
        for j, nd in enumerate(self.frontier):
            p = softmax_f64(rows[j], T_d)
            for r, t in enumerate(topk_tokens(rows[j], top_k)):
                self.parent.append(nd)
                self.token.append(int(t))
                self.depth.append(self.depth[nd] + 1)
                self.conf.append(float(p[t]))
                self.value.append(self.value[nd] * float(p[t]))
                self.rank.append(r)
                new.append(len(self.parent) - 1)
        if policy == "best_first":
            has_kids = set(self.parent[1:])
            pool = [i for i in range(len(self.parent)) if i not in has_kids and self.depth[i] < MAX_DEPTH]
        else:
            pool = new
        order = sorted(pool, key=lambda i: (-self.value[i], i))
        # the next frontier and its order (the order fixes the next round's ids)
        cut = min(select_k, len(order))
        for a, b in zip(order[:cut], order[1:cut + 1]):
            if _near(self.value[a], self.value[b]):
                self.ties.append(("frontier", self.rounds))
                break
        self.frontier = order[:cut]
        self.rounds += 1
        return new

    def rerank(self, n_final: int):
        """Returns (parent, tokens, ids) of the flattened tree (n <= n_final nodes)."""
        cand = sorted(range(1, len(self.parent)), key=lambda i: (-self.value[i], self.depth[i], i))
        keep_n = min(n_final - 1, len(cand))
        if keep_n < len(cand) and keep_n > 0 and _near(self.value[cand[keep_n - 1]], self.value[cand[keep_n]]):
            self.ties.append(("rerank", self.rounds))
        keep = set([0] + cand[:keep_n])
        for i in keep:
            assert self.parent[i] == -1 or self.parent[i] in keep  # the rerank lemma
        flat, pos, level = [0], {0: 0}, [0]
        while level:
            nxt = []
            for pi in level:
                kids = sorted((i for i in keep if self.parent[i] == pi), key=lambda i: (-self.conf[i], i))
                for c in kids:
                    pos[c] = len(flat)
                    flat.append(c)
                    nxt.append(c)
            level = nxt
        parent = np.array([-1] + [pos[self.parent[i]] for i in flat[1:]], np.int32)
        tokens = np.array([self.token[i] for i in flat], np.int32)
        return parent, tokens, np.array(flat, np.int32)


def expand_values(frontier_values, select_k, child_confidences):
    """The value arithmetic of one expand round on its own: keep the ``select_k``
    frontier nodes of largest value (ties to the earlier), give kept node j the
    children whose confidences are ``child_confidences[j]``; a child's value is its
    parent's times its confidence.  Returns (kept indices, child values, child parent
    indices), children in creation order."""
    fv = np.asarray(frontier_values, np.float64)
    kept = sorted(range(fv.size), key=lambda i: (-fv[i], i))[:select_k]
    vals, par = [], []
    for j, fi in enumerate(kept):
        for c in child_confidences[j]:
            vals.append(fv[fi] * float(c))
            par.append(fi)
    return kept, np.array(vals), np.array(par, np.int64)


def build_tree(row_of, root_token, T_d, top_k, depth, n_final, select_k=None, policy="layer"):
    """A whole tree: ``depth`` expand rounds, then rerank and flatten.
    ``row_of(tokens_on_path)`` returns the draft logits at the node whose root path
    carries those tokens (root token first)."""
    select_k = top_k if select_k is None else select_k
    t = TreeBuild(root_token)
    for _ in range(depth):
        if not t.frontier:
            break
        rows = [row_of(path_tokens(t, nd)) for nd in t.frontier]
        t.expand(rows, T_d, top_k, select_k, policy)
    parent, tokens, ids = t.rerank(n_final)
    return t, parent, tokens, ids


def path_tokens(t: TreeBuild, nd: int):
    """Tokens on the root path of node ``nd`` (root first)."""
    out = []
    while nd >= 0:
        out.append(t.token[nd])
        nd = t.parent[nd]
    return tuple(out[::-1])
