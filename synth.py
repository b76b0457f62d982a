"""Seeded synthetic inputs for the tree-verification step (test and benchmark support).

This module only *makes inputs*: draft trees, token ids, logits, Q/K/V activations,
paged block tables and uniforms.  It holds none of the verification arithmetic (no
masks, no attention, no rejection rule) and no tree-construction method: the
EAGLE-2 trees of workloads 2 and 5 come from a tree builder the caller passes in
(the tests pass the CPU oracle's, the benchmark builds them on the GPU with the
library's own expand / rerank calls).  Where an input's statistics are defined by a
draft distribution (i.i.d. sibling draws, the top-2 children of the 7-node tree) the
generator evaluates that distribution with plain numpy as part of making the input.

Workloads follow the shapes the pages discuss: Llama-3-8B-like GQA heads and
128k vocabularies, EAGLE-2 expand/rerank trees of 60 nodes, 16-token DFlash
blocks verified as chains, a batch of small random trees over a paged KV cache,
and a long-context 64/8-head shard with heavy-tailed logits.  No public
benchmark item is used; every value is drawn from a seeded PCG64 stream.

Uniform convention: every uniform is k * 2**-24 for an integer k drawn uniformly
from [0, 2**24), so it is exactly representable in fp32 and lies in [0, 1)
(0 included).
"""
from __future__ import annotations

import math
import zlib

import numpy as np

# --------------------------------------------------------------------------
# basic seeded draws
# --------------------------------------------------------------------------


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 stream addressed by a tuple of integers (seed, purpose, id...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key])))


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draft_probs(dft_row: np.ndarray, Td: float) -> np.ndarray:
    """Draft distribution used to shape trees (generator-side, float64)."""
    z = dft_row.astype(np.float64) / Td
    z -= z.max()
    e = np.exp(z)
    return e / e.sum()


def _topk_desc(row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries, descending, ties to the lower index."""
    idx = np.argpartition(-row, k)[:k] if k < row.shape[0] else np.arange(row.shape[0])
    order = np.lexsort((idx, -row[idx]))
    return idx[order]


# --------------------------------------------------------------------------
# logit rows, addressed per tree node so a node's rows never depend on order
# --------------------------------------------------------------------------


class RowSource:
    """Target/draft logit rows for a node id.

    kind "normal": target ~ N(0, sigma_t); "student_t": target = scale_t * t(3).
    draft = target + N(0, sigma_d).
    """

    def __init__(self, seed: int, vocab: int, kind: str = "normal", sigma_t: float = 3.0,
                 sigma_d: float = 1.0, scale_t: float = 2.0):
        self.seed, self.vocab, self.kind = seed, vocab, kind
        self.sigma_t, self.sigma_d, self.scale_t = sigma_t, sigma_d, scale_t
        self._cache: dict[int, tuple[np.ndarray, np.ndarray]] = {}

    def rows(self, uid: int) -> tuple[np.ndarray, np.ndarray]:
        if uid not in self._cache:
            r = rng_for(self.seed, 11, uid)
            if self.kind == "normal":
                t = r.normal(0.0, self.sigma_t, self.vocab)
            elif self.kind == "student_t":
                t = self.scale_t * r.standard_t(3.0, self.vocab)
            else:
                raise ValueError(self.kind)
            d = t + r.normal(0.0, self.sigma_d, self.vocab)
            self._cache[uid] = (t.astype(np.float32), d.astype(np.float32))
        return self._cache[uid]


# --------------------------------------------------------------------------
# tree shapes
# --------------------------------------------------------------------------


def topk_binary_tree(src: RowSource, Td: float, root_token: int):
    """Depth-2 complete binary tree (7 nodes, BFS), children = top-2 draft tokens of the parent."""
    parent = np.array([-1, 0, 0, 1, 1, 2, 2], np.int32)
    tokens = np.zeros(7, np.int32)
    tokens[0] = root_token
    for p in range(3):
        _, dft = src.rows(p)
        kids = [c for c in range(7) if parent[c] == p]
        for c, tok in zip(kids, _topk_desc(dft.astype(np.float64), 2)):
            tokens[c] = tok
    return parent, tokens, list(range(7))


def chain_tree(n: int):
    return np.arange(-1, n - 1, dtype=np.int32)


def path_rows(seed: int, path, vocab: int, kind: str = "normal", scale: float = 3.0, noise: float = 1.0):
    """(target, draft) logit rows at the tree node whose root path carries the tokens
    ``path`` (root first), seeded by the path itself, so a node gets the same rows
    whatever builds the tree and in whatever order it visits the nodes.  kind "normal":
    target ~ N(0, scale); "student_t": target = scale * t(3); draft = target + N(0, noise)."""
    key = np.asarray(path, np.int64)
    r = np.random.default_rng([seed, len(key), zlib.crc32(key.tobytes())])
    base = r.normal(0.0, scale, vocab) if kind == "normal" else scale * r.standard_t(3.0, vocab)
    return base.astype(np.float32), (base + r.normal(0.0, noise, vocab)).astype(np.float32)


def path_row(seed: int, path, vocab: int, kind: str = "normal", scale: float = 3.0, noise: float = 1.0):
    """The draft row of ``path_rows``."""
    return path_rows(seed, path, vocab, kind, scale, noise)[1]


class PathRows:
    """``path_rows`` of one workload, cached per path (a RowSource keyed by paths)."""

    def __init__(self, seed: int, vocab: int, kind: str, scale: float, noise: float):
        self.seed, self.vocab, self.kind, self.scale, self.noise = seed, vocab, kind, scale, noise
        self._cache: dict = {}

    def rows(self, path):
        path = tuple(int(t) for t in path)
        if path not in self._cache:
            self._cache[path] = path_rows(self.seed, path, self.vocab, self.kind, self.scale, self.noise)
        return self._cache[path]


def random_tree(rng: np.random.Generator, n: int, max_branch: int = 4, max_depth: int = 8):
    """Breadth-first (FIFO) random tree: each popped node gets U{1..max_branch} children
    while the node budget lasts and its depth is below max_depth; regenerate on a dead end."""
    while True:
        parent = [-1]
        depth = [0]
        queue = [0]
        while queue and len(parent) < n:
            p = queue.pop(0)
            if depth[p] >= max_depth:
                continue
            nb = int(rng.integers(1, max_branch + 1))
            for _ in range(nb):
                if len(parent) >= n:
                    break
                parent.append(p)
                depth.append(depth[p] + 1)
                queue.append(len(parent) - 1)
        if len(parent) == n:
            return np.array(parent, np.int32)


def sample_iid_tokens(rng, parent, dft_rows, Td):
    """Token of every non-root node drawn i.i.d. from its parent's draft distribution."""
    tokens = np.zeros(len(parent), np.int32)
    for c in range(1, len(parent)):
        q = _draft_probs(dft_rows[parent[c]], Td)
        cdf = np.cumsum(q)
        tokens[c] = min(int(np.searchsorted(cdf, rng.random() * cdf[-1], side="right")), len(q) - 1)
    return tokens


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

CONFIGS = {
    1: "tiny: 1 x 7-node binary tree, ctx 128, 4/4 heads, d 64, fp32, vocab 1024, T=1",
    2: "llama3-8b-shape: 1 x 60-node EAGLE-2 tree (k=10, depth 6), ctx 4096, 32/8 heads, d 128, bf16, vocab 128256",
    3: "chain-16 (DFlash block): ctx 8192, 32/8 heads, d 128, bf16, vocab 151936, T=0.7",
    4: "batch 8 x 32-node random trees, ctx U[512,8192], paged KV (16-token pages), 32/8 heads, bf16, vocab 128256",
    5: "long-context shard: 1 x 64-node EAGLE-2 tree (k=8, depth 8), ctx 32768, 64/8 heads, bf16, vocab 152064, t(3)x2 logits",
    6: "cost-table grid: B x N-node random trees, one ctx for all requests, contiguous KV, 32/8 heads, d 128, bf16, vocab 128256",
}


def _activations(rng, B, n_max, hq, hkv, d, s_cap, bf16):
    q = rng.standard_normal((B, n_max, hq, d), dtype=np.float32)
    k = rng.standard_normal((B, s_cap, hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, s_cap, hkv, d), dtype=np.float32)
    if bf16:
        q, k, v = to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
    return q, k, v


def make_config(cfg: int, seed: int = 0, T: float | None = None, with_kv: bool = True,
                ctx_override: int | None = None, vocab_override: int | None = None, grid=None, tree_builder=None):
    """Build one input set for workload ``cfg`` (1..6).  Returns a dict of numpy arrays
    and scalars.  ``ctx_override`` / ``vocab_override`` shrink a workload for fast tests
    while keeping its tree generator and head geometry.  Workload 6 takes
    ``grid = (B, ctx, N)``: workload 4's trees, tokens and logits with N nodes per tree,
    every request at context ``ctx`` and contiguous KV (see ``grid_point`` for cutting
    smaller points out of one such input).

    Workloads 2 and 5 need ``tree_builder(row_of, root_token, T_d, top_k, depth,
    n_final) -> (parent, tokens, paths)``: an EAGLE-2 expand / rerank over the draft
    rows ``row_of(path)`` (path = the tokens on a node's root path, root first),
    returning the flattened tree and each node's path; every node's target and draft
    rows are then ``path_rows`` of its path."""
    rng = rng_for(seed, cfg, 1)
    inp: dict = {"cfg": cfg, "seed": seed, "page_size": 0, "n_pages": 0, "block_table": None}
    if cfg == 1:
        V, hq, hkv, d, ctx = 1024, 4, 4, 64, 128
        V = vocab_override or V
        ctx = ctx_override or ctx
        T_ = 1.0 if T is None else T
        src = RowSource(seed * 7919 + 1, V, "normal", sigma_t=2.0, sigma_d=1.0)
        parent, tokens, uids = topk_binary_tree(src, 1.0, root_token=int(rng.integers(V)))
        trees = [(parent, tokens, uids)]
        Td, bf16, B = T_ if T_ > 0 else 1.0, False, 1
        ctxs = [ctx]
    elif cfg in (2, 5):
        if tree_builder is None:
            raise ValueError("workloads 2 and 5 take their EAGLE-2 tree from a tree_builder")
        if cfg == 2:
            V, hq, hkv, d, ctx, k, depth, n = 128256, 32, 8, 128, 4096, 10, 6, 60
            src_kw = dict(kind="normal", scale=3.0, noise=1.0)
        else:
            V, hq, hkv, d, ctx, k, depth, n = 152064, 64, 8, 128, 32768, 8, 8, 64
            src_kw = dict(kind="student_t", scale=2.0, noise=1.5)
        V = vocab_override or V
        ctx = ctx_override or ctx
        T_ = 1.0 if T is None else T
        Td = T_ if T_ > 0 else 1.0
        src = PathRows(seed * 7919 + cfg, V, **src_kw)
        parent, tokens, paths = tree_builder(lambda path: src.rows(path)[1], int(rng.integers(V)), Td, k, depth, n)
        trees = [(np.asarray(parent, np.int32), np.asarray(tokens, np.int32), [tuple(p) for p in paths])]
        bf16, B = True, 1
        ctxs = [ctx]
    elif cfg == 3:
        V, hq, hkv, d, ctx, n = 151936, 32, 8, 128, 8192, 16
        V = vocab_override or V
        ctx = ctx_override or ctx
        T_ = 0.7 if T is None else T
        Td = 1.0
        src = RowSource(seed * 7919 + 3, V, "normal", sigma_t=3.0, sigma_d=0.5)
        parent = chain_tree(n)
        dft_rows = [src.rows(i)[1] for i in range(n)]
        tokens = sample_iid_tokens(rng, parent, dft_rows, Td)
        tokens[0] = int(rng.integers(V))
        trees = [(parent, tokens, list(range(n)))]
        bf16, B = True, 1
        ctxs = [ctx]
    elif cfg in (4, 6):
        V, hq, hkv, d, n, B = 128256, 32, 8, 128, 32, 8
        V = vocab_override or V
        T_ = 1.0 if T is None else T
        Td = T_ if T_ > 0 else 1.0
        if cfg == 4:
            hi = ctx_override or 8192
            lo = min(512, hi)
            ctxs = [int(c) for c in rng.integers(lo, hi + 1, size=B)]
        else:
            B, c_all, n = (int(x) for x in grid)
            ctxs = [c_all] * B
        trees = []
        for b in range(B):
            src = RowSource(seed * 7919 + 4000 + b, V, "normal", sigma_t=3.0, sigma_d=1.0)
            parent = random_tree(rng_for(seed, 4, 2, b), n, 4, 8)
            dft_rows = [src.rows(i)[1] for i in range(n)]
            tokens = sample_iid_tokens(rng_for(seed, 4, 3, b), parent, dft_rows, Td)
            tokens[0] = int(rng.integers(V))
            trees.append((parent, tokens, list(range(n)), src))
        bf16 = True
    else:
        raise ValueError(cfg)

    n_max = max(len(t[0]) for t in trees)
    parent = np.full((B, n_max), -1, np.int32)
    tokens = np.zeros((B, n_max), np.int32)
    n_nodes = np.zeros(B, np.int32)
    tgt = np.zeros((B, n_max, V), np.float32)
    dft = np.zeros((B, n_max, V), np.float32)
    for b, t in enumerate(trees):
        p, tk, uids = t[0], t[1], t[2]
        s = t[3] if len(t) > 3 else src
        nb = len(p)
        parent[b, :nb] = p
        tokens[b, :nb] = tk
        n_nodes[b] = nb
        for i, uid in enumerate(uids):
            tr, dr = s.rows(uid)
            tgt[b, i] = tr
            dft[b, i] = dr
    urng = rng_for(seed, cfg, 9)
    # temperatures are fp32 values (what the library receives), carried as Python floats
    T_, Td = float(np.float32(T_)), float(np.float32(Td))
    inp.update(dict(B=B, n_max=n_max, V=V, hq=hq, hkv=hkv, d=d, T=T_, Td=Td, bf16=bf16,
                    parent=parent, tokens=tokens, n_nodes=n_nodes, tgt_logits=tgt, dft_logits=dft,
                    u_accept=uniforms(urng, (B, n_max)), u_sample=uniforms(urng, (B, n_max)),
                    ctx_len=np.array(ctxs, np.int32)))
    if with_kv:
        arng = rng_for(seed, cfg, 5)
        if cfg == 4:  # workload 6 keeps the contiguous layout
            page = 16
            pages_per = [math.ceil((ctxs[b] + n_nodes[b]) / page) for b in range(B)]
            n_pages = sum(pages_per) + 8  # a few spare pages that no request owns
            max_pages = max(pages_per)
            perm = arng.permutation(n_pages).astype(np.int32)
            bt = np.full((B, max_pages), -1, np.int32)
            o = 0
            for b in range(B):
                bt[b, : pages_per[b]] = perm[o: o + pages_per[b]]
                o += pages_per[b]
            q = arng.standard_normal((B, n_max, hq, d), dtype=np.float32)
            k = arng.standard_normal((n_pages, page, hkv, d), dtype=np.float32)
            v = arng.standard_normal((n_pages, page, hkv, d), dtype=np.float32)
            q, k, v = to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
            inp.update(page_size=page, n_pages=n_pages, block_table=bt, kv_capacity=max_pages)
        else:
            s_cap = int(max(ctxs) + n_max)
            q, k, v = _activations(arng, B, n_max, hq, hkv, d, s_cap, bf16)
            inp.update(kv_capacity=s_cap)
        inp.update(q=q, k=k, v=v)
    else:
        inp.update(q=None, k=None, v=None)
    return inp


def grid_point(inp: dict, B: int, ctx: int, N: int) -> dict:
    """A smaller point of the cost-table grid cut out of a workload-6 input: the first
    B requests, the first N nodes of each tree and context ``ctx`` for every request.
    The trees are built breadth-first, so every parent precedes its children and a
    prefix of the node order is again a tree.  K/V keep their capacity; the tree's own
    entries move with the context (slots ctx .. ctx + N - 1), whose contents are as
    random as the prompt's."""
    assert inp["cfg"] == 6 and inp["block_table"] is None
    assert B <= inp["B"] and N <= inp["n_max"] and ctx + N <= inp["kv_capacity"]
    par = inp["parent"][:B, :N]
    assert np.all(par[:, 1:] < np.arange(1, N)[None, :]) and np.all(par[:, 0] == -1)
    out = dict(inp)
    for key in ("parent", "tokens", "tgt_logits", "dft_logits", "u_accept", "u_sample"):
        out[key] = np.ascontiguousarray(inp[key][:B, :N])
    if inp.get("q") is not None:
        out["q"] = np.ascontiguousarray(inp["q"][:B, :N])
        out["k"], out["v"] = inp["k"][:B], inp["v"][:B]
    out.update(B=B, n_max=N, n_nodes=np.full(B, N, np.int32), ctx_len=np.full(B, ctx, np.int32))
    return out


# --------------------------------------------------------------------------
# statistical workloads (16-token vocabulary)
# --------------------------------------------------------------------------


def log_probs_f32(p: np.ndarray) -> np.ndarray:
    """Logits that encode a probability vector (zeros become -inf)."""
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64)).astype(np.float32)


def q_variant(kind: str, p: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    V = p.size
    if kind == "noisy":
        z = np.log(np.maximum(p, 1e-300)) + rng.normal(0, 1, V)
        z -= z.max()
        q = np.exp(z)
    elif kind == "uniform":
        q = np.ones(V)
    elif kind == "equal":
        q = p.copy()
    elif kind == "zeros":  # q vanishes on part of p's support
        q = rng.dirichlet(np.ones(V))
        q[np.argsort(-p)[:3]] = 0.0
    elif kind == "onehot":
        q = np.full(V, 0.03 / (V - 1))
        q[int(rng.integers(V))] = 0.97
    else:
        raise ValueError(kind)
    return q / q.sum()


def star_trials(rng, p_root, q_root, n_children, n_trials, leaf_p=None):
    """n_trials independent stars: root with n_children i.i.d. children drawn from q_root."""
    V = p_root.size
    n = 1 + n_children
    parent = np.tile(np.array([-1] + [0] * n_children, np.int32), (n_trials, 1))
    cdf = np.cumsum(q_root)
    draws = np.searchsorted(cdf, rng.random((n_trials, n_children)) * cdf[-1], side="right")
    tokens = np.zeros((n_trials, n), np.int32)
    tokens[:, 1:] = np.minimum(draws, V - 1)
    tgt = np.empty((n_trials, n, V), np.float32)
    dft = np.empty((n_trials, n, V), np.float32)
    tgt[:, 0] = log_probs_f32(p_root)
    dft[:, 0] = log_probs_f32(q_root)
    lp = leaf_p if leaf_p is not None else np.full(V, 1.0 / V)
    tgt[:, 1:] = log_probs_f32(lp)
    dft[:, 1:] = log_probs_f32(np.full(V, 1.0 / V))
    return dict(parent=parent, tokens=tokens, n_nodes=np.full(n_trials, n, np.int32), tgt_logits=tgt,
                dft_logits=dft, u_accept=uniforms(rng, (n_trials, n)), u_sample=uniforms(rng, (n_trials, n)))


def depth2_trials(rng, p_root, q_root, P2, Q2, k1, k2, n_trials):
    """Root with k1 i.i.d. children ~ q_root; each child c has k2 i.i.d. children ~ Q2[token(c)].
    Rows are keyed by the path: child c's target row is P2[token(c)]."""
    V = p_root.size
    n = 1 + k1 + k1 * k2
    par = [-1] + [0] * k1
    for c in range(k1):
        par += [1 + c] * k2
    parent = np.tile(np.array(par, np.int32), (n_trials, 1))
    tokens = np.zeros((n_trials, n), np.int32)
    cdf = np.cumsum(q_root)
    tokens[:, 1:1 + k1] = np.minimum(np.searchsorted(cdf, rng.random((n_trials, k1)) * cdf[-1], side="right"), V - 1)
    Q2c = np.cumsum(Q2, axis=1)
    for c in range(k1):
        t1 = tokens[:, 1 + c]
        rr = rng.random((n_trials, k2))
        for j in range(k2):
            cd = Q2c[t1]
            tokens[:, 1 + k1 + c * k2 + j] = np.minimum(
                (cd < (rr[:, j] * cd[:, -1])[:, None]).sum(axis=1), V - 1)
    lP2, lQ2 = log_probs_f32(P2), log_probs_f32(Q2)
    tgt = np.empty((n_trials, n, V), np.float32)
    dft = np.empty((n_trials, n, V), np.float32)
    tgt[:, 0] = log_probs_f32(p_root)
    dft[:, 0] = log_probs_f32(q_root)
    for c in range(k1):
        t1 = tokens[:, 1 + c]
        tgt[:, 1 + c] = lP2[t1]
        dft[:, 1 + c] = lQ2[t1]
    tgt[:, 1 + k1:] = log_probs_f32(np.full(V, 1.0 / V))
    dft[:, 1 + k1:] = log_probs_f32(np.full(V, 1.0 / V))
    return dict(parent=parent, tokens=tokens, n_nodes=np.full(n_trials, n, np.int32), tgt_logits=tgt,
                dft_logits=dft, u_accept=uniforms(rng, (n_trials, n)), u_sample=uniforms(rng, (n_trials, n)))


def alpha_pq(alpha: float, V: int = 16):
    """p = alpha*U(S) + (1-alpha)*U(A), q = alpha*U(S) + (1-alpha)*U(B) with S, A, B disjoint
    (S = first half, A and B the two remaining quarters), so sum_x min(p, q) = alpha."""
    S = np.arange(V // 2)
    A = np.arange(V // 2, V // 2 + V // 4)
    Bs = np.arange(V // 2 + V // 4, V)
    p = np.zeros(V)
    q = np.zeros(V)
    p[S] += alpha / S.size
    q[S] += alpha / S.size
    p[A] += (1 - alpha) / A.size
    q[Bs] += (1 - alpha) / Bs.size
    return p, q


def chain_trials(rng, p, q, depth, n_trials):
    """Chains of `depth` drafted tokens (depth + 1 nodes), every level with the same p, q;
    drafted tokens i.i.d. from q."""
    V = p.size
    n = depth + 1
    parent = np.tile(np.arange(-1, n - 1, dtype=np.int32), (n_trials, 1))
    cdf = np.cumsum(q)
    tokens = np.zeros((n_trials, n), np.int32)
    tokens[:, 1:] = np.minimum(np.searchsorted(cdf, rng.random((n_trials, depth)) * cdf[-1], side="right"), V - 1)
    tgt = np.broadcast_to(log_probs_f32(p), (n_trials, n, V)).copy()
    dft = np.broadcast_to(log_probs_f32(q), (n_trials, n, V)).copy()
    return dict(parent=parent, tokens=tokens, n_nodes=np.full(n_trials, n, np.int32), tgt_logits=tgt,
                dft_logits=dft, u_accept=uniforms(rng, (n_trials, n)), u_sample=uniforms(rng, (n_trials, n)))


def chain_redraw(tgt_rows, dft_rows, Td: float, root_token: int, n_trials: int, rng):
    """Trials on one chain whose logit rows are fixed (tgt_rows, dft_rows: [n, V]):
    every trial draws its own tokens, token i from the draft distribution of row
    i - 1 at temperature Td, and its own uniforms.  Returns the tree arrays
    ([n_trials, n]); the rows are the caller's to broadcast."""
    n, V = tgt_rows.shape
    tokens = np.zeros((n_trials, n), np.int32)
    tokens[:, 0] = root_token
    for i in range(1, n):
        cdf = np.cumsum(_draft_probs(dft_rows[i - 1], Td))
        tokens[:, i] = np.minimum(np.searchsorted(cdf, rng.random(n_trials) * cdf[-1], side="right"), V - 1)
    return dict(parent=np.tile(chain_tree(n), (n_trials, 1)), tokens=tokens, n_nodes=np.full(n_trials, n, np.int32),
                u_accept=uniforms(rng, (n_trials, n)), u_sample=uniforms(rng, (n_trials, n)))


def path_keyed_logits(seed: int, path_tokens, vocab: int) -> np.ndarray:
    """Target logits that depend only on (seed, tokens of the path so far)."""
    return rng_for(seed, 77, len(path_tokens), *path_tokens).normal(0.0, 2.0, vocab).astype(np.float32)


def greedy_tree_trials(seed: int, n_trials: int, vocab: int = 64, max_branch: int = 3, n_nodes: int = 12):
    """Random trees whose target rows are path-keyed; each child's token equals the
    target argmax of its parent with probability 1/2, else a uniform token."""
    trees = []
    rng = rng_for(seed, 78)
    for t in range(n_trials):
        parent = random_tree(rng, n_nodes, max_branch, 6)
        tokens = np.zeros(n_nodes, np.int32)
        tokens[0] = int(rng.integers(vocab))
        paths = [[int(tokens[0])]]
        rows = [path_keyed_logits(seed + t, paths[0], vocab)]
        for c in range(1, n_nodes):
            prow = rows[parent[c]]
            tok = int(np.argmax(prow)) if rng.random() < 0.5 else int(rng.integers(vocab))
            tokens[c] = tok
            paths.append(paths[parent[c]] + [tok])
            rows.append(path_keyed_logits(seed + t, paths[c], vocab))
        trees.append((parent, tokens, np.stack(rows)))
    parent = np.stack([t[0] for t in trees])
    tokens = np.stack([t[1] for t in trees])
    tgt = np.stack([t[2] for t in trees])
    return dict(parent=parent, tokens=tokens, n_nodes=np.full(n_trials, n_nodes, np.int32), tgt_logits=tgt,
                dft_logits=None, u_accept=None, u_sample=None)
