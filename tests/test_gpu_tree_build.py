"""GPU parity of the EAGLE-2 draft-tree construction (spec_tree_build_init,
spec_tree_expand, spec_tree_rerank) against the oracle: after every expand round the
node arrays (parent, token, path key exactly; value and confidence within 1e-5
relative) and the frontier; after the rerank the flattened tree, bit for bit.
Decisions the oracle records as near ties (two values within 1e-5) may legitimately
differ; such requests are counted and only checked for validity."""
import sys

import numpy as np
import pytest
import torch

from oracle import tree_build as otb
from tree_verification_masked_amd import binding as B
import synth
from tree_verification_masked_amd.draft_tree import DraftTree

pytestmark = pytest.mark.gpu
BAD_INPUT = -4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def gpu_path_tokens(st, b, nd):
    out = []
    while nd >= 0:
        out.append(int(st["token"][b, nd]))
        nd = int(st["parent"][b, nd])
    return tuple(out[::-1])


def oracle_path_keys(o):
    keys = []
    for i in range(len(o.parent)):
        d, key, nd = o.depth[i], np.uint64(o.depth[i]) << np.uint64(60), i
        while nd > 0:
            key |= np.uint64(o.rank[nd]) << np.uint64(60 - 4 * o.depth[nd])
            nd = o.parent[nd]
        keys.append(key)
    return np.array(keys, np.uint64)


def compare_state(st, b, o, tag):
    n = len(o.parent)
    assert st["count"][b] == n, tag
    assert st["parent"][b, :n].tolist() == o.parent, tag
    assert st["token"][b, :n].tolist() == o.token, tag
    assert np.array_equal(st["path"][b, :n], oracle_path_keys(o)), tag
    assert np.allclose(st["value"][b, :n], o.value, rtol=1e-5, atol=0), tag
    assert np.allclose(st["conf"][b, :n], o.conf, rtol=1e-5, atol=0), tag
    fc = st["frontier_count"][b]
    assert fc == len(o.frontier) and st["frontier"][b, :fc].tolist() == o.frontier, tag


def run_build(Bn, V, k, depth, n_final, T_d, kind, seed, select_k=None, cap=1024, scale=3.0, noise=1.0,
              row_hook=None, policy="layer"):
    sk = k if select_k is None else select_k
    R = max(sk, 1)
    rng = np.random.default_rng(seed)
    roots = rng.integers(0, V, size=Bn).astype(np.int32)
    dt = DraftTree(Bn, cap, R, V)
    dt.init(torch.from_numpy(roots).cuda())
    orc = [otb.TreeBuild(int(r)) for r in roots]
    tied = set()

    def row(path):
        r = synth.path_row(seed, path, V, kind, scale, noise)
        return row_hook(path, r) if row_hook else r

    for rnd in range(depth):
        st = dt.host_state()
        rows = np.zeros((Bn, R, V), np.float32)
        for b in range(Bn):
            for j in range(int(st["frontier_count"][b])):
                rows[b, j] = row(gpu_path_tokens(st, b, int(st["frontier"][b, j])))
        for b, o in enumerate(orc):
            if o.frontier:
                o.expand([row(otb.path_tokens(o, nd)) for nd in o.frontier], T_d, k, sk, policy)
        dt.expand(torch.from_numpy(rows).cuda(), T_d, k, sk, policy=policy)
        st = dt.host_state()
        assert st["status"][0] == 0
        for b, o in enumerate(orc):
            if o.ties:
                tied.add(b)
            if b not in tied:
                compare_state(st, b, o, f"request {b} round {rnd}")
    parent, tokens, n_nodes, cand_id = (t.cpu().numpy() for t in dt.rerank(n_final))
    assert dt.host_state()["status"][0] == 0
    for b, o in enumerate(orc):
        op, ot, oid = o.rerank(n_final)
        n = len(op)
        assert n_nodes[b] == n
        pb = parent[b, :n]
        assert pb[0] == -1 and np.all(pb[1:] < np.arange(1, n)) and np.all(pb[1:] >= 0)  # always a valid tree
        assert np.all(parent[b, n:] == -1) and np.all(tokens[b, n:] == -1) and np.all(cand_id[b, n:] == -1)
        if o.ties:
            tied.add(b)
        if b not in tied:
            assert pb.tolist() == op.tolist() and tokens[b, :n].tolist() == ot.tolist()
            assert cand_id[b, :n].tolist() == oid.tolist()
    return dt, (parent, tokens, n_nodes, cand_id), orc, tied


@pytest.mark.parametrize("Bn,V,k,depth,n,T,kind,sk", [
    (3, 1000, 4, 4, 20, 1.0, "normal", None),      # vocabulary not a multiple of 4: scalar loads
    (2, 4096 * 3, 5, 5, 30, 0.7, "normal", 3),     # select_k below top_k
    (4, 32000, 8, 3, 64, 1.5, "student_t", None),
    (1, 8195, 16, 3, 64, 1.0, "normal", 16),       # widest frontier and fan-out; ragged last chunk
])
def test_build_small(Bn, V, k, depth, n, T, kind, sk):
    say("tree build", Bn, V, k, depth, n, T, kind, sk)
    _, _, _, tied = run_build(Bn, V, k, depth, n, T, kind, seed=V + k, select_k=sk)
    assert len(tied) == 0


def test_build_llama8b_shape():
    # top-k 10, depth 6, 60 nodes over a 128256-token vocabulary (the 60-node verify tree)
    say("tree build 128256 k10 d6 n60")
    dt, out, orc, tied = run_build(1, 128256, 10, 6, 60, 1.0, "normal", seed=11, scale=3.0, noise=1.0)
    assert len(tied) == 0 and out[2][0] == 60
    assert int(dt.host_state()["count"][0]) == 1 + 10 + 5 * 100


def test_build_long_context_shard_shape():
    # top-k 8, depth 8, 64 nodes, 152064 tokens, 2 t(3) logits with noise 1.5
    say("tree build 152064 k8 d8 n64")
    dt, out, orc, tied = run_build(1, 152064, 8, 8, 64, 1.0, "student_t", seed=12, scale=2.0, noise=1.5)
    assert len(tied) == 0 and out[2][0] == 64


def test_tree_feeds_the_mask_build():
    say("tree build -> mask build")
    dt, (parent, tokens, n_nodes, cand_id), _, _ = run_build(2, 5000, 6, 5, 48, 1.0, "normal", seed=5)
    anc = torch.zeros((2, 48), dtype=torch.int64, device="cuda")
    child = torch.zeros_like(anc)
    depth = torch.zeros((2, 48), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.spec_tree_mask_build(torch.from_numpy(parent).cuda(), torch.from_numpy(n_nodes).cuda(), anc, child, depth,
                           status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st = dt.host_state()
    d = depth.cpu().numpy()
    for b in range(2):  # the mask build's depths are the path keys' depths
        n = int(n_nodes[b])
        assert d[b, :n].tolist() == [int(st["path"][b, i] >> np.uint64(60)) for i in cand_id[b, :n]]


def test_degenerate_rows_and_edges():
    say("tree build: -inf entries, vocab = top_k, n_final above the node count")

    def few_finite(path, r):  # only 3 finite logits: the other children get confidence 0
        out = np.full_like(r, -np.inf)
        out[:3] = r[:3]
        return out

    run_build(2, 4000, 5, 3, 40, 1.0, "normal", seed=21, row_hook=few_finite)
    run_build(1, 4, 4, 3, 64, 1.0, "normal", seed=22)  # the whole vocabulary as children
    _, out, orc, _ = run_build(2, 300, 3, 1, 10, 1.0, "normal", seed=23)
    assert out[2].tolist() == [4, 4]


def _empty_rows(dt):
    return torch.zeros((dt.batch, dt.R, dt.vocab), dtype=torch.float32, device="cuda")


def test_depth_limit_and_capacity():
    say("tree build: depth 15 limit, capacity")
    V = 64
    dt = DraftTree(1, 1024, 1, V)
    dt.init(torch.tensor([3], dtype=torch.int32, device="cuda"))
    rows = _empty_rows(dt)
    rows[0, 0] = torch.arange(V, dtype=torch.float32, device="cuda")
    for _ in range(15):  # a chain to depth 15
        dt.expand(rows, 1.0, 1)
    st = dt.host_state()
    assert st["status"][0] == 0 and st["count"][0] == 16 and st["frontier_count"][0] == 1
    dt.expand(rows, 1.0, 1)  # its frontier sits at depth 15: refused
    st = dt.host_state()
    assert st["status"][0] == BAD_INPUT and st["count"][0] == 16 and st["frontier_count"][0] == 0
    dt.expand(rows, 1.0, 1)  # nothing left to grow: a no-op
    assert dt.host_state()["count"][0] == 16
    parent, tokens, n_nodes, _ = dt.rerank(64)
    assert n_nodes.item() == 16 and parent.cpu().numpy()[0, :16].tolist() == [-1] + list(range(15))

    dt = DraftTree(1, 20, 4, V)
    dt.init(torch.tensor([0], dtype=torch.int32, device="cuda"))
    rows = _empty_rows(dt)
    rows[0, :] = torch.arange(V, dtype=torch.float32, device="cuda")
    dt.expand(rows, 1.0, 4)  # 5 nodes
    dt.expand(rows, 1.0, 4)  # 21 > 20: refused
    st = dt.host_state()
    assert st["status"][0] == BAD_INPUT and st["count"][0] == 5 and st["frontier_count"][0] == 0


def test_bad_row_stops_only_its_request():
    say("tree build: NaN row")
    V, k = 2000, 4
    seed = 31

    dt = DraftTree(2, 1024, k, V)
    roots = np.array([5, 6], np.int32)
    dt.init(torch.from_numpy(roots).cuda())
    o = otb.TreeBuild(5)
    rows = np.zeros((2, k, V), np.float32)
    rows[0, 0] = synth.path_row(seed, (5,), V)
    rows[1, 0] = synth.path_row(seed, (6,), V)
    rows[1, 0, 17] = np.nan
    dt.expand(torch.from_numpy(rows).cuda(), 1.0, k)
    o.expand([rows[0, 0]], 1.0, k, k)
    st = dt.host_state()
    assert st["status"][0] == BAD_INPUT
    assert st["count"][1] == 1 and st["frontier_count"][1] == 0
    compare_state(st, 0, o, "healthy request beside a bad one")


@pytest.mark.parametrize("Bn,V,k,sk,rounds,n", [
    (2, 3000, 4, 1, 12, 24),      # the one-pop heap
    (3, 1000, 3, 2, 10, 30),      # scalar loads, two pops per round
    (1, 128256, 8, 4, 8, 64),     # full vocabulary
])
def test_best_first_parity(Bn, V, k, sk, rounds, n):
    say("tree build best-first", Bn, V, k, sk, rounds, n)
    _, _, orc, tied = run_build(Bn, V, k, rounds, n, 1.0, "normal", seed=V + sk, select_k=sk, policy="best_first")
    assert len(tied) == 0
    # the heap goes back to shallower nodes: some expanded node is not on the last
    # round's depth (unlike the layer policy)
    depths = [o.depth[i] for o in orc for i in set(o.parent[1:])]
    assert len(set(depths)) > 1


def test_best_first_stops_at_the_depth_limit():
    say("tree build best-first: depth 15")
    V = 64
    dt = DraftTree(1, 1024, 1, V)
    dt.init(torch.tensor([3], dtype=torch.int32, device="cuda"))
    rows = _empty_rows(dt)
    rows[0, 0] = torch.arange(V, dtype=torch.float32, device="cuda")
    for _ in range(15):  # a chain: its only leaf reaches depth 15, which is not grown
        dt.expand(rows, 1.0, 1, policy="best_first")
    st = dt.host_state()
    assert st["status"][0] == 0 and st["count"][0] == 16 and st["frontier_count"][0] == 0
    dt.expand(rows, 1.0, 1, policy="best_first")  # nothing left to grow: a no-op
    st = dt.host_state()
    assert st["status"][0] == 0 and st["count"][0] == 16
