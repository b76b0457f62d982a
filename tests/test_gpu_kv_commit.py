"""GPU parity of spec_tree_kv_commit against the CPU oracle: the cache after the
commit, the committed lengths, the released pages and the page table, bit-exact
(the commit only moves bytes)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from tree_verification_masked_amd import binding as B
import synth
import support
from tree_verification_masked_amd.step import VerifyStep, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _to_dev(a, bf16):
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _from_dev(t, bf16):
    if bf16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _paths(rng, n_nodes, n_max, kinds):
    """One path per request: an increasing walk from the root inside the tree."""
    Bn = len(n_nodes)
    path = np.full((Bn, n_max), -1, np.int32)
    al = np.zeros(Bn, np.int32)
    for b in range(Bn):
        n = int(n_nodes[b])
        path[b, 0] = 0
        kind = kinds[b % len(kinds)]
        if kind == "chain":  # every node accepted: the identity move
            L = n - 1
            path[b, 1:n] = np.arange(1, n)
        elif kind == "none":
            L = 0
        elif kind == "shift":  # 0 -> 2 -> 3 -> ...: each destination is an earlier source
            L = max(0, n - 2)
            path[b, 1:L + 1] = np.arange(2, n)
        elif kind == "refused":
            L = -1
        elif kind == "invalid":  # not increasing
            L = min(2, n - 1)
            if L == 2:
                path[b, 1:3] = [2, 1]
            else:
                L = -1
        else:
            L = int(rng.integers(0, n))
            path[b, 1:L + 1] = np.sort(rng.choice(np.arange(1, n), size=L, replace=False))
        al[b] = L
    return path, al


@pytest.mark.parametrize("bf16,paged,d,hkv,page,layers", [
    (True, False, 128, 8, 0, 1), (False, False, 64, 4, 0, 1), (True, True, 128, 8, 16, 1), (False, True, 64, 2, 1, 1),
    (True, True, 64, 4, 7, 1), (True, False, 128, 8, 0, 5), (False, True, 64, 2, 3, 3)])
def test_kv_commit_parity(bf16, paged, d, hkv, page, layers):
    say("kv_commit", bf16, paged, d, hkv, page, layers)
    rng = np.random.default_rng(d + hkv + page)
    Bn, n_max = 7, 40
    n_nodes = rng.integers(1, n_max + 1, size=Bn).astype(np.int32)
    n_nodes[0] = n_max
    n_nodes[5] = max(n_nodes[5], 3)  # room for the invalid (non-increasing) path
    ctx = rng.integers(0, 300, size=Bn).astype(np.int32)
    kinds = ["random", "chain", "none", "shift", "refused", "invalid", "random"]
    path, al = _paths(rng, n_nodes, n_max, kinds)
    if paged:
        need = [-(-(int(ctx[b]) + int(n_nodes[b])) // page) for b in range(Bn)]
        n_pages = sum(need) + 3
        perm = rng.permutation(n_pages).astype(np.int32)
        cap = max(need) + 2
        bt = np.full((Bn, cap), -1, np.int32)
        o = 0
        for b in range(Bn):
            bt[b, :need[b]] = perm[o:o + need[b]]
            o += need[b]
        shape = (n_pages, page, hkv, d)
    else:
        bt, n_pages, cap = None, 0, int(ctx.max()) + n_max + 5
        shape = (Bn, cap, hkv, d)
    if layers > 1:  # every layer's cache, stacked on a leading axis
        shape = (layers,) + shape
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if bf16:
        k, v = synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    rk, rv, rlen, rfreed, rbt = oracle.kv_commit(k, v, ctx, n_nodes, path, al, block_table=bt, page_size=page,
                                                 n_pages=n_pages)
    gk, gv = _to_dev(k, bf16), _to_dev(v, bf16)
    gbt = None if bt is None else torch.from_numpy(bt.copy()).cuda()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    new_len = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    freed = torch.zeros((Bn, 64), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.spec_tree_kv_commit(gk, gv, i32(ctx), i32(n_nodes), i32(path), i32(al), new_len, freed, block_table=gbt,
                          page_size=page, n_pages=n_pages, status=status)
    torch.cuda.synchronize()
    assert new_len.cpu().numpy().tolist() == rlen.tolist()
    assert np.array_equal(_from_dev(gk, bf16), rk) and np.array_equal(_from_dev(gv, bf16), rv)
    if paged:
        assert np.array_equal(freed.cpu().numpy(), rfreed)
        assert np.array_equal(gbt.cpu().numpy(), rbt)
    assert int(status.item()) == -4  # SPEC_ERR_BAD_INPUT, from the "invalid" request
    assert rlen[4] == -1 and rlen[5] == -1  # refused and invalid requests stay untouched


@pytest.mark.parametrize("cfg", [2, 4])
def test_kv_commit_after_the_full_step(cfg):
    """The step's own path, committed on the step's cache (config 4 is paged)."""
    say("kv_commit after step", cfg)
    inp = support.make_config(cfg, seed=5, T=1.0)
    d = to_device(inp)
    st = VerifyStep(d)
    st.run()
    got = st.results()
    assert got["status"][0] == 0
    k, v = d["k"].clone(), d["v"].clone()
    bt = None if d.get("block_table") is None else d["block_table"].clone()
    Bn = inp["B"]
    new_len = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    freed = torch.zeros((Bn, 64), dtype=torch.int32, device="cuda")
    B.spec_tree_kv_commit(k, v, d["ctx_len"], d["n_nodes"], st.path_nodes, st.accept_len, new_len, freed,
                          block_table=bt, page_size=inp.get("page_size", 0), n_pages=inp.get("n_pages", 0),
                          status=st.status)
    torch.cuda.synchronize()
    rk, rv, rlen, rfreed, rbt = oracle.kv_commit(inp["k"], inp["v"], inp["ctx_len"], inp["n_nodes"], got["path_nodes"],
                                                 got["accept_len"], block_table=inp.get("block_table"),
                                                 page_size=inp.get("page_size", 0), n_pages=inp.get("n_pages", 0))
    assert int(st.status.item()) == 0
    assert new_len.cpu().numpy().tolist() == rlen.tolist()
    assert (rlen == inp["ctx_len"] + 1 + got["accept_len"]).all()
    assert np.array_equal(_from_dev(k, True), rk) and np.array_equal(_from_dev(v, True), rv)
    if bt is not None:
        assert np.array_equal(bt.cpu().numpy(), rbt) and np.array_equal(freed.cpu().numpy(), rfreed)
