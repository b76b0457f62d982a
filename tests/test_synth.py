"""Checks of the seeded input generators: tree shapes of every workload (the EAGLE-2
trees of workloads 2 and 5 through the tree-builder hook, with the CPU oracle's
builder), path-keyed rows, exact uniforms and seed reproducibility.  The EAGLE-2
value arithmetic itself (part E.3's expand example, part G's product rule) is pinned
in test_oracle_tree_build.py: this module holds no tree-construction method."""
import json
import os

import numpy as np

import synth
import support


def test_uniforms_are_exact_and_half_open():
    u = synth.uniforms(synth.rng_for(1), 1 << 22)
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()
    k = u.astype(np.float64) * 2 ** 24
    assert np.array_equal(k, np.round(k))
    assert (k % 2 == 0).any() and (k % 2 == 1).any()  # the whole 2^-24 grid, not every other point
    assert k.min() < 2 ** 8 and k.max() > 2 ** 24 - 2 ** 8


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # exact ties round to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), ref)


def test_eagle2_tree_shape():
    inp = support.make_config(2, seed=5, ctx_override=32, vocab_override=4096, with_kv=False)
    parent, tokens = inp["parent"][0], inp["tokens"][0]
    assert parent.size == 60 and parent[0] == -1
    assert all(0 <= parent[i] < i for i in range(1, 60))
    depth = np.zeros(60, int)
    for i in range(1, 60):
        depth[i] = depth[parent[i]] + 1
    assert (np.diff(depth) >= 0).all()  # breadth-first order
    assert depth.max() <= 6
    for p in range(60):  # siblings have distinct tokens (top-k of one draft row)
        kids = tokens[parent == p]
        assert len(set(kids.tolist())) == kids.size
    # every node's rows are the path-keyed rows of its root path, and each child's
    # token is among the top-10 of its parent's draft row
    for i in range(1, 60):
        path, j = [], i
        while j >= 0:
            path.append(int(tokens[j]))
            j = int(parent[j])
        t, d = synth.path_rows(5 * 7919 + 2, path[::-1], 4096)
        assert np.array_equal(inp["tgt_logits"][0, i], t) and np.array_equal(inp["dft_logits"][0, i], d)
        top = np.argsort(-inp["dft_logits"][0, parent[i]].astype(np.float64), kind="stable")[:10]
        assert tokens[i] in top


def test_eagle2_workloads_need_a_tree_builder():
    import pytest
    with pytest.raises(ValueError):
        synth.make_config(2, seed=1, ctx_override=64, vocab_override=2048)


def test_path_row_is_the_draft_row_of_path_rows():
    t, d = synth.path_rows(3, (5, 9, 2), 1000)
    assert np.array_equal(synth.path_row(3, (5, 9, 2), 1000), d)
    assert not np.array_equal(t, d)


def test_configs_are_reproducible_and_shaped():
    a = support.make_config(1, seed=3)
    b = support.make_config(1, seed=3)
    c = support.make_config(1, seed=4)
    for key in ("parent", "tokens", "tgt_logits", "dft_logits", "u_accept", "u_sample", "q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["tgt_logits"], c["tgt_logits"])
    assert a["parent"].tolist() == [[-1, 0, 0, 1, 1, 2, 2]]
    assert a["q"].shape == (1, 7, 4, 64) and a["k"].shape == (1, 128 + 7, 4, 64)
    # children are the top-2 draft tokens of their parent, in descending draft logit
    for p in range(3):
        kids = [c for c in range(7) if a["parent"][0, c] == p]
        top = np.argsort(-a["dft_logits"][0, p], kind="stable")[:2]
        assert a["tokens"][0, kids].tolist() == top.tolist()


def test_small_variants_of_the_large_workloads():
    c2 = support.make_config(2, seed=1, ctx_override=64, vocab_override=2048)
    assert c2["parent"].shape == (1, 60) and c2["k"].dtype == np.uint16 and c2["hq"] == 32
    c3 = support.make_config(3, seed=1, ctx_override=64, vocab_override=2048)
    assert c3["parent"][0].tolist() == list(range(-1, 15)) and c3["T"] == float(np.float32(0.7))
    c4 = support.make_config(4, seed=1, ctx_override=100, vocab_override=2048)
    assert c4["B"] == 8 and c4["block_table"] is not None and c4["page_size"] == 16
    used = c4["block_table"][c4["block_table"] >= 0]
    assert len(set(used.tolist())) == used.size and used.max() < c4["n_pages"]
    for b in range(8):
        need = -(-(c4["ctx_len"][b] + c4["n_nodes"][b]) // 16)
        assert (c4["block_table"][b, :need] >= 0).all()
    c5 = support.make_config(5, seed=1, ctx_override=64, vocab_override=2048)
    assert c5["parent"].shape == (1, 64) and c5["hq"] == 64
