"""Checks of the seeded input generators: the EAGLE-2 expand example printed by the
notes on tree verification (part E.3), the value product rule of the worked example
(part G), tree shapes, and seed reproducibility."""
import json
import os

import numpy as np

from tree_verification_masked_amd import synth


def test_expand_step_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "expand_step.json")))
    kept, vals, parents = synth.expand_step(g["frontier_values"], g["k"], g["child_confidences_of_kept"])
    assert kept.tolist() == g["kept_frontier_indices"]
    np.testing.assert_allclose(np.sort(vals)[::-1], g["new_frontier_values_sorted"], rtol=0, atol=1e-12)
    # a strong child of the weaker parent outranks a weak child of the stronger parent
    assert vals[parents == 1].max() > vals[parents == 0].min()


def test_worked_example_values_follow_the_product_rule(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))["printed_by_the_page"]
    conf = g["draft_confidence"]
    _, lvl1, _ = synth.expand_step([1.0], 1, [[conf["1"], conf["2"]]])
    _, lvl2, _ = synth.expand_step(list(lvl1), 2, [[conf["3"], conf["4"]], [conf["5"], conf["6"]]])
    np.testing.assert_allclose([1.0] + list(lvl1) + list(lvl2), g["node_values"], rtol=0, atol=1e-12)


def test_uniforms_are_exact_and_open():
    u = synth.uniforms(synth.rng_for(1), 1 << 20)
    assert u.dtype == np.float32 and (u > 0).all() and (u < 1).all()
    k = (u.astype(np.float64) * 2 ** 24 - 1) / 2
    assert np.array_equal(k, np.round(k))


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # exact ties round to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), ref)


def test_eagle2_tree_shape():
    src = synth.RowSource(5, 4096, "normal", sigma_t=3.0, sigma_d=1.0)
    parent, tokens, uids, values = synth.eagle2_tree(src, 10, 6, 60, 1.0, root_token=3)
    assert parent.size == 60 and parent[0] == -1
    assert all(0 <= parent[i] < i for i in range(1, 60))
    depth = np.zeros(60, int)
    for i in range(1, 60):
        depth[i] = depth[parent[i]] + 1
    assert (np.diff(depth) >= 0).all()  # breadth-first order
    assert depth.max() <= 6
    for i in range(1, 60):  # values never grow along a path
        assert values[i] <= values[parent[i]] + 1e-15
    for p in range(60):  # siblings have distinct tokens (top-k of one draft row)
        kids = tokens[parent == p]
        assert len(set(kids.tolist())) == kids.size


def test_configs_are_reproducible_and_shaped():
    a = synth.make_config(1, seed=3)
    b = synth.make_config(1, seed=3)
    c = synth.make_config(1, seed=4)
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
    c2 = synth.make_config(2, seed=1, ctx_override=64, vocab_override=2048)
    assert c2["parent"].shape == (1, 60) and c2["k"].dtype == np.uint16 and c2["hq"] == 32
    c3 = synth.make_config(3, seed=1, ctx_override=64, vocab_override=2048)
    assert c3["parent"][0].tolist() == list(range(-1, 15)) and c3["T"] == float(np.float32(0.7))
    c4 = synth.make_config(4, seed=1, ctx_override=100, vocab_override=2048)
    assert c4["B"] == 8 and c4["block_table"] is not None and c4["page_size"] == 16
    used = c4["block_table"][c4["block_table"] >= 0]
    assert len(set(used.tolist())) == used.size and used.max() < c4["n_pages"]
    for b in range(8):
        need = -(-(c4["ctx_len"][b] + c4["n_nodes"][b]) // 16)
        assert (c4["block_table"][b, :need] >= 0).all()
    c5 = synth.make_config(5, seed=1, ctx_override=64, vocab_override=2048)
    assert c5["parent"].shape == (1, 64) and c5["hq"] == 64
