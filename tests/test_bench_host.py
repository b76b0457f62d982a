"""Host-side pieces of bench.py: algorithmic bytes and FLOPs, the roofline entry, the
measured-traffic parser and the deepest-path construction used for the KV-commit
timing.  No GPU."""
import os
import sys

import numpy as np

import support

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import synth  # noqa: E402


def test_algorithmic_bytes_and_flops_of_the_60_node_step():
    inp = support.make_config(2, seed=0, with_kv=False)
    attn, logits, sampling = bench.algorithmic_bytes(inp)
    kv = 2 * (4096 + 60) * 8 * 128 * 2            # K and V of every position, bf16
    qo = 2 * 60 * 32 * 128 * 2                    # Q in, O out
    assert attn == kv + qo == 18006016
    # the draft rows count only at nodes with children (a leaf's draft row takes no part)
    par = inp["parent"][0]
    internal = sum(1 for n in range(60) if (par[n + 1:60] == n).any())
    assert internal == bench.internal_rows(inp) == 13
    assert logits == 60 * 128256 * 4 and sampling == logits + internal * 128256 * 4
    assert bench.attention_flops(inp) == 4 * 32 * 128 * 60 * (4096 + 60)


def test_roofline_switches_to_mfma_above_the_ridge():
    e = bench.roofline_entry("k", 1_000_000, 10.0, None, flops=0)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and abs(e["achieved"] - 100.0) < 1e-9
    ridge = bench.MFMA_BF16_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    below = bench.roofline_entry("k", 1_000_000, 10.0, None, flops=int(0.9 * ridge * 1_000_000))
    above = bench.roofline_entry("k", 1_000_000, 10.0, None, flops=int(1.1 * ridge * 1_000_000))
    assert below["bound"] == "hbm" and above["bound"] == "mfma" and above["unit"] == "TFLOP/s"
    assert abs(above["frac"] - above["achieved"] / bench.MFMA_BF16_PEAK_TFLOPS) < 1e-3


def test_deepest_paths():
    parent = np.array([[-1, 0, 0, 1, 3, 2, -1], [-1, 0, -1, -1, -1, -1, -1]], np.int32)
    path, L = bench.deepest_paths(parent, np.array([6, 2]))
    assert L.tolist() == [3, 1]
    assert path[0, :4].tolist() == [0, 1, 3, 4] and path[1, :2].tolist() == [0, 1]


def test_measured_traffic_matches_the_committed_sources():
    # the committed counter summary lists the sources' hashes; bench reports traffic only
    # while they match, and the values are per-call byte counts
    t = bench.measured_traffic()
    for call in ("spec_tree_attention", "spec_tree_softmax_pair"):
        assert call in t
        assert t[call] is None or t[call] > 10_000_000


def test_measured_traffic_covers_the_sampling_branch():
    t = bench.measured_traffic()
    assert "sampling_branch" in t
    if t["sampling_branch"] is not None and t["spec_tree_softmax_pair"] is not None:
        assert t["sampling_branch"] > t["spec_tree_softmax_pair"]  # the sampler's own traffic comes on top


def test_oracle_check_counts_identical_and_flagged_walks():
    """bench.oracle_check on outputs that equal the oracle's (all identical) and on
    outputs with one request altered (one fewer); the near-tie count is the oracle's."""
    import oracle

    inp = synth.make_config(1, seed=3, with_kv=False)
    m = 6
    rng = synth.rng_for(70)
    first = {k: np.repeat(inp[k][:1], m, 0) for k in ("parent", "tokens", "n_nodes")}
    first["u_accept"] = synth.uniforms(rng, (m, inp["n_max"]))
    first["u_sample"] = synth.uniforms(rng, (m, inp["n_max"]))
    tgt = np.broadcast_to(inp["tgt_logits"][:1], (m,) + inp["tgt_logits"].shape[1:])
    dft = np.broadcast_to(inp["dft_logits"][:1], (m,) + inp["dft_logits"].shape[1:])
    r = oracle.reject_sample(tgt, dft, inp["T"], inp["Td"], first["tokens"], first["parent"], first["n_nodes"],
                             first["u_accept"], first["u_sample"])
    r.update(oracle.accept_path(r["accepted_child"], r["term_token"], first["tokens"], first["n_nodes"]))
    first["out"] = {k: r[k].copy() for k in ("path_nodes", "out_tokens", "accepted_child", "term_token")}
    got = bench.oracle_check(inp, first, m=m)
    flagged = sum(int(r["tie_flags"][b][r["path_nodes"][b][r["path_nodes"][b] >= 0]].any()) for b in range(m))
    assert got == {"trials": m, "near_tie_requests": flagged, "identical_to_oracle": m}
    first["out"]["term_token"][2, 0] += 1
    assert bench.oracle_check(inp, first, m=m)["identical_to_oracle"] == m - 1
