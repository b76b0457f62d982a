"""Pins of the oracle's tree rejection sampling and accept-path walk.

What pins it (none of these compares against another implementation):
  * the worked example of the notes on tree verification (part G), reproduced by hand
    in tests/golden/worked_example.json, plus two hand-computed variants of it;
  * losslessness (notes part C; the acceptance rule of the gingerlabs page): over 10^6
    seeded trials on a 16-token vocabulary, the first emitted token is distributed as p
    for several kinds of q and sibling counts, and the second token as the target's
    conditional, by a chi-square test;
  * chain acceptance (notes parts A and D.1): P(accept_len >= d) = alpha^d;
  * greedy verification equals a target-only greedy decode (gingerlabs page,
    evaluation protocol);
  * special cases: q = p always accepts; disjoint supports never accept and the bonus
    is then distributed as p; T -> 0+ reproduces greedy.
"""
import json
import os

import numpy as np
import pytest
import scipy.stats

import oracle
import synth

TRIALS = 1_000_000


def _run(inp, T=1.0, Td=1.0, mode="lazy"):
    r = oracle.reject_sample(inp["tgt_logits"], inp["dft_logits"], T, Td, inp["tokens"], inp["parent"],
                             inp["n_nodes"], inp["u_accept"], inp["u_sample"], mode=mode)
    r.update(oracle.accept_path(r["accepted_child"], r["term_token"], inp["tokens"], inp["n_nodes"]))
    return r


def _chi2_p(observed, probs):
    """Chi-square goodness of fit, merging cells whose expected count is below 5."""
    observed = np.asarray(observed, np.float64)
    expected = np.asarray(probs, np.float64) * observed.sum()
    assert observed[expected == 0].sum() == 0, "an impossible outcome was emitted"
    keep = expected >= 5
    obs = list(observed[keep])
    exp = list(expected[keep])
    if (~keep).any() and expected[~keep].sum() > 0:
        obs.append(observed[~keep].sum())
        exp.append(expected[~keep].sum())
    if len(obs) < 2:
        return 1.0
    return scipy.stats.chisquare(obs, exp).pvalue


# ---------------------------------------------------------------- worked example

def _worked_inputs(g, scen):
    tgt = synth.log_probs_f32(np.array(g["target_probs"]))[None]
    dft = synth.log_probs_f32(np.array(g["draft_probs"]))[None]
    return dict(tgt_logits=tgt, dft_logits=dft, tokens=np.array([g["tokens"]], np.int32),
                parent=np.array([g["printed_by_the_page"]["parent"]], np.int32), n_nodes=np.array([7], np.int32),
                u_accept=np.array([scen["u_accept"]], np.float32), u_sample=np.array([scen["u_sample"]], np.float32))


@pytest.mark.parametrize("mode", ["lazy", "all"])
def test_worked_example_by_hand(golden_dir, mode):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    page = g["printed_by_the_page"]
    tp, dp = np.array(g["target_probs"]), np.array(g["draft_probs"])
    # the fixture encodes the numbers the page prints
    assert tp[0, 0] == page["p_root_of_一"] and dp[0, 0] == page["q_root_of_一"]
    assert tp[1, 4] == page["p_node1_of_百"] and dp[1, 4] == page["q_node1_of_百"]
    assert g["scenarios"][0]["u_accept"][3] == page["uniform_for_node3"]
    for scen in g["scenarios"]:
        r = _run(_worked_inputs(g, scen), mode=mode)
        L = scen["accept_len"]
        assert r["accept_len"][0] == L, scen["name"]
        assert r["path_nodes"][0, :L + 1].tolist() == scen["path_nodes"]
        assert (r["path_nodes"][0, L + 1:] == -1).all()
        assert r["out_tokens"][0, :L + 1].tolist() == scen["out_tokens"]
        assert (r["tie_flags"][0, scen["path_nodes"]] == 0).all()
    # the page's own run emits three tokens: 一, 百 and the bonus 万
    assert len(g["scenarios"][0]["out_tokens"]) == page["tokens_emitted"]


def test_worked_example_lazy_and_all_agree_on_visited_nodes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    for scen in g["scenarios"]:
        inp = _worked_inputs(g, scen)
        lazy, full = _run(inp, mode="lazy"), _run(inp, mode="all")
        seen = lazy["accepted_child"][0] != oracle.NOT_EVALUATED
        assert (lazy["accepted_child"][0][seen] == full["accepted_child"][0][seen]).all()
        assert (lazy["term_token"][0][seen] == full["term_token"][0][seen]).all()
        assert (full["accepted_child"][0] != oracle.NOT_EVALUATED).all()


# ---------------------------------------------------------------- losslessness

def _p_root(seed):
    rng = synth.rng_for(seed, 500)
    p = rng.dirichlet(np.full(16, 0.7))
    p[int(rng.integers(16))] = 0.0  # a zero in p as well
    return p / p.sum()


@pytest.mark.parametrize("qkind,k", [("noisy", 1), ("uniform", 1), ("equal", 2), ("zeros", 2), ("onehot", 4),
                                      ("noisy", 4), ("zeros", 4), ("noisy", 2)])
def test_first_token_is_distributed_as_p(qkind, k):
    seed = 1000 + 10 * k + len(qkind)
    p = _p_root(seed)
    rng = synth.rng_for(seed, 501)
    q = synth.q_variant(qkind, p, rng)
    counts = np.zeros(16)
    for chunk in range(5):
        tr = synth.star_trials(rng, p, q, k, TRIALS // 5)
        r = _run(tr)
        counts += np.bincount(r["out_tokens"][:, 0], minlength=16)
    pv = _chi2_p(counts, p)
    assert pv > 0.01, (qkind, k, pv)


def test_disjoint_supports_never_accept_and_bonus_is_p():
    p = np.zeros(16)
    q = np.zeros(16)
    p[:8] = synth.rng_for(7, 1).dirichlet(np.ones(8))
    q[8:] = synth.rng_for(7, 2).dirichlet(np.ones(8))
    rng = synth.rng_for(7, 3)
    tr = synth.star_trials(rng, p, q, 3, TRIALS)
    r = _run(tr)
    assert (r["accept_len"] == 0).all()
    assert _chi2_p(np.bincount(r["out_tokens"][:, 0], minlength=16), p) > 0.01


def test_second_token_follows_the_target_conditional():
    V = 16
    rng = synth.rng_for(8, 1)
    p_root = rng.dirichlet(np.ones(V))
    q_root = synth.q_variant("noisy", p_root, rng)
    P2 = rng.dirichlet(np.ones(V), size=V)
    Q2 = np.stack([synth.q_variant("noisy", P2[t], rng) for t in range(V)])
    firsts, seconds = [], []
    for chunk in range(5):
        tr = synth.depth2_trials(rng, p_root, q_root, P2, Q2, 2, 2, TRIALS // 5)
        r = _run(tr)
        firsts.append(r["out_tokens"][:, 0])
        ok = r["accept_len"] >= 1
        seconds.append(np.stack([r["out_tokens"][ok, 0], r["out_tokens"][ok, 1]], 1))
    first = np.concatenate(firsts)
    assert _chi2_p(np.bincount(first, minlength=V), p_root) > 0.01
    pairs = np.concatenate(seconds)
    # given an accepted first token t1, the second emitted token is distributed as P2[t1]
    stat, dof = 0.0, 0
    for t1 in range(V):
        sel = pairs[pairs[:, 0] == t1, 1]
        if sel.size < 50:
            continue
        obs = np.bincount(sel, minlength=V).astype(float)
        exp = P2[t1] * sel.size
        keep = exp >= 5
        o = list(obs[keep]) + ([obs[~keep].sum()] if (~keep).any() else [])
        e = list(exp[keep]) + ([exp[~keep].sum()] if (~keep).any() else [])
        stat += sum((oi - ei) ** 2 / ei for oi, ei in zip(o, e))
        dof += len(o) - 1
    assert scipy.stats.chi2.sf(stat, dof) > 0.01


# ---------------------------------------------------------------- chains: alpha^d

def test_chain_acceptance_is_alpha_to_the_d(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "chain_alpha.json")))
    alpha = g["alpha"]
    # the page's rounded figures are alpha^4 and alpha^8
    assert round(alpha ** 4, 2) == g["printed"]["d4"] and round(alpha ** 8, 3) == g["printed"]["d8"]
    p, q = synth.alpha_pq(alpha)
    assert abs(np.minimum(p, q).sum() - alpha) < 1e-15
    rng = synth.rng_for(9, 1)
    tr = synth.chain_trials(rng, p, q, 8, TRIALS)
    r = _run(tr)
    L = r["accept_len"]
    n = L.size
    for d in range(1, 9):
        emp = (L >= d).mean()
        sd = np.sqrt(alpha ** d * (1 - alpha ** d) / n)
        assert abs(emp - alpha ** d) < 5 * sd, (d, emp, alpha ** d)
    # after a rejection the bonus comes from the residual, which is uniform on A
    rej = L < 8
    bonus = r["out_tokens"][np.arange(n)[rej], L[rej]]
    assert set(np.unique(bonus)) <= set(range(8, 12))
    assert _chi2_p(np.bincount(bonus - 8, minlength=4), np.full(4, 0.25)) > 0.01


def test_q_equal_p_accepts_every_drafted_token():
    rng = synth.rng_for(10, 1)
    p = rng.dirichlet(np.ones(16))
    tr = synth.chain_trials(rng, p, p.copy(), 6, 20000)
    tr["dft_logits"] = tr["tgt_logits"].copy()  # bitwise identical rows
    r = _run(tr)
    assert (r["accept_len"] == 6).all()


# ---------------------------------------------------------------- greedy

def test_greedy_equals_target_only_decode():
    seed, V = 21, 64
    tr = synth.greedy_tree_trials(seed, 300, vocab=V)
    r = oracle.reject_sample(tr["tgt_logits"], None, 0.0, 1.0, tr["tokens"], tr["parent"], tr["n_nodes"], None,
                             None)
    r.update(oracle.accept_path(r["accepted_child"], r["term_token"], tr["tokens"], tr["n_nodes"]))
    lens = r["accept_len"]
    assert lens.max() >= 2 and (lens == 0).any()
    for t in range(lens.size):
        seq = [int(tr["tokens"][t, 0])]
        for _ in range(lens[t] + 1):  # target-only greedy decode from the root
            seq.append(int(np.argmax(synth.path_keyed_logits(seed + t, seq, V))))
        assert r["out_tokens"][t, :lens[t] + 1].tolist() == seq[1:]


def test_small_temperature_reproduces_greedy():
    seed, V = 22, 64
    tr = synth.greedy_tree_trials(seed, 200, vocab=V)
    srt = np.sort(tr["tgt_logits"], axis=-1)
    gap_ok = ((srt[..., -1] - srt[..., -2]) > 0.05).all(axis=1)
    g = oracle.reject_sample(tr["tgt_logits"], None, 0.0, 1.0, tr["tokens"], tr["parent"], tr["n_nodes"], None,
                             None)
    g.update(oracle.accept_path(g["accepted_child"], g["term_token"], tr["tokens"], tr["n_nodes"]))
    rng = synth.rng_for(seed, 5)
    dft = rng.normal(0, 1, tr["tgt_logits"].shape).astype(np.float32)
    B, n = tr["parent"].shape
    s = oracle.reject_sample(tr["tgt_logits"], dft, 1e-3, 1.0, tr["tokens"], tr["parent"], tr["n_nodes"],
                             synth.uniforms(rng, (B, n)), synth.uniforms(rng, (B, n)))
    s.update(oracle.accept_path(s["accepted_child"], s["term_token"], tr["tokens"], tr["n_nodes"]))
    assert gap_ok.sum() > 50
    for t in np.nonzero(gap_ok)[0]:
        assert s["accept_len"][t] == g["accept_len"][t]
        assert (s["out_tokens"][t] == g["out_tokens"][t]).all()


# ---------------------------------------------------------------- bookkeeping

def test_bad_requests_are_flagged():
    rng = synth.rng_for(30, 1)
    p = rng.dirichlet(np.ones(16))
    tr = synth.star_trials(rng, p, p, 2, 4)
    tr["parent"][1, 0] = 0           # root with a parent
    tr["tokens"][2, 1] = 16          # token outside the vocabulary
    tr["tgt_logits"][3, 0, 5] = np.nan
    r = _run(tr)
    assert r["accept_len"].tolist()[1:] == [-1, -1, -1]
    assert r["accept_len"][0] >= 0
    assert (r["accepted_child"][1:, 0] == oracle.BAD_REQUEST).all()
    assert (r["path_nodes"][1:] == -1).all() and (r["out_tokens"][1:] == -1).all()


def test_near_ties_are_flagged():
    # the first test lands within 1e-5 of its ratio
    p = np.full(16, 1 / 16)
    q = np.full(16, 1 / 16)
    p[0], p[1] = 0.5 / 16, 1.5 / 16
    tr = synth.star_trials(synth.rng_for(31, 1), p, q, 1, 1)
    tr["tokens"][0, 1] = 0
    tr["u_accept"][0, 1] = np.float32(0.5 + 2 ** -20)
    r = _run(tr)
    assert r["tie_flags"][0, 0] & oracle.TIE_TEST
