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

def test_leaf_draft_rows_take_no_part():
    """[ZS] part C: the draft distribution produced at a node serves only to test that
    node's children, and a leaf's bonus is drawn from its target row (part G), so a
    leaf's draft row takes no part: NaN, +inf or arbitrary values there change no
    output (every node evaluated), while NaN in the root's draft row, which tests the
    root's children, makes the request bad."""
    rng = synth.rng_for(30, 2)
    p, q = rng.dirichlet(np.ones(16)), rng.dirichlet(np.ones(16))
    tr = synth.star_trials(rng, p, q, 3, 64, leaf_p=rng.dirichlet(np.ones(16)))
    ref = _run(tr, mode="all")
    alt = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in tr.items()}
    alt["dft_logits"][:, 1, 3] = np.nan
    alt["dft_logits"][:, 2, :] = np.inf
    alt["dft_logits"][:, 3] = rng.standard_normal((64, 16)).astype(np.float32)
    got = _run(alt, mode="all")
    for k in ("accepted_child", "term_token", "accept_len", "path_nodes", "out_tokens"):
        assert np.array_equal(got[k], ref[k]), k
    assert (ref["term_token"][:, 1:] >= 0).all()  # the leaves were evaluated: each drew its bonus
    alt["dft_logits"][5, 0, 7] = np.nan
    got = _run(alt, mode="all")
    assert got["accept_len"][5] == -1 and got["accepted_child"][5, 0] == oracle.BAD_REQUEST
    assert np.array_equal(np.delete(got["out_tokens"], 5, 0), np.delete(ref["out_tokens"], 5, 0))


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


# ---------------------------------------------------------------- near-tie bands
#
# The oracle flags a decision when its uniform falls inside the decision boundary's
# range over relative perturbations of every probability by at most eps (1e-6).
# Each case below derives that range's half-width by hand, to first order in eps,
# places the uniform at 0.8 and at 1.25 times it (the literal 1e-5 band of accept
# tests lying inside the first), and asserts the flag set and unset.

EPS = 1e-6


def _star3(p, q, child_tokens, u_acc, u_draw, leaf_p=None):
    tr = synth.star_trials(synth.rng_for(32, len(child_tokens)), np.asarray(p), np.asarray(q), len(child_tokens), 1,
                           leaf_p=None if leaf_p is None else np.asarray(leaf_p))
    tr["tokens"][0, 1:] = child_tokens
    tr["u_accept"][0, 1:] = np.float32(u_acc)
    tr["u_sample"][0, 0] = np.float32(u_draw)
    return tr


def _probs64(p):
    """p as the oracle sees it: the fp64 softmax of the fp32 logits that encode it."""
    e = np.exp(synth.log_probs_f32(np.asarray(p)).astype(np.float64))
    return e / e.sum()


P3 = (0.1, 0.5, 0.4)
Q3 = (0.4, 0.45, 0.15)


@pytest.mark.parametrize("side", [-1, 1])
def test_later_sibling_test_band(side):
    """Second child, after the first was rejected.  With c_1 = 1 the ratio is
    (p1 - q1) / (W q1), W = sum over p > q of (p - q) = 0.3.  Over the box:
    p1 - c q1 moves by eps (p1 + 2 q1) / (p1 - q1) = 28 eps relative (c itself is
    1 +- eps), W by eps * sum over p > q of (p + 2 q) / W = 7 eps, and q1 by eps:
    half-width 36 eps times the ratio, 1.33e-5 here."""
    p, q = _probs64(P3), _probs64(Q3)
    W = (p - q)[p > q].sum()
    ratio = (p[1] - q[1]) / (W * q[1])
    half = 36 * EPS * ratio
    assert 1e-5 < 0.8 * half  # the enclosure, not the literal band, decides the inside probe
    for frac, flagged in ((0.8, True), (1.25, False)):
        u = ratio + side * frac * half
        tr = _star3(P3, Q3, [0, 1], 0.9, 0.5)
        tr["u_accept"][0, 2] = np.float32(u)
        r = _run(tr)
        assert r["accepted_child"][0, 0] == (2 if side < 0 else oracle.NONE)
        assert bool(r["tie_flags"][0, 0] & oracle.TIE_TEST) == flagged, (frac, side)


@pytest.mark.parametrize("side", [-1, 1])
def test_leaf_draw_band(side):
    """A root without children draws from p.  The edge between tokens 0 and 1 sits at
    F = p0; over the box F / (F + (1 - F)) moves by 2 F (1 - F) eps."""
    p = _probs64((0.2, 0.3, 0.5))
    F = p[0]
    half = 2 * F * (1 - F) * EPS
    for frac, flagged in ((0.8, True), (1.25, False)):
        tr = _star3((0.2, 0.3, 0.5), (0.2, 0.3, 0.5), [], 0.5, F + side * frac * half)
        r = _run(tr)
        assert r["term_token"][0, 0] == (0 if side < 0 else 1)
        assert bool(r["tie_flags"][0, 0] & oracle.TIE_DRAW) == flagged, (frac, side)
        assert not r["tie_flags"][0, 0] & oracle.TIE_TEST


@pytest.mark.parametrize("side", [-1, 1])
def test_residual_draw_band(side):
    """One child (token 0, ratio 0.25) rejected; the bonus comes from the residual
    max(0, p - q) / W = (0, 0.05, 0.25) / 0.3, with its edge at F = 1/6.  Over the box
    the masses 0.05 and 0.25 move by 1.4 eps and 0.7 eps (p + 2 q each, c = 1 +- eps),
    so F moves by (28 - 7/3) eps relative."""
    p, q = _probs64(P3), _probs64(Q3)
    w = np.maximum(0.0, p - q)
    F = w[1] / w.sum()
    half = F * (28 - 7 / 3) * EPS
    for frac, flagged in ((0.8, True), (1.25, False)):
        tr = _star3(P3, Q3, [0], 0.9, F + side * frac * half)
        r = _run(tr)
        assert r["accepted_child"][0, 0] == oracle.NONE
        assert r["term_token"][0, 0] == (1 if side < 0 else 2)
        assert bool(r["tie_flags"][0, 0] & oracle.TIE_DRAW) == flagged, (frac, side)
        assert not r["tie_flags"][0, 0] & oracle.TIE_TEST


def test_zero_uniforms():
    """u = 0 (the uniform grid k * 2^-24 includes it): a test accepts exactly when its
    ratio is positive, and a draw returns the smallest token with positive mass, a
    decision the oracle flags (u sits on the first bin's lower edge)."""
    p, q = (0.0, 0.3, 0.7), (0.5, 0.25, 0.25)
    tr = _star3(p, q, [0, 2], 0.0, 0.0, leaf_p=(0.0, 0.5, 0.5))
    tr["u_sample"][:] = 0.0
    r = _run(tr)
    assert r["accepted_child"][0, 0] == 2       # token 0 has ratio 0: rejected; token 2 accepted
    assert r["term_token"][0, 2] == 1           # leaf draw at u = 0: first token with mass
    assert r["out_tokens"][0, :2].tolist() == [2, 1]
    assert r["tie_flags"][0, 2] & oracle.TIE_DRAW
    tr = _star3(p, q, [0], 0.0, 0.0)
    r = _run(tr)
    assert r["accepted_child"][0, 0] == oracle.NONE and r["term_token"][0, 0] == 1


# ---------------------------------------------------------------- acceptance rates

def test_acceptance_rate_special_cases():
    for a in (0.0, 0.3, 0.7, 1.0):
        p, q = synth.alpha_pq(a)
        got = oracle.acceptance_rate(synth.log_probs_f32(p), synth.log_probs_f32(q), 1.0, 1.0)
        assert abs(got - a) < 1e-6, (a, got)
    rng = synth.rng_for(33)
    l = rng.normal(0, 2, (3, 50)).astype(np.float32)
    assert np.allclose(oracle.acceptance_rate(l, l, 0.8, 0.8), 1.0, atol=1e-12)
    # the same rows at different temperatures: 1 - total variation distance
    p = oracle.softmax(l, 0.5)["probs"]
    q = oracle.softmax(l, 1.5)["probs"]
    assert np.allclose(oracle.acceptance_rate(l, l, 0.5, 1.5), 1 - 0.5 * np.abs(p - q).sum(-1), atol=1e-12)


def test_chain_lengths_follow_the_product_of_level_rates():
    """Workload 3's generator (16-node chain, T = 0.7 against a draft at T_d = 1, draft =
    target + N(0, 0.5)), with the vocabulary cut to 4096: the logit rows of each level
    are fixed, while every trial redraws the drafted tokens from the draft rows and
    the uniforms.  The rows do not depend on the drafted tokens, so levels pass
    independently and P(L >= k) = prod_{i <= k} alpha_i, alpha_i the acceptance rate
    of level i's rows."""
    inp = synth.make_config(3, seed=4, with_kv=False, vocab_override=4096)
    T, Td = inp["T"], inp["Td"]
    tgt, dft = inp["tgt_logits"][0], inp["dft_logits"][0]
    n = tgt.shape[0]
    alpha = oracle.acceptance_rate(tgt[:-1], dft[:-1], T, Td)
    pred = np.concatenate([[1.0], np.cumprod(alpha)])  # P(L >= k), k = 0 .. n - 1
    L = []
    for batch in range(16):
        tr = synth.chain_redraw(tgt, dft, Td, int(inp["tokens"][0, 0]), 625, synth.rng_for(34, batch))
        r = _run(dict(tr, tgt_logits=np.broadcast_to(tgt, (625,) + tgt.shape),
                      dft_logits=np.broadcast_to(dft, (625,) + dft.shape)), T=T, Td=Td)
        L.append(r["accept_len"])
    L = np.concatenate(L)
    assert (L >= 0).all()
    for k in range(1, n):
        emp = (L >= k).mean()
        sd = np.sqrt(pred[k] * (1 - pred[k]) / L.size)
        assert abs(emp - pred[k]) < 5 * sd + 1e-12, (k, emp, pred[k])
    probs = np.append(pred[:-1] - pred[1:], pred[-1])  # P(L = k)
    assert _chi2_p(np.bincount(L, minlength=n), probs) > 0.01
