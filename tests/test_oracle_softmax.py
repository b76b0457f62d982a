"""Pins of the oracle's per-node softmax against scipy's softmax (a library routine)
and the defining properties of a probability row."""
import numpy as np
import scipy.special

import oracle


def test_matches_library_softmax_and_sums_to_one():
    rng = np.random.default_rng(0)
    for T in (1.0, 0.7, 2.5, 0.05):
        logits = (rng.standard_normal((9, 1000)) * 3).astype(np.float32)
        r = oracle.softmax(logits, T)
        ref = scipy.special.softmax(logits.astype(np.float64) / T, axis=1)
        np.testing.assert_allclose(r["probs"], ref, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(r["max"], logits.max(axis=1).astype(np.float64))
        np.testing.assert_allclose(r["sumexp"], np.exp((logits.astype(np.float64) - logits.max(axis=1, keepdims=True)) / T).sum(1),
                                   rtol=1e-12)


def test_argmax_lowest_index_on_ties_and_greedy():
    logits = np.zeros((3, 50), np.float32)
    logits[0, [7, 9, 30]] = 5.0
    logits[1, 49] = 1.0
    logits[2, :] = -2.0
    r = oracle.softmax(logits, 0.0)
    assert r["argmax"].tolist() == [7, 49, 0]
    assert r["probs"] is None


def test_negative_infinity_is_probability_zero_and_nan_is_invalid():
    logits = np.zeros((3, 8), np.float32)
    logits[0, :4] = -np.inf
    logits[1, 3] = np.nan
    logits[2, :] = -np.inf
    r = oracle.softmax(logits, 1.0)
    assert r["valid"].tolist() == [1, 0, 0]
    np.testing.assert_allclose(r["probs"][0], [0, 0, 0, 0, .25, .25, .25, .25], atol=1e-15)
    logits[1, 3] = np.inf
    assert oracle.softmax(logits, 1.0)["valid"][1] == 0


def test_heavy_tails_do_not_underflow_the_definition():
    rng = np.random.default_rng(5)
    logits = (2 * rng.standard_t(3, (4, 152064))).astype(np.float32)
    r = oracle.softmax(logits, 1.0)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(r["probs"], ref, rtol=1e-11, atol=0)
