"""Pins for the oracle's per-token log-probability difference."""
import math

import numpy as np

from oracle import policy


def _rand(seed, T=7, V=50, scale=3.0):
    rng = np.random.default_rng(seed)
    return rng.normal(0, scale, (T, V)), rng.normal(0, scale, (T, V)), rng.integers(0, V, T)


def test_identical_policies_give_zero():
    a, _, lab = _rand(0)
    assert np.array_equal(policy.logprob_diff(a, a, lab), np.zeros(len(lab)))


def test_row_shift_invariance():
    a, r, lab = _rand(1)
    d = policy.logprob_diff(a, r, lab)
    shift = np.arange(a.shape[0])[:, None] * 37.5 - 100.0
    assert np.allclose(policy.logprob_diff(a + shift, r - 2 * shift, lab), d, atol=1e-12, rtol=0)


def test_two_token_vocabulary_closed_form():
    # V = 2: log p(0) = -log(1 + exp(v1 - v0)) = log sigmoid(v0 - v1)
    a = np.array([[0.3, -1.2], [2.0, 5.0]])
    r = np.array([[1.0, 1.0], [-3.0, 0.5]])
    lab = np.array([0, 1])
    ls = lambda z: -math.log1p(math.exp(-z))  # noqa: E731  log sigmoid
    want = [ls(0.3 + 1.2) - ls(0.0), ls(5.0 - 2.0) - ls(0.5 + 3.0)]
    assert np.allclose(policy.logprob_diff(a, r, lab), want, atol=1e-14, rtol=0)


def test_matches_explicit_probabilities():
    # brute force: normalise exp() by its sum directly (moderate logits)
    a, r, lab = _rand(2, scale=1.0)
    pa = np.exp(a) / np.exp(a).sum(axis=1, keepdims=True)
    pr = np.exp(r) / np.exp(r).sum(axis=1, keepdims=True)
    t = np.arange(len(lab))
    assert np.allclose(policy.logprob_diff(a, r, lab), np.log(pa[t, lab]) - np.log(pr[t, lab]), atol=1e-12)


def test_large_logits_stay_finite_and_planted_mistake_fails():
    a, r, lab = _rand(3, scale=1.0)
    a = a + 800.0  # exp overflows without the row maximum
    d = policy.logprob_diff(a, r, lab)
    assert np.all(np.isfinite(d))
    # a mistake planted in the oracle (normalising by the sum, not its log)
    wrong = (a[np.arange(len(lab)), lab] - np.exp(a - a.max(1, keepdims=True)).sum(1) - a.max(1)) - \
        policy.log_softmax_at(r, lab)
    assert np.abs(wrong - d).max() > 1e-3
