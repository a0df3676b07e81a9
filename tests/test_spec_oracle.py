"""Pins of the CPU reference of the speculative acceptance rule (oracle/ref_spec.py).

Each test checks the reference against something other than itself: the
distributional identity the pages prove ("Warmup Guide", Ch.6: the output is
distributed exactly as the target), the pages' printed expected accepted
length (2.94 at alpha = 0.7, k = 5), and cases worked out by hand.  A wrong
residual planted in a copy of the reference is caught by the same histogram
statistic.
"""
import math
import os

import numpy as np
import pytest
import scipy.stats

from oracle import ref_spec as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_dist(rng, n, V):
    x = rng.gamma(0.7, size=(n, V)).astype(np.float32)
    return (x / x.sum(axis=1, keepdims=True)).astype(np.float32)


def run_one_position(rng, p, q, N, accept_fn=None):
    """N independent verify steps with k = 1 at one position whose target is
    p and draft q (the draft token is drawn from q); returns the first output
    token of each step."""
    V = len(p)
    xs = np.array([S.sample_inverse_cdf(q, u) for u in rng.random(N, dtype=np.float32)])
    u_acc = rng.random((N, 1), dtype=np.float32)
    u_smp = rng.random(N, dtype=np.float32)
    P = np.broadcast_to(p, (N, 2, V)).astype(np.float32)
    Q = np.broadcast_to(q, (N, 1, V)).astype(np.float32)
    fn = accept_fn or S.spec_accept
    _, out = fn(xs.reshape(N, 1), Q, P, u_acc, u_smp)
    return out[:, 0]


def chi2_pvalue(tokens, p):
    V = len(p)
    counts = np.bincount(tokens, minlength=V)
    expected = p * len(tokens)
    keep = expected > 0
    stat = float(np.sum((counts[keep] - expected[keep]) ** 2 / expected[keep]))
    assert counts[~keep].sum() == 0, "a zero-probability token was emitted"
    return float(scipy.stats.chi2.sf(stat, keep.sum() - 1))


def test_output_is_distributed_as_the_target():
    """Ch.6: P(out = x) = min(q, p) + P(reject) * residual(x) = p(x) for any q."""
    rng = np.random.default_rng(31)
    p, q = rand_dist(rng, 2, 6)
    toks = run_one_position(rng, p, q, 40000)
    assert chi2_pvalue(toks, p.astype(np.float64)) > 1e-4


def test_histogram_statistic_rejects_a_wrong_residual(monkeypatch):
    """Plant the plausible mistake 'resample from p instead of the residual'
    in the reference: the same statistic must reject it."""
    rng = np.random.default_rng(32)
    p, q = rand_dist(rng, 2, 6)

    def wrong(draft_tokens, draft_probs, target_probs, u_accept, u_sample):
        real = S.sample_inverse_cdf
        # a residual call is the one whose weights p - q have negative entries
        monkeypatch.setattr(S, "sample_inverse_cdf",
                            lambda w, u: real(p, u) if np.any(np.asarray(w) < 0) else real(w, u))
        try:
            return S.spec_accept(draft_tokens, draft_probs, target_probs, u_accept, u_sample)
        finally:
            monkeypatch.setattr(S, "sample_inverse_cdf", real)

    toks = run_one_position(rng, p, q, 40000, accept_fn=wrong)
    assert chi2_pvalue(toks, p.astype(np.float64)) < 1e-6


def test_expected_tokens_per_pass_matches_the_pages():
    """FA-SD page: with acceptance a = 0.7 per token and k = 5, a target pass
    yields (1 - a^6) / (1 - a) = 2.94 tokens on average.  Every position has
    q = [1, 0], p = [0.7, 0.3], so each draft (always token 0) is accepted
    with probability 0.7."""
    figs = {}
    with open(os.path.join(GOLDEN, "pages_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, *kv = line.split()
                figs[name] = {a: float(b) for a, b in (x.split("=") for x in kv)}
    fig = figs["spec_expected_tokens"]
    a, k = fig["alpha"], int(fig["k"])
    assert round((1 - a ** (k + 1)) / (1 - a), 2) == fig["tokens"]
    rng = np.random.default_rng(33)
    N = 60000
    p = np.tile(np.array([a, 1 - a], dtype=np.float32), (N, k + 1, 1))
    q = np.tile(np.array([1.0, 0.0], dtype=np.float32), (N, k, 1))
    n_acc, out = S.spec_accept(np.zeros((N, k), dtype=np.int32), q, p, rng.random((N, k), dtype=np.float32),
                               rng.random(N, dtype=np.float32))
    tokens_per_pass = n_acc + 1
    se = tokens_per_pass.std() / math.sqrt(N)
    assert abs(tokens_per_pass.mean() - fig["tokens"]) < 4 * se + 0.005
    # after a rejection the residual max(0, p - q) = [0, 0.3] forces token 1
    rej = n_acc < k
    assert np.all(out[rej, n_acc[rej]] == 1)


def test_hand_cases():
    # draft token 2 with q(2) = 1, p(2) = 0.25: accepted iff u < 0.25
    p = np.array([[[0.25, 0.5, 0.25, 0.0], [0.1, 0.2, 0.3, 0.4]]], dtype=np.float32)
    q = np.array([[[0.0, 0.0, 1.0, 0.0]]], dtype=np.float32)
    x = np.array([[2]])
    n, out = S.spec_accept(x, q, p, [[0.2]], [0.5])
    # accepted; bonus from p[1]: running sums 0.1, 0.3, 0.6, 1.0 -> T = 0.5 * total -> index 2
    assert n[0] == 1 and out[0].tolist() == [2, 2]
    n, out = S.spec_accept(x, q, p, [[0.3]], [0.5])
    # rejected; residual max(0, p - q) = [0.25, 0.5, 0, 0]: T = 0.375 of the
    # full mass, running sums 0.25, 0.75 -> index 1
    assert n[0] == 0 and out[0].tolist() == [1, -1]
    # boundary convention: the token is the first index whose running sum
    # EXCEEDS T
    assert S.sample_inverse_cdf([0.5, 0.25, 0.25], 0.75) == 2
    assert S.sample_inverse_cdf([0.5, 0.25, 0.25], 0.7499) == 1
    assert S.sample_inverse_cdf([0.5, 0.25, 0.25], 0.0) == 0
    assert S.sample_inverse_cdf([0.0, 0.0, 0.3], 0.0) == 2
    assert S.sample_inverse_cdf([0.0, 0.0], 0.5) == -1
    assert S.sample_inverse_cdf([0.2, float("nan"), 0.2], 0.6) == 2  # NaN weighs 0


def test_fallback_and_degenerate_inputs():
    p = np.array([[[0.5, 0.5], [0.9, 0.1]]], dtype=np.float32)
    q = np.array([[[0.5, 0.5]]], dtype=np.float32)
    # u = 1 forces a rejection with p = q: the residual has no mass -> sample p
    n, out = S.spec_accept([[0]], q, p, [[1.0]], [0.6])
    assert n[0] == 0 and out[0].tolist() == [1, -1]
    # a draft token outside the vocabulary is rejected
    n, out = S.spec_accept([[7]], q, p, [[0.0]], [0.1])
    assert n[0] == 0 and out[0].tolist() == [0, -1]
    # q(x) = 0: kept iff p(x) > 0
    q0 = np.array([[[0.0, 1.0]]], dtype=np.float32)
    n, _ = S.spec_accept([[0]], q0, p, [[0.99]], [0.1])
    assert n[0] == 1
    # k = 0: only the bonus token, from p[0]
    n, out = S.spec_accept(np.zeros((1, 0), dtype=np.int32), np.zeros((1, 0, 2), dtype=np.float32), p[:, :1],
                           np.zeros((1, 0), dtype=np.float32), [0.75])
    assert n[0] == 0 and out[0].tolist() == [1]
