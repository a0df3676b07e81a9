"""CPU reference of the speculative-decoding acceptance rule.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference the HIP
library's sampler is checked against.  Only the test suite and the smoke check
may import it; the library and its binding never do, and it shares no code
with them.

What it computes, step by step, per sequence:

* "Warmup Guide -- Inference Optimization at Depth", Ch.6 (The Acceptance
  Rule): drafted token x, with draft probability q(x) and target probability
  p(x), is accepted with probability min(1, p(x)/q(x)); on the first rejection
  a replacement is sampled from norm(max(0, p - q)) and speculation stops.
* "FlashAttention, speculative decoding, quantisation and parallelism",
  Mechanics / Speculative decoding (the three-step listing): the uniform r of
  each position is compared with min(1, p/q); if every draft is accepted, one
  more token is sampled from the target's distribution at position k.

Readings where the pages are silent (each is listed with the design notes):

* the uniforms are inputs (u_accept per draft position, u_sample per
  sequence), so a run is reproducible;
* the ratio p/q and the comparison are evaluated in fp32 (the inputs'
  precision); a token the draft gave q(x) = 0 is accepted iff p(x) > 0, and a
  token outside the vocabulary is rejected;
* "sample(dist)" is the inverse CDF on a fixed-point grid: weights clamped to
  [0, 1] (NaN as 0), W = floor(w * 2^40), T = floor(u * sum W) in float64
  (clamped to [0, sum W - 1]; a NaN or negative u counts as 0), and the token
  is the first index whose running sum of W exceeds T;
* a residual with no mass (possible only through rounding, or p = q with a
  forced rejection) falls back to p at that position; a distribution with no
  mass at all yields token -1.

Pinned by tests/test_spec_oracle.py: the distributional identity of Ch.6 by
histogram (and a planted wrong residual that the same statistic rejects), the
pages' expected accepted length 2.94 at alpha = 0.7, k = 5, and hand-worked
cases.
"""
from __future__ import annotations

import math

import numpy as np

FIX = 2.0 ** 40


def fixed_weights(w) -> np.ndarray:
    """Fixed-point weights W = floor(clamp(w, 0, 1) * 2^40), int64; NaN counts as 0."""
    w = np.asarray(w, dtype=np.float32)
    w = np.fmin(np.fmax(w, np.float32(0.0)), np.float32(1.0))  # fmax/fmin drop NaN
    return np.floor(w.astype(np.float64) * FIX).astype(np.int64)


def sample_inverse_cdf(w, u: float) -> int:
    """The first index whose running sum of the fixed-point weights exceeds
    T = floor(u * total); -1 when the weights have no mass."""
    W = fixed_weights(w)
    total = int(W.sum())  # below 2^62 for at most 2^22 entries
    if total == 0:
        return -1
    uu = float(np.float32(u))
    if not uu >= 0.0:
        uu = 0.0
    T = math.floor(float(np.float64(uu) * np.float64(total)))
    T = min(max(T, 0), total - 1)
    running = np.cumsum(W)
    return int(np.searchsorted(running, T, side="right"))


def accept_one(x: int, q_row, p_row, u: float) -> bool:
    """The acceptance test of one drafted token x (fp32 arithmetic)."""
    V = len(p_row)
    if x < 0 or x >= V:
        return False
    qx = np.float32(q_row[x])
    px = np.float32(p_row[x])
    uu = np.float32(u)
    if qx > 0:
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            ratio = np.float32(px / qx)
        return bool(uu < np.fmin(np.float32(1.0), ratio))
    return bool(px > 0)


def spec_accept(draft_tokens, draft_probs, target_probs, u_accept, u_sample):
    """(n_accepted [B], out_tokens [B, k+1]) for B sequences.

    draft_tokens [B, k] ints; draft_probs [B, k, V] and target_probs
    [B, k+1, V] (fp32 values); u_accept [B, k]; u_sample [B].  out_tokens
    holds the accepted drafts, the sampled token, then -1.
    """
    target_probs = np.asarray(target_probs, dtype=np.float32)
    B, k1, V = target_probs.shape
    k = k1 - 1
    draft_tokens = np.asarray(draft_tokens).reshape(B, k)
    draft_probs = np.asarray(draft_probs, dtype=np.float32).reshape(B, k, V)
    u_accept = np.asarray(u_accept, dtype=np.float32).reshape(B, k)
    u_sample = np.asarray(u_sample, dtype=np.float32).reshape(B)
    n_acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, k + 1), -1, dtype=np.int32)
    for b in range(B):
        j = k
        for i in range(k):
            if not accept_one(int(draft_tokens[b, i]), draft_probs[b, i], target_probs[b, i], u_accept[b, i]):
                j = i
                break
        if j < k:
            residual = target_probs[b, j] - draft_probs[b, j]  # fp32
            tok = sample_inverse_cdf(residual, u_sample[b])
            if tok < 0:
                tok = sample_inverse_cdf(target_probs[b, j], u_sample[b])
        else:
            tok = sample_inverse_cdf(target_probs[b, k], u_sample[b])
        n_acc[b] = j
        out[b, :j] = draft_tokens[b, :j]
        out[b, j] = tok
    return n_acc, out
