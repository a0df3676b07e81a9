"""Pins of the CPU fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against a closed form, an invariant of the
definition, an independent pure-Python brute force, or a library routine
(torch's CPU attention, scipy's logsumexp), so that a dropped scale, a wrong
sign, a transposed operand, a wrong causal offset or a wrong GQA head mapping
fails at least one of them.  Definitions: "Warmup Guide -- Inference
Optimization at Depth", Ch.1-Ch.4; the split-KV combine: "Making Decode Fast",
§5 (Flash-Decoding).
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import ref_attention as ref
from exact_attention_04_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- pin 1
@pytest.mark.parametrize("H,Hkv", [(1, 1), (4, 2), (6, 3)])
def test_one_key_gives_v0(H, Hkv):
    """Sk = 1: softmax over one key is 1, so O_i = V_0 and LSE_i = s_i0."""
    q, k, v = rnd(1, 2, H, 5, 8), rnd(2, 2, Hkv, 1, 8), rnd(3, 2, Hkv, 1, 8)
    o, lse = ref.attention(q, k, v, False, 0.3)
    for b in range(2):
        for h in range(H):
            g = h // (H // Hkv)
            np.testing.assert_allclose(o[b, h], np.repeat(v[b, g, :1], 5, 0), atol=1e-14)
            s = 0.3 * (q[b, h] @ k[b, g, 0])
            np.testing.assert_allclose(lse[b, h], s, atol=1e-14)


# ---------------------------------------------------------------- pin 2
def test_equal_logits_gives_mean_and_log_count():
    """Q = 0: every visible logit is 0, P is uniform on the visible keys,
    O_i = mean of visible V rows and LSE_i = ln |J_i|."""
    Sq = Sk = 7
    q = np.zeros((1, 2, Sq, 4))
    k, v = rnd(4, 1, 2, Sk, 4), rnd(5, 1, 2, Sk, 4)
    o, lse = ref.attention(q, k, v, False, 0.5)
    np.testing.assert_allclose(o[0, 1], np.repeat(v[0, 1].mean(0, keepdims=True), Sq, 0), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(Sk), atol=1e-13)
    o, lse = ref.attention(q, k, v, True, 0.5)
    for i in range(Sq):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :i + 1].mean(0), atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, i], math.log(i + 1), atol=1e-13)


def test_equal_keys_gives_mean_and_shifted_log_count():
    """All K rows equal: logits of row i all equal c_i = scale*q_i.k, so
    O_i = mean of visible V and LSE_i = c_i + ln |J_i| (bottom-right causal)."""
    Sq, Sk = 4, 9
    q = rnd(6, 1, 1, Sq, 5)
    k = np.repeat(rnd(7, 1, 1, 1, 5), Sk, axis=2)
    v = rnd(8, 1, 1, Sk, 5)
    o, lse = ref.attention(q, k, v, True, 0.7)
    for i in range(Sq):
        n = i + Sk - Sq + 1
        c = 0.7 * float(q[0, 0, i] @ k[0, 0, 0])
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(0), atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, i], c + math.log(n), atol=1e-13)


# ---------------------------------------------------------------- pin 3
@pytest.mark.parametrize("causal", [False, True])
def test_row_constant_shift_invariance(causal):
    """Safe softmax's shift invariance ("Warmup Guide", Ch.2) through the
    public interface: append Q' = [Q, c_i/scale], K' = [K, 1].  Every logit of
    row i moves by c_i, so O is unchanged and LSE moves by c_i."""
    scale = 0.25
    q, k, v = rnd(9, 1, 2, 6, 4), rnd(10, 1, 2, 6, 4), rnd(11, 1, 2, 6, 4)
    c = rnd(12, 1, 2, 6) * 5
    q2 = np.concatenate([q, (c / scale)[..., None]], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 2, 6, 1))], axis=-1)
    o1, l1 = ref.attention(q, k, v, causal, scale)
    o2, l2 = ref.attention(q2, k2, v, causal, scale)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + c, atol=1e-12)


# ---------------------------------------------------------------- pin 4
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    """With V = I (one value dimension per key) the output of ``attention``
    is P itself, so its rows are probability vectors: non-negative, summing
    to one, zero above the causal diagonal.  They also agree with the LSE
    output: P_ij = exp(s_ij - LSE_i)."""
    B, H, Hkv, S, d, scale = 2, 4, 2, 9, 6, 0.4
    q, k = rnd(13, B, H, S, d) * 3, rnd(14, B, Hkv, S, d)
    eye = np.broadcast_to(np.eye(S), (B, Hkv, S, S)).copy()
    P, lse = ref.attention(q, k, eye, causal, scale)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14 * S)
    assert (P >= 0).all()
    iu = np.triu_indices(S, 1)
    if causal:  # nothing above the diagonal
        assert np.all(P[..., iu[0], iu[1]] == 0)
    else:
        assert np.all(P[..., iu[0], iu[1]] > 0)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h // (H // Hkv)].T)
            vis = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
            np.testing.assert_allclose(np.where(vis, np.exp(s - lse[b, h][:, None]), 0.0), P[b, h],
                                       rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- pin 5
def test_causal_row0_is_v0():
    q, k, v = rnd(15, 2, 2, 8, 4), rnd(16, 2, 2, 8, 4), rnd(17, 2, 2, 8, 4)
    o, lse = ref.attention(q, k, v, True, 0.9)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-14)
    s00 = 0.9 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], s00, atol=1e-14)


# ---------------------------------------------------------------- pin 6
def brute_force(q, k, v, causal, scale):
    """Independent pure-Python three-pass safe softmax, scalar loops only."""
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    O = [[[[0.0] * v.shape[3] for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    L = [[[float("-inf")] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h * Hkv // H
            for i in range(Sq):
                vis = [j for j in range(Sk) if (not causal) or j <= i + Sk - Sq]
                if not vis:
                    continue
                s = {}
                for j in vis:
                    acc = 0.0
                    for c in range(d):
                        acc += float(q[b, h, i, c]) * float(k[b, g, j, c])
                    s[j] = scale * acc
                m = max(s.values())                       # pass 1
                tot = sum(math.exp(s[j] - m) for j in vis)  # pass 2
                for c in range(v.shape[3]):                 # pass 3 + P V
                    O[b][h][i][c] = sum(math.exp(s[j] - m) / tot * float(v[b, g, j, c]) for j in vis)
                L[b][h][i] = m + math.log(tot)
    return np.array(O), np.array(L)


@pytest.mark.parametrize("seed", range(6))
def test_against_pure_python_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.integers(1, 3))
    Sq, Sk, d = int(rng.integers(1, 17)), int(rng.integers(1, 17)), int(rng.integers(1, 9))
    causal = bool(rng.integers(0, 2))
    scale = float(rng.uniform(0.1, 2.0))
    q = rng.standard_normal((2, H, Sq, d)) * 3
    k = rng.standard_normal((2, Hkv, Sk, d))
    v = rng.standard_normal((2, Hkv, Sk, d))
    o, lse = ref.attention(q, k, v, causal, scale)
    ob, lb = brute_force(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ob, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-13)


def test_naive_fp32_softmax_overflows_where_max_subtraction_does_not():
    """Demonstration for the Q-times-16 stress inputs ("Warmup Guide", Ch.2):
    without the max subtraction exp overflows fp32 once a logit exceeds
    ln(FLT_MAX) ~ 88.72; with it the oracle stays finite."""
    x = np.array([100.0, 95.0, 1.0], dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(x) / np.sum(np.exp(x))
    assert not np.all(np.isfinite(naive))
    q = np.array([[[[100.0], [95.0], [1.0]]]])  # logits q*k with k = 1
    o, lse = ref.attention(q[:, :, :1], np.ones((1, 1, 3, 1)) * np.array([1.0, 0.95, 0.01])[None, None, :, None],
                           np.eye(3)[None, None], False, 1.0)
    assert np.all(np.isfinite(o)) and np.isfinite(lse).all()
    np.testing.assert_allclose(o[0, 0, 0].sum(), 1.0, atol=1e-14)


# ---------------------------------------------------------------- pin 7
def compositions(n):
    for cuts in itertools.product([0, 1], repeat=n - 1):
        sizes, cur = [], 1
        for c in cuts:
            if c:
                sizes.append(cur)
                cur = 1
            else:
                cur += 1
        sizes.append(cur)
        yield sizes


def test_online_softmax_every_block_partition():
    """"Warmup Guide", Ch.3 and its Lab 01 step: streaming (m, l) and the
    rescaled accumulator equal the three-pass values for every partition."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(8) * 4
    V = rng.standard_normal((8, 3))
    m3 = float(np.max(x))
    l3 = float(np.sum(np.exp(x - m3)))
    o3 = (np.exp(x - m3) / l3) @ V
    n = 0
    for blocks in compositions(8):
        m, l = ref.online_softmax_1d(x, blocks)
        assert m == m3
        assert abs(l - l3) <= 1e-13 * l3
        o, lse = ref.online_attention_row(x, V, blocks)
        np.testing.assert_allclose(o, o3, rtol=1e-13, atol=1e-14)
        assert abs(lse - (m3 + math.log(l3))) <= 1e-13
        n += 1
    assert n == 128


def test_online_softmax_increasing_maxima():
    """Every block raises the max: the rescale factor is hit at each step."""
    x = np.array([-5.0, -1.0, 0.5, 3.0, 7.0, 7.5])
    V = np.arange(18.0).reshape(6, 3)
    o, lse = ref.online_attention_row(x, V, [1] * 6)
    p = scipy.special.softmax(x)
    np.testing.assert_allclose(o, p @ V, rtol=1e-13)
    assert abs(lse - scipy.special.logsumexp(x)) < 1e-13


# ---------------------------------------------------------------- pin 8
@pytest.mark.parametrize("seed", range(4))
def test_split_kv_merge_equals_unsplit(seed):
    """"Making Decode Fast", §5: split the keys, then combine per-part
    (O_s, LSE_s) with the Ch.3 algebra; equals the unsplit result."""
    rng = np.random.default_rng(200 + seed)
    Sk = 37
    q = rng.standard_normal((1, 4, 3, 8)) * 2
    k = rng.standard_normal((1, 2, Sk, 8))
    v = rng.standard_normal((1, 2, Sk, 8))
    cuts = sorted(rng.choice(np.arange(1, Sk), size=3, replace=False).tolist())
    bounds = [0] + cuts + [Sk]
    parts = [ref.attention(q, k[:, :, a:b], v[:, :, a:b], False, 0.35) for a, b in zip(bounds, bounds[1:])]
    o, lse = ref.lse_merge(parts)
    o_ref, l_ref = ref.attention(q, k, v, False, 0.35)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, atol=1e-12)


def test_merge_ignores_empty_parts():
    q, k, v = rnd(20, 1, 1, 2, 4), rnd(21, 1, 1, 5, 4), rnd(22, 1, 1, 5, 4)
    full = ref.attention(q, k, v, False, 1.0)
    empty = (np.zeros_like(full[0]), np.full_like(full[1], -np.inf))
    o, lse = ref.lse_merge([empty, full, empty])
    np.testing.assert_allclose(o, full[0], atol=1e-14)
    np.testing.assert_allclose(lse, full[1], atol=1e-14)
    o, lse = ref.lse_merge([empty, empty])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- pin 9
def torch_reference(q, k, v, causal, scale):
    """torch's CPU attention in float64 with an explicit bottom-right mask,
    and scipy's logsumexp of the masked scores for LSE."""
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    kk = np.repeat(k, H // Hkv, axis=1)
    vv = np.repeat(v, H // Hkv, axis=1)
    mask = np.ones((Sq, Sk), dtype=bool)
    if causal:
        mask = np.tril(np.ones((Sq, Sk), dtype=bool), k=Sk - Sq)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(kk), torch.from_numpy(vv),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()
    s = scale * np.einsum("bhid,bhjd->bhij", q, kk)
    s = np.where(mask, s, -np.inf)
    lse = scipy.special.logsumexp(s, axis=-1)
    return o, lse


@pytest.mark.parametrize("Sq,Sk,causal,H,Hkv", [(300, 300, True, 2, 2), (300, 300, False, 4, 2),
                                                 (64, 500, True, 4, 1), (129, 257, False, 2, 1)])
def test_against_torch_sdpa_and_scipy_logsumexp(Sq, Sk, causal, H, Hkv):
    rng = np.random.default_rng(Sq + Sk)
    q = rng.standard_normal((1, H, Sq, 32)) * 2
    k = rng.standard_normal((1, Hkv, Sk, 32))
    v = rng.standard_normal((1, Hkv, Sk, 32))
    o, lse = ref.attention(q, k, v, causal, 0.177)
    o_t, l_t = torch_reference(q, k, v, causal, 0.177)
    np.testing.assert_allclose(o, o_t, atol=1e-10)
    np.testing.assert_allclose(lse, l_t, atol=1e-10)


# ---------------------------------------------------------------- pin 10
def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = rnd(30, 2, 8, 6, 4), rnd(31, 2, 2, 9, 4), rnd(32, 2, 2, 9, 4)
    o1, l1 = ref.attention(q, k, v, True, 0.5)
    o2, l2 = ref.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), True, 0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------- pin 11
def test_verify_equals_forward_and_prefix_noncausal():
    """Verify of kq new queries equals causal attention with Sq = kq and
    Sk = seqlens[b] (bottom-right); row i equals non-causal attention over
    keys [0, seqlens[b] - kq + i]."""
    rng = np.random.default_rng(40)
    B, H, Hkv, kq, d, smax = 3, 4, 2, 5, 8, 23
    q = rng.standard_normal((B, H, kq, d))
    kc = rng.standard_normal((B, Hkv, smax, d))
    vc = rng.standard_normal((B, Hkv, smax, d))
    sl = np.array([23, 9, 3])  # the last one has fewer keys than queries
    o, lse = ref.verify(q, kc, vc, sl, 0.3)
    for b in range(B):
        ob, lb = ref.attention(q[b:b + 1], kc[b:b + 1, :, :sl[b]], vc[b:b + 1, :, :sl[b]], True, 0.3)
        np.testing.assert_allclose(o[b], ob[0], atol=1e-13)
        np.testing.assert_array_equal(np.isneginf(lse[b]), np.isneginf(lb[0]))
        for i in range(kq):
            n = sl[b] - kq + i + 1
            if n <= 0:
                assert np.all(o[b, :, i] == 0) and np.all(np.isneginf(lse[b, :, i]))
                continue
            oi, li = ref.attention(q[b:b + 1, :, i:i + 1], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], False, 0.3)
            np.testing.assert_allclose(o[b, :, i], oi[0, :, 0], atol=1e-13)
            np.testing.assert_allclose(lse[b, :, i], li[0, :, 0], atol=1e-13)


# ---------------------------------------------------------------- pin 12
def test_linear_in_v_and_key_permutation_invariant():
    q, k = rnd(50, 1, 2, 7, 5), rnd(51, 1, 2, 11, 5)
    v1, v2 = rnd(52, 1, 2, 11, 5), rnd(53, 1, 2, 11, 5)
    o1, l1 = ref.attention(q, k, v1, False, 0.6)
    o2, _ = ref.attention(q, k, v2, False, 0.6)
    o12, l12 = ref.attention(q, k, v1 - 2.5 * v2, False, 0.6)
    np.testing.assert_allclose(o12, o1 - 2.5 * o2, atol=1e-12)
    np.testing.assert_array_equal(l12, l1)
    perm = np.random.default_rng(54).permutation(11)
    op, lp = ref.attention(q, k[:, :, perm], v1[:, :, perm], False, 0.6)
    np.testing.assert_allclose(op, o1, atol=1e-12)
    np.testing.assert_allclose(lp, l1, atol=1e-12)


# ---------------------------------------------------------------- pin 13
def test_hardmax_limit():
    """With distinct logits and a huge scale the softmax tends to a one-hot on
    the largest logit: O_i -> V_argmax."""
    q, k, v = rnd(60, 1, 1, 6, 3), rnd(61, 1, 1, 8, 3), rnd(62, 1, 1, 8, 3)
    o, lse = ref.attention(q, k, v, False, 1e3)
    s = q[0, 0] @ k[0, 0].T
    srt = np.sort(s, axis=1)
    assert np.all(srt[:, -1] - srt[:, -2] > 0.05)  # distinct enough: gap*scale > 50
    np.testing.assert_allclose(o[0, 0], v[0, 0][np.argmax(s, axis=1)], atol=1e-10)
    np.testing.assert_allclose(lse[0, 0], 1e3 * srt[:, -1], rtol=1e-12)


# ---------------------------------------------------------------- hand-derived worked example
def test_hand_derived_rational_example():
    """Keys k_j = (ln w_j, 0), query (1, 0), scale 1: the logits are ln w_j, so
    P = w / sum(w) exactly (w = 1, 2, 3, 4).  Values are small integers, so O
    is a rational computed here with Fractions; LSE = ln(sum of visible w).
    The same inputs with scale 0.5 and logits 2 ln w_j give the same P (the
    scale is applied), and the causal form gives prefix sums per row."""
    w = [1, 2, 3, 4]
    V = [(1, 0), (0, 1), (1, 1), (2, -1)]
    for scale, mult in [(1.0, 1.0), (0.5, 2.0)]:
        q = np.zeros((1, 1, 4, 2))
        q[..., 0] = 1.0
        k = np.zeros((1, 1, 4, 2))
        k[0, 0, :, 0] = [mult * math.log(x) for x in w]
        v = np.array(V, dtype=np.float64)[None, None]
        for causal in (False, True):
            o, lse = ref.attention(q, k, v, causal, scale)
            for i in range(4):
                n = i + 1 if causal else 4
                tot = sum(w[:n])
                exp = [sum(Fraction(w[j], tot) * V[j][c] for j in range(n)) for c in range(2)]
                np.testing.assert_allclose(o[0, 0, i], [float(x) for x in exp], atol=1e-14)
                assert abs(lse[0, 0, i] - math.log(tot)) < 1e-14
    # bottom-right alignment with Sq = 2 < Sk = 4: query 0 sees keys 0..2
    q = np.zeros((1, 1, 2, 2))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 4, 2))
    k[0, 0, :, 0] = [math.log(x) for x in w]
    o, lse = ref.attention(q, k, np.array(V, dtype=np.float64)[None, None], True, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], [4 / 6, 5 / 6], atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [1.2, 0.1], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [math.log(6), math.log(10)], atol=1e-14)


def test_empty_rows_convention():
    """Sq > Sk with a causal mask: the first Sq - Sk queries see no key."""
    q, k, v = rnd(70, 1, 1, 6, 4), rnd(71, 1, 1, 2, 4), rnd(72, 1, 1, 2, 4)
    o, lse = ref.attention(q, k, v, True, 1.0)
    assert np.all(o[0, 0, :4] == 0) and np.all(np.isneginf(lse[0, 0, :4]))
    assert np.all(np.isfinite(lse[0, 0, 4:]))
    o, lse = ref.attention(q, k[:, :, :0], v[:, :, :0], False, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_rows_subset_matches_full():
    q, k, v = rnd(80, 1, 2, 40, 8), rnd(81, 1, 1, 40, 8), rnd(82, 1, 1, 40, 8)
    o, lse = ref.attention(q, k, v, True, 0.3, row_chunk=7)
    rows = [0, 5, 17, 39]
    o2, l2 = ref.attention(q, k, v, True, 0.3, rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(l2, lse[:, :, rows])


def test_worker_pool_matches_serial():
    q, k, v = rnd(90, 1, 4, 33, 8), rnd(91, 1, 2, 33, 8), rnd(92, 1, 2, 33, 8)
    a = ref.attention(q, k, v, True, 0.3, workers=1)
    b = ref.attention(q, k, v, True, 0.3, workers=2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------- page figures
def test_workload_shapes_reproduce_the_pages_score_matrix_sizes():
    """The 8192-token prefill workload is the page's 17.2 GB score-matrix
    shape; the 32K workload's per-head score matrix is the page's ~2 GB."""
    figs = []
    with open(os.path.join(GOLDEN, "pages_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                _, *kv = line.split()
                figs.append({a: float(b) for a, b in (x.split("=") for x in kv)})
    w3 = synth.CAUSAL_BF16_S8192
    f0 = figs[0]
    assert (w3.B, w3.H, w3.Sq) == (f0["B"], f0["H"], f0["S"])
    assert round(w3.B * w3.H * w3.Sq * w3.Sk * 2 / 1e9, 1) == f0["GB"]
    w5 = synth.CAUSAL_BF16_S32768_D128
    assert w5.Sq == figs[1]["S"]
    assert round(w5.Sq * w5.Sk * 2 / 2**30) == figs[1]["GB"]


def test_synth_is_seeded_and_rounded():
    a = synth.random_qkv(3, 1, 2, 1, 5, 6, 8, synth.BF16)
    b = synth.random_qkv(3, 1, 2, 1, 5, 6, 8, synth.BF16)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
        assert x.dtype == torch.bfloat16
    q, k, v, sl = synth.verify_inputs(synth.VERIFY_BF16)
    L = synth.verify_lengths(synth.VERIFY_BF16)
    assert np.all(sl.numpy() == L + 5)
    assert k.shape == (8, 8, int(sl.max()), 128)
    assert L.min() >= 1024 and L.max() <= 16384


# ---------------------------------------------------------------- paged cache
def test_gather_paged_hand_example():
    """"Warmup Guide", Ch.8: logical key t of sequence b is row t % page of
    page table[b][t // page].  Pages of 2 tokens whose entries name their own
    (page, row); sequence 0 uses pages 2 then 0, sequence 1 shares page 1 for
    both of its blocks (prefix sharing), sequence 2 has entries that name no
    page (-1 and 7 >= num_pages), so its keys do not exist."""
    page, npg = 2, 3
    pages = np.zeros((npg, 1, page, 2))
    for p in range(npg):
        for r in range(page):
            pages[p, 0, r] = [p, r]
    table = np.array([[2, 0], [1, 1], [-1, 7]])
    sl = [3, 4, 4]
    got, present = ref.gather_paged(pages, table, sl, page)
    expect0 = [[2, 0], [2, 1], [0, 0]]            # page 2 rows 0,1, then page 0 row 0
    expect1 = [[1, 0], [1, 1], [1, 0], [1, 1]]    # page 1 twice
    np.testing.assert_array_equal(got[0, 0, :3], expect0)
    np.testing.assert_array_equal(got[1, 0], expect1)
    np.testing.assert_array_equal(present, [[1, 1, 1, 0], [1, 1, 1, 1], [0, 0, 0, 0]])


def test_verify_paged_absent_keys_hand_example():
    """Keys of a block whose table entry names no page are absent: the result
    is attention over the keys that exist, computed here by hand.  One query
    head, kq = 2, d = 1, scale 1, pages of 2 keys.  Sequence 0 has 6 keys in
    blocks [page 0, invalid, page 1]: keys 0,1 and 4,5 exist, 2,3 do not.
    New token 0 (key 4) sees keys 0..4 -> {0, 1, 4}; new token 1 sees {0, 1, 4, 5}.
    Sequence 1 has 2 keys, both new tokens, in an invalid block: its rows see
    nothing, so O = 0 and LSE = -inf."""
    page = 2
    kp = np.zeros((2, 1, page, 1))
    vp = np.zeros((2, 1, page, 1))
    # logits q*k with q = 1: ln 1, ln 2 on page 0; ln 3, ln 4 on page 1
    kp[0, 0, :, 0] = [np.log(1.0), np.log(2.0)]
    kp[1, 0, :, 0] = [np.log(3.0), np.log(4.0)]
    vp[0, 0, :, 0] = [10.0, 20.0]
    vp[1, 0, :, 0] = [30.0, 40.0]
    table = np.array([[0, -1, 1], [5, -1, -1]])
    q = np.ones((2, 1, 2, 1))
    o, lse = ref.verify_paged(q, kp, vp, table, [6, 2], page, 1.0)
    # row 0: weights 1, 2, 3 on values 10, 20, 30; row 1: weights 1..4 on 10..40
    np.testing.assert_allclose(o[0, 0, :, 0], [(10 + 40 + 90) / 6, (10 + 40 + 90 + 160) / 10], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [np.log(6.0), np.log(10.0)], rtol=1e-14)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("page", [1, 4, 32])
def test_verify_paged_equals_contiguous_under_any_page_permutation(page):
    """Paging changes where K/V live, not the result: scatter a contiguous
    cache into randomly permuted pages (with spare pages full of NaN that no
    table entry names) and the paged oracle must give the contiguous result
    up to summation order."""
    rng = np.random.default_rng(11)
    B, H, Hkv, kq, d = 3, 4, 2, 3, 8
    sl = np.array([37, 5, 64])
    smax = int(sl.max())
    q = rng.standard_normal((B, H, kq, d))
    k = rng.standard_normal((B, Hkv, smax, d))
    v = rng.standard_normal((B, Hkv, smax, d))
    nblk = (sl + page - 1) // page
    total = int(nblk.sum())
    perm = rng.permutation(total + 5)  # 5 spare pages
    kp = np.full((total + 5, Hkv, page, d), np.nan)
    vp = np.full((total + 5, Hkv, page, d), np.nan)
    table = np.full((B, int(nblk.max())), -1)
    i = 0
    for b in range(B):
        for blk in range(nblk[b]):
            phys = perm[i]
            i += 1
            table[b, blk] = phys
            n = min(page, sl[b] - blk * page)
            kp[phys] = 0.0
            vp[phys] = 0.0
            kp[phys, :, :n] = k[b, :, blk * page:blk * page + n]
            vp[phys, :, :n] = v[b, :, blk * page:blk * page + n]
    o_c, l_c = ref.verify(q, k, v, sl, 0.4)
    o_p, l_p = ref.verify_paged(q, kp, vp, table, sl, page, 0.4)
    assert np.all(ref.gather_paged(kp, table, sl, page)[1] == (np.arange(smax)[None, :] < sl[:, None]))
    # the paged path applies the mask through an explicit visibility matrix,
    # the contiguous one through ``attention``: equal up to summation order
    np.testing.assert_allclose(o_p, o_c, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_p, l_c, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- tree verify
def chain_masks(B, kq):
    return np.array([[(1 << (i + 1)) - 1 for i in range(kq)]] * B)


def ancestor_masks(parents):
    """Bitmask of each node's ancestors and itself from a parent array (-1 = root)."""
    out = []
    for i in range(len(parents)):
        m, j = 0, i
        while j >= 0:
            m |= 1 << j
            j = parents[j]
        out.append(m)
    return out


def test_verify_tree_chain_mask_is_causal_verify():
    rng = np.random.default_rng(21)
    B, H, Hkv, kq, d = 3, 4, 2, 5, 8
    sl = np.array([12, 5, 30])
    q = rng.standard_normal((B, H, kq, d))
    k = rng.standard_normal((B, Hkv, 30, d))
    v = rng.standard_normal((B, Hkv, 30, d))
    o_c, l_c = ref.verify(q, k, v, sl, 0.35)
    o_t, l_t = ref.verify_tree(q, k, v, sl, chain_masks(B, kq), 0.35)
    np.testing.assert_allclose(o_t, o_c, atol=1e-13)
    np.testing.assert_allclose(l_t, l_c, atol=1e-13)


def test_verify_tree_each_root_to_leaf_path_is_a_chain():
    """A node of a draft tree sees exactly the cache and its root-to-node path,
    so re-running the path alone as a chain verify must give its row."""
    rng = np.random.default_rng(22)
    parents = [-1, 0, 0, 1, 1, 2, 5, 3]
    kq, H, Hkv, d, L = len(parents), 4, 2, 8, 9
    q = rng.standard_normal((1, H, kq, d))
    k = rng.standard_normal((1, Hkv, L + kq, d))
    v = rng.standard_normal((1, Hkv, L + kq, d))
    masks = np.array([ancestor_masks(parents)])
    o_t, l_t = ref.verify_tree(q, k, v, [L + kq], masks, 0.5)
    leaves = [i for i in range(kq) if i not in parents]
    assert leaves == [4, 6, 7]
    for leaf in leaves:
        path, j = [], leaf
        while j >= 0:
            path.append(j)
            j = parents[j]
        path = path[::-1]
        sel = [L + t for t in path]
        kk = np.concatenate([k[:, :, :L], k[:, :, sel]], axis=2)
        vv = np.concatenate([v[:, :, :L], v[:, :, sel]], axis=2)
        o_c, l_c = ref.verify(q[:, :, path], kk, vv, [L + len(path)], 0.5)
        np.testing.assert_allclose(o_t[:, :, path], o_c, atol=1e-13)
        np.testing.assert_allclose(l_t[:, :, path], l_c, atol=1e-13)


def test_verify_tree_hand_example():
    """d = 1, scale = 1, q = 1: logits are the keys, chosen as ln w, so the
    probabilities are w / sum(w) over the visible keys.  Cache key w=2 (v=10);
    tree root n0 (w=3, v=20) with children n1 (w=5, v=30) and n2 (w=7, v=50).
    n2 must not see its sibling n1."""
    w = [2, 3, 5, 7]
    vals = [10, 20, 30, 50]
    k = np.log(np.array(w, dtype=np.float64)).reshape(1, 1, 4, 1)
    v = np.array(vals, dtype=np.float64).reshape(1, 1, 4, 1)
    q = np.ones((1, 1, 3, 1))
    masks = np.array([ancestor_masks([-1, 0, 0])])  # [0b001, 0b011, 0b101]
    o, lse = ref.verify_tree(q, k, v, [4], masks, 1.0)
    expect = {0: [0, 1], 1: [0, 1, 2], 2: [0, 1, 3]}  # visible key indices
    for i, vis in expect.items():
        num = sum(Fraction(w[t]) * vals[t] for t in vis)
        den = sum(Fraction(w[t]) for t in vis)
        assert abs(o[0, 0, i, 0] - float(num / den)) < 1e-12
        assert abs(lse[0, 0, i] - math.log(float(den))) < 1e-12
    # the chain would have let n2 see n1
    o_c, _ = ref.verify(q, k, v, [4], 1.0)
    assert abs(o_c[0, 0, 2, 0] - float(Fraction(580, 17))) < 1e-12


def test_verify_tree_empty_rows():
    """No cache keys and a node whose mask is 0: O = 0, LSE = -inf."""
    q = np.ones((1, 1, 2, 3))
    k = np.ones((1, 1, 2, 3))
    v = np.ones((1, 1, 2, 3))
    o, lse = ref.verify_tree(q, k, v, [2], np.array([[0, 3]]), 1.0)
    assert np.all(o[0, 0, 0] == 0) and np.isneginf(lse[0, 0, 0])
    np.testing.assert_allclose(o[0, 0, 1], 1.0)
    assert abs(lse[0, 0, 1] - (3.0 + math.log(2.0))) < 1e-12


# ---------------------------------------------------------------- backward
def loss_and_grads(q, k, v, do, causal, scale):
    o, _ = ref.attention(q, k, v, causal, scale)
    return float(np.sum(o * do)), ref.attention_backward(q, k, v, do, causal, scale)


@pytest.mark.parametrize("causal,Sq,Sk,H,Hkv", [(False, 5, 7, 2, 1), (True, 6, 6, 2, 2), (True, 4, 9, 4, 2),
                                               (True, 7, 3, 1, 1)])
def test_backward_matches_central_differences(causal, Sq, Sk, H, Hkv):
    """The gradient of L = sum(dO * O) against central finite differences of
    the forward oracle, for every element of Q, K and V (fp64, step 1e-6)."""
    rng = np.random.default_rng(41)
    d = 3
    q, k, v = rng.standard_normal((1, H, Sq, d)), rng.standard_normal((1, Hkv, Sk, d)), rng.standard_normal((1, Hkv, Sk, d))
    do = rng.standard_normal((1, H, Sq, d))
    _, grads = loss_and_grads(q, k, v, do, causal, 0.7)
    eps = 1e-6
    for x, gx in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp, _ = loss_and_grads(q, k, v, do, causal, 0.7)
            x[idx] = keep - eps
            lm, _ = loss_and_grads(q, k, v, do, causal, 0.7)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(gx, num, atol=1e-7, rtol=1e-6)


@pytest.mark.parametrize("causal,Sq,Sk", [(False, 33, 20), (True, 40, 40), (True, 17, 50)])
def test_backward_matches_torch_autograd(causal, Sq, Sk):
    """torch CPU autograd in fp64 through scaled_dot_product_attention with an
    explicit bottom-right mask (grouped heads expanded by repeat)."""
    rng = np.random.default_rng(42)
    B, H, Hkv, d, scale = 2, 4, 2, 16, 0.3
    q, k, v = rng.standard_normal((B, H, Sq, d)), rng.standard_normal((B, Hkv, Sk, d)), rng.standard_normal((B, Hkv, Sk, d))
    do = rng.standard_normal((B, H, Sq, d))
    dq, dk, dv = ref.attention_backward(q, k, v, do, causal, scale)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    mask = torch.tensor(ref.visible_mask(Sq, Sk, causal))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(H // Hkv, dim=1), tv.repeat_interleave(H // Hkv, dim=1), attn_mask=mask, scale=scale)
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-10)


def test_backward_closed_forms():
    """One key: P = 1, so dV_0 = sum_i dO_i and dQ = dK = 0.  Rows of dS sum
    to zero, so the keys' dK vectors sum to zero."""
    rng = np.random.default_rng(43)
    q, k, v, do = rng.standard_normal((1, 2, 6, 4)), rng.standard_normal((1, 1, 1, 4)), \
        rng.standard_normal((1, 1, 1, 4)), rng.standard_normal((1, 2, 6, 4))
    dq, dk, dv = ref.attention_backward(q, k, v, do, False, 0.5)
    np.testing.assert_allclose(dv[0, 0, 0], do[0].sum(axis=(0, 1)), atol=1e-12)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    q, k, v, do = (rng.standard_normal((1, 2, 9, 4)) for _ in range(4))
    for causal in (False, True):
        _, dk, _ = ref.attention_backward(q, k, v, do, causal, 0.5)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
