"""CPU fp64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference that the
HIP library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library and its binding never
do, and it shares no code, tables or helpers with them.

What it computes is the plain, materialised definition of attention, written
out step by step so that it can be checked against the pages by eye:

* "Warmup Guide -- Inference Optimization at Depth", Ch.1 (Why Attention Is
  Memory-Bound): S = Q K^T, P = softmax(S), O = P V, with S materialised.
* same page, Ch.4 (FlashAttention -- Tiling the Whole Thing): the scores are
  divided by sqrt(d) (here: multiplied by the caller's ``scale``) and a causal
  mask hides the keys after the query.
* same page, Ch.2 (Numerically Safe Softmax, the max-subtracted equation):
  three sweeps over each row -- the max, the sum of exponentials, the
  normalised probabilities.
* "FlashAttention, speculative decoding, quantisation and parallelism",
  Mechanics / FlashAttention: the tiled algorithm is exact up to
  floating-point associativity, which is why the reference may be the
  un-tiled definition.

Readings where the pages are silent (each one is also listed with the design
notes of the library):

* causal alignment when Sq != Sk is bottom-right: query i sits at absolute
  position Sk - Sq + i and sees keys j <= i + Sk - Sq;
* LSE is m + ln(l) of the *scaled* logits, natural log;
* a row with no visible key has O = 0 and LSE = -inf;
* grouped-query attention maps query head h to KV head h // (H // Hkv).

All arithmetic is float64.  Every function pinned by the CPU test suite
(tests/test_oracle.py) against closed forms, invariants, an independent
pure-Python brute force and torch/scipy library routines.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "visible_mask",
    "attention",
    "attention_backward",
    "verify_tree",
    "gather_paged",
    "verify_paged",
    "verify",
    "online_softmax_1d",
    "online_attention_row",
    "lse_merge",
]


def visible_mask(Sq: int, Sk: int, causal: bool, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [len(rows), Sk]: True where key j is visible to query i.

    "Warmup Guide", Ch.4: the causal mask hides keys above the diagonal.
    Bottom-right reading for Sq != Sk: key j is visible to query i iff
    j <= i + (Sk - Sq).
    """
    r = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(Sk)
    if not causal:
        return np.ones((len(r), Sk), dtype=bool)
    return j[None, :] <= (r[:, None] + (Sk - Sq))


def _one_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
              rows: Optional[np.ndarray], Sq: int, row_chunk: int) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for one (batch, head): q [R, d] (the selected rows), k/v [Sk, d]."""
    R, d = q.shape
    Sk = k.shape[0]
    rows_all = np.arange(Sq) if rows is None else rows
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    if Sk == 0:
        return out, lse
    for r0 in range(0, R, row_chunk):
        r1 = min(R, r0 + row_chunk)
        # Ch.1 step 1 (with Ch.4's scale): the full rows of S, materialised.
        s = scale * (q[r0:r1] @ k.T)
        # Ch.4: causal mask (bottom-right alignment).
        vis = visible_mask(Sq, Sk, causal, rows_all[r0:r1])
        s = np.where(vis, s, -np.inf)
        has = vis.any(axis=1)
        # Ch.2, pass 1: the row maximum.
        m = np.max(s, axis=1)
        m_safe = np.where(has, m, 0.0)
        # Ch.2, pass 2: the sum of max-subtracted exponentials.
        e = np.exp(s - m_safe[:, None])
        l = np.sum(e, axis=1)
        # Ch.2, pass 3: normalise.
        l_safe = np.where(has, l, 1.0)
        p = e / l_safe[:, None]
        # Ch.1 step 3: O = P V.
        out[r0:r1] = np.where(has[:, None], p @ v, 0.0)
        lse[r0:r1] = np.where(has, m_safe + np.log(l_safe), -np.inf)
    return out, lse


def _blas_one_thread():
    """Context limiting BLAS to one thread per worker (when threadpoolctl exists)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except ImportError:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def attention(q, k, v, causal: bool, scale: float, rows: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[Tuple[int, int]]] = None, workers: int = 1,
              row_chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """O and LSE of softmax(scale * Q K^T + mask) V, materialised, in float64.

    q: [B, H, Sq, d]; k, v: [B, Hkv, Sk, d] (any float dtype; widened to
    float64).  ``scale`` is used as given (callers pass the fp32 value the
    library receives).  ``rows`` restricts the output to those query indices;
    ``heads`` restricts it to those (b, h) pairs (outputs for other heads stay
    0 / -inf).  Returns O [B, H, R, d] and LSE [B, H, R] where R = len(rows)
    or Sq.

    Definition: "Warmup Guide", Ch.1 (S, P, O) and Ch.2 (safe softmax);
    causal mask and scale from Ch.4.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch between q, k and v")
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    group = H // Hkv
    rows_arr = None if rows is None else np.asarray(rows, dtype=np.int64)
    R = Sq if rows_arr is None else len(rows_arr)
    dv = v.shape[3]
    out = np.zeros((B, H, R, dv), dtype=np.float64)
    lse = np.full((B, H, R), -np.inf, dtype=np.float64)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    tasks = []
    for (b, h) in todo:
        g = h // group  # grouped-query attention: contiguous groups of query heads
        qs = q[b, h] if rows_arr is None else q[b, h][rows_arr]
        tasks.append((qs, k[b, g], v[b, g], causal, float(scale), rows_arr, Sq, row_chunk))
    if workers > 1 and len(tasks) > 1:
        # worker threads (NumPy releases the GIL inside its kernels), one BLAS
        # thread each; no process is forked
        with _blas_one_thread(), ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda t: _one_head(*t), tasks))
    else:
        results = [_one_head(*t) for t in tasks]
    for (b, h), (o_bh, l_bh) in zip(todo, results):
        out[b, h] = o_bh
        lse[b, h] = l_bh
    return out, lse


def verify(q, k_cache, v_cache, seqlens_k, scale: float,
           heads: Optional[Sequence[Tuple[int, int]]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Speculative-verify attention: kq new queries per sequence vs a ragged cache.

    q: [B, H, kq, d]; caches: [B, Hkv, Smax, d] of which the first
    seqlens_k[b] rows are valid (the kq new tokens' keys are the last kq of
    them).  Query i of sequence b sees keys [0, seqlens_k[b] - kq + i]: the
    target model scores all drafted positions in one pass with a causal mask
    ("FlashAttention, speculative decoding, quantisation and parallelism",
    Mechanics / Speculative decoding; "Making Decode Fast", §1).  Each
    sequence is plain causal attention with Sq = kq, Sk = seqlens_k[b]
    (bottom-right alignment).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, kq, d = q.shape
    sl = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    out = np.zeros((B, H, kq, np.asarray(v_cache).shape[3]), dtype=np.float64)
    lse = np.full((B, H, kq), -np.inf, dtype=np.float64)
    for b in range(B):
        hs = None if heads is None else [(0, h) for (bb, h) in heads if bb == b]
        if hs is not None and not hs:
            continue
        o_b, l_b = attention(q[b:b + 1], np.asarray(k_cache[b:b + 1, :, :sl[b]]),
                             np.asarray(v_cache[b:b + 1, :, :sl[b]]), True, scale, heads=hs)
        out[b] = o_b[0]
        lse[b] = l_b[0]
    return out, lse


def _bwd_kv_group(q, k, v, dout, vis, scale):
    """Gradients for the query heads q/dout [G, Sq, d] that read one KV head
    k/v [Sk, d]: dQ [G, Sq, d] and that KV head's dK, dV [Sk, d] (summed over
    the G query heads in order)."""
    G, Sq, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(G):
        s = scale * (q[h] @ k.T)
        s = np.where(vis, s, -np.inf)
        P = np.zeros_like(s)
        for i in range(Sq):
            if vis[i].any():
                m = np.max(s[i])
                e = np.exp(s[i] - m)
                P[i] = e / np.sum(e)
        dv += P.T @ dout[h]
        dP = dout[h] @ v.T
        dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
        dq[h] = scale * (dS @ k)
        dk += scale * (dS.T @ q[h])
    return dq, dk, dv


def attention_backward(q, k, v, dout, causal: bool, scale: float,
                       kv_heads: Optional[Sequence[Tuple[int, int]]] = None, workers: int = 1):
    """Gradients (dQ, dK, dV) of sum(dout * O) for O = attention(q, k, v).

    "Warmup Guide -- Inference Optimization at Depth", Ch.4 (backward pass):
    P is recomputed from Q and K with the per-row statistics of the forward
    pass instead of being stored.  Here every quantity is materialised in
    float64 from the definition of Ch.1 (S = scale Q K^T with the mask, P =
    softmax(S) per row, O = P V), and the gradients are that definition's
    derivatives:
        dV = P^T dO;  dP = dO V^T;  dS = P * (dP - rowsum(P * dP));
        dQ = scale dS K;  dK = scale dS^T Q.
    For grouped-query attention dK and dV of a KV head sum over the query
    heads that read it.  Rows that see no key contribute nothing.
    ``kv_heads`` restricts the work to those (b, KV head g) pairs and their
    query heads (other gradients stay 0); ``workers`` > 1 runs the pairs on
    that many threads, one BLAS thread each.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = H // Hkv
    vis = visible_mask(Sq, Sk, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if kv_heads is None else list(kv_heads)
    tasks = [(q[b, g * G:(g + 1) * G], k[b, g], v[b, g], dout[b, g * G:(g + 1) * G], vis, scale) for b, g in todo]
    if workers > 1 and len(tasks) > 1:
        with _blas_one_thread(), ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda t: _bwd_kv_group(*t), tasks))
    else:
        results = [_bwd_kv_group(*t) for t in tasks]
    for (b, g), (dq_g, dk_g, dv_g) in zip(todo, results):
        dq[b, g * G:(g + 1) * G] = dq_g
        dk[b, g] = dk_g
        dv[b, g] = dv_g
    return dq, dk, dv


def _masked_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray, scale: float):
    """O [R, dv] and LSE [R] for one head with an explicit visibility matrix
    vis [R, Sk]: S = scale * q k^T materialised, -inf where not visible, then
    the three sweeps of "Warmup Guide", Ch.2 (max, sum of exponentials,
    normalised probabilities), O = P v and LSE = m + ln l.  Rows that see
    nothing: O = 0, LSE = -inf."""
    R = q.shape[0]
    s = scale * (q @ k.T)
    s = np.where(vis, s, -np.inf)
    o = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    for i in range(R):
        if not vis[i].any():
            continue
        m = np.max(s[i])
        e = np.exp(s[i] - m)
        l_ = np.sum(e)
        o[i] = (e / l_) @ v
        lse[i] = m + math.log(l_)
    return o, lse


def verify_tree(q, k_cache, v_cache, seqlens_k, tree_mask, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Tree-attention verify: the kq new tokens of a sequence are the nodes of
    a draft tree scored in one verify pass ("Making Decode Fast", §3, trees
    beat chains: candidates proposed as a tree and verified with tree
    attention).  Node t's key is at position seqlens_k[b] - kq + t; node i
    sees every earlier cache key and new key t iff bit t of tree_mask[b][i]
    is set (its ancestors and itself for a tree; 2^(i+1) - 1 for the causal
    chain of ``verify``).  q: [B, H, kq, d]; caches [B, Hkv, Smax, d];
    tree_mask [B, kq] of non-negative ints.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, kq, d = q.shape
    Hkv = np.asarray(k_cache).shape[1]
    G = H // Hkv
    sl = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    masks = np.asarray(tree_mask).astype(np.int64) & 0xFFFFFFFF
    out = np.zeros((B, H, kq, np.asarray(v_cache).shape[3]), dtype=np.float64)
    lse = np.full((B, H, kq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = sl[b]
        nk0 = n - kq  # position of new token 0
        vis = np.zeros((kq, n), dtype=bool)
        for i in range(kq):
            for t in range(n):
                rel = t - nk0
                vis[i, t] = rel < 0 or bool((int(masks[b, i]) >> rel) & 1)
        k_b = np.asarray(k_cache[b, :, :n], dtype=np.float64)
        v_b = np.asarray(v_cache[b, :, :n], dtype=np.float64)
        for h in range(H):
            out[b, h], lse[b, h] = _masked_head(q[b, h], k_b[h // G], v_b[h // G], vis, scale)
    return out, lse


def gather_paged(pages, block_table, seqlens_k, page_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """The logical cache [B, Hkv, max_len, d] held by a paged store, and which
    of its keys exist: present [B, max_len] bool.

    "Warmup Guide", Ch.8 (PagedAttention): KV storage is divided into
    fixed-size blocks of ``page_size`` tokens and each sequence holds a block
    table mapping its logical blocks to physical ones.  Logical key t of
    sequence b is therefore row t % page_size of physical page
    block_table[b][t // page_size].  pages: [num_pages, Hkv, page_size, d].
    A table entry that is not a physical page index in [0, num_pages) maps its
    logical block to no storage: the keys of that block do not exist (present
    is False, their rows are left zero and must not be attended to).  Keys at
    or past seqlens_k[b] are not present either.
    """
    pages = np.asarray(pages, dtype=np.float64)
    table = np.asarray(block_table)
    sl = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    num_pages, Hkv, ps, d = pages.shape
    if ps != page_size:
        raise ValueError("pages must be [num_pages, Hkv, page_size, d]")
    B = len(sl)
    max_len = max(sl) if sl else 0
    out = np.zeros((B, Hkv, max_len, d), dtype=np.float64)
    present = np.zeros((B, max_len), dtype=bool)
    for b in range(B):
        for blk in range((sl[b] + page_size - 1) // page_size):
            phys = int(table[b, blk])
            t0 = blk * page_size
            n = min(page_size, sl[b] - t0)
            if 0 <= phys < num_pages:
                out[b, :, t0:t0 + n] = pages[phys, :, :n]
                present[b, t0:t0 + n] = True
    return out, present


def verify_paged(q, k_pages, v_pages, block_table, seqlens_k, page_size: int, scale: float,
                 heads: Optional[Sequence[Tuple[int, int]]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Speculative-verify attention over a paged KV cache.

    Paging changes where K/V live, not what attention computes: the logical
    cache of ``gather_paged`` is attended to as in ``verify`` (query i of
    sequence b sees keys [0, seqlens_k[b] - kq + i]), restricted to the keys
    that exist.  A key in a block whose table entry names no page is absent,
    exactly like a key past the sequence's length; a row left with no key
    gets O = 0 and LSE = -inf.  ``heads`` restricts the work to those (b, h)
    pairs (other outputs stay 0 / -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, kq, d = q.shape
    k, present = gather_paged(k_pages, block_table, seqlens_k, page_size)
    v, _ = gather_paged(v_pages, block_table, seqlens_k, page_size)
    G = H // k.shape[1]
    sl = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    out = np.zeros((B, H, kq, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, kq), -np.inf, dtype=np.float64)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for (b, h) in todo:
        n = sl[b]
        # the causal verify mask (bottom-right: Sq = kq, Sk = n) and presence
        vis = visible_mask(kq, n, True) & present[b, :n][None, :]
        out[b, h], lse[b, h] = _masked_head(q[b, h], k[b, h // G, :n], v[b, h // G, :n], vis, scale)
    return out, lse


def online_softmax_1d(x: Sequence[float], blocks: Iterable[int]) -> Tuple[float, float]:
    """Streaming (m, l) over the blocks of a 1-D score vector.

    "Warmup Guide", Ch.3 (Online Softmax): per block b with local max m~_b and
    local exp-sum l~_b, m_new = max(m, m~_b) and
    l_new = l * exp(m - m_new) + l~_b * exp(m~_b - m_new).
    ``blocks`` are the block lengths (they must sum to len(x)).
    """
    x = np.asarray(x, dtype=np.float64)
    m, l, pos = -math.inf, 0.0, 0
    for n in blocks:
        blk = x[pos:pos + n]
        pos += n
        mb = float(np.max(blk))
        lb = float(np.sum(np.exp(blk - mb)))
        m_new = max(m, mb)
        l = l * math.exp(m - m_new) + lb * math.exp(mb - m_new)
        m = m_new
    if pos != len(x):
        raise ValueError("blocks must cover x")
    return m, l


def online_attention_row(s: Sequence[float], V: np.ndarray, blocks: Iterable[int]) -> Tuple[np.ndarray, float]:
    """One output row by streaming blocks of scores with the rescaled accumulator.

    "Warmup Guide", Ch.3 (last paragraph): keep O = sum_j p_j v_j
    un-normalised, multiply it by exp(m - m_new) whenever the max moves, and
    divide by l once at the end.  Returns (O, LSE = m + ln l).
    """
    s = np.asarray(s, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m, l = -math.inf, 0.0
    acc = np.zeros(V.shape[1], dtype=np.float64)
    pos = 0
    for n in blocks:
        blk, vb = s[pos:pos + n], V[pos:pos + n]
        pos += n
        m_new = max(m, float(np.max(blk)))
        corr = math.exp(m - m_new)
        p = np.exp(blk - m_new)
        acc = acc * corr + p @ vb
        l = l * corr + float(np.sum(p))
        m = m_new
    return acc / l, m + math.log(l)


def lse_merge(parts: List[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine normalised partial results over disjoint key sets.

    "Making Decode Fast", §5 (Flash-Decoding): keys are split across compute
    units, then a small final combine.  The combine is Ch.3's two-block (m, l)
    update of the "Warmup Guide" written with LSE_s = m_s + ln l_s:
    LSE = M + ln sum_s exp(LSE_s - M) with M = max_s LSE_s, and
    O = sum_s exp(LSE_s - LSE) * O_s.  ``parts`` are (O_s [..., d], LSE_s [...])
    pairs; parts with LSE_s = -inf (no visible key) contribute nothing.
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])  # [n, ...]
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])  # [n, ..., d]
    M = np.max(lses, axis=0)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w_un = np.exp(lses - M_safe[None])
    tot = np.sum(w_un, axis=0)
    lse = np.where(empty, -np.inf, M_safe + np.log(np.where(empty, 1.0, tot)))
    lse_safe = np.where(empty, 0.0, lse)
    w = np.where(empty[None], 0.0, np.exp(lses - lse_safe[None]))
    out = np.sum(w[..., None] * outs, axis=0)
    return out, lse


def default_workers() -> int:
    """Host cores available to this process (the oracle's worker-thread count)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)
