"""GPU parity of attn_bwd (gradients of exact attention) against the CPU
fp64 oracle.

The oracle materialises S, P, dP and dS in float64 from the definition of
"Warmup Guide -- Inference Optimization at Depth", Ch.1 and takes their
derivatives (Ch.4, backward pass); the GPU recomputes P tile by tile from Q,
K and the forward pass's LSE.  Both see the same bf16 inputs; the GPU's O and
LSE come from attn_fwd on those inputs.

Tolerance (bf16 inputs and outputs, fp32 accumulation), per gradient tensor
G against the oracle's R:
  * max |G - R| <= 1e-2 * max |R|   (elementwise, scaled to the tensor), and
  * ||G - R||_2 <= 5e-3 * ||R||_2   (no systematic drift hiding under the max),
with an absolute floor of 1e-5 per element for gradients that are zero only
by cancellation.
The error sources are the bf16 rounding of the stored gradient (relative
2^-9 per element), of P and dS where they enter the second products as bf16
MFMA operands (relative 2^-9 each, averaging over the summed rows or keys),
and of O in D = rowsum(dO * O).  Observed errors sit near 4e-3 (max) and
2e-3 (norm).
"""
import numpy as np
import pytest
import torch

from exact_attention_04_amd import synth
from oracle import ref_attention as ref
from tests import parity as P

pytestmark = pytest.mark.gpu

TOL_MAX = 1e-2
TOL_NORM = 5e-3
ATOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from exact_attention_04_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding


def run_bwd(q, k, v, do, causal, scale):
    from exact_attention_04_amd import binding
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = binding.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare_grad(g: np.ndarray, r: np.ndarray, name: str, what: str) -> dict:
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
    if r.size == 0:
        return {}
    # ATOL covers gradients that vanish only by cancellation (one key: dS = 0
    # up to the rounding of D) against inputs of unit size
    scale_max = max(float(np.abs(r).max()), ATOL / TOL_MAX)
    scale_norm = max(float(np.linalg.norm(r)), ATOL / TOL_NORM * np.sqrt(r.size))
    err = np.abs(g - r)
    res = {f"{name}_max": float(err.max()) / scale_max,
           f"{name}_norm": float(np.linalg.norm(err)) / scale_norm}
    assert res[f"{name}_max"] <= TOL_MAX, f"{what}: {name} {res}"
    assert res[f"{name}_norm"] <= TOL_NORM, f"{what}: {name} {res}"
    return res


def bwd_case(seed, B, H, Hkv, Sq, Sk, d, causal, what=""):
    P.log(f"[bwd] {what} seed={seed} B={B} H={H} Hkv={Hkv} Sq={Sq} Sk={Sk} d={d} causal={causal}")
    q, k, v = synth.random_qkv(seed, B, H, Hkv, Sq, Sk, d, "bf16", device="cuda")
    do = synth.normal(np.random.default_rng(seed + 1000), (B, H, Sq, d), "bf16").cuda()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    dq, dk, dv = run_bwd(q, k, v, do, causal, scale)
    rq, rk, rv = ref.attention_backward(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), synth.to_f64(do),
                                        causal, scale)
    res = {}
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        res.update(compare_grad(synth.to_f64(g), r, name, what))
    # rows that see no key get exactly zero dQ; keys no row sees get zero dK, dV
    vis = ref.visible_mask(Sq, Sk, causal)
    if Sq and Sk:
        dead_rows = ~vis.any(axis=1)
        dead_keys = ~vis.any(axis=0)
        assert np.all(synth.to_f64(dq)[:, :, dead_rows] == 0), f"{what}: dQ of rows without keys"
        assert np.all(synth.to_f64(dk)[:, :, dead_keys] == 0), f"{what}: dK of keys without rows"
        assert np.all(synth.to_f64(dv)[:, :, dead_keys] == 0), f"{what}: dV of keys without rows"
    P.log(f"    ok {res}")
    return res


CASES = [
    # (B, H, Hkv, Sq, Sk, d, causal)
    (1, 2, 2, 256, 256, 128, False),   # whole tiles, no masked tile
    (1, 2, 2, 256, 256, 128, True),
    (1, 2, 2, 200, 200, 128, True),    # ragged tail
    (2, 4, 1, 130, 300, 128, False),   # grouped-query heads, Sk > Sq
    (1, 4, 2, 300, 333, 128, True),    # causal with Sk > Sq (offset diagonal)
    (1, 4, 4, 100, 333, 64, True),
    (1, 2, 1, 333, 100, 64, True),     # Sq > Sk: the first rows see no key
    (2, 2, 2, 77, 45, 64, False),
    (1, 1, 1, 1, 1, 128, True),        # one row, one key
    (1, 1, 1, 1, 200, 64, False),
    (1, 1, 1, 200, 1, 128, False),
    (1, 3, 1, 513, 513, 128, True),    # several key blocks and query tiles
]


@pytest.mark.parametrize("B,H,Hkv,Sq,Sk,d,causal", CASES)
def test_bwd_matches_oracle(B, H, Hkv, Sq, Sk, d, causal):
    bwd_case(11 + Sq + Sk + d, B, H, Hkv, Sq, Sk, d, causal, what="small")


@pytest.mark.parametrize("H,Hkv,Sq,Sk,d,causal", [
    (2, 2, 2048, 2048, 128, True),   # 8 query blocks of 256 rows, 64 key tiles of 32, 8 key blocks of 256
    (2, 1, 2048, 2048, 64, True),    # d = 64: key tiles of 64, grouped-query heads
    (2, 2, 1000, 1500, 128, False),  # ragged query block and key tile, a long unmasked run
    (3, 1, 3000, 3000, 128, True),   # 36 blocks per kernel, not a multiple of the XCD count
])
def test_bwd_larger_sequence(H, Hkv, Sq, Sk, d, causal):
    """Sequences long enough that every pipeline buffer of both kernels is
    reused many times, against the oracle on every element."""
    bwd_case(5 + Sq + d, 1, H, Hkv, Sq, Sk, d, causal, what="long")


def test_bwd_empty_query_or_key_side():
    from exact_attention_04_amd import binding
    rng = np.random.default_rng(3)
    # no queries: dK = dV = 0
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = synth.normal(rng, (1, 2, 70, 128), "bf16").cuda()
    v = synth.normal(rng, (1, 2, 70, 128), "bf16").cuda()
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    dq, dk, dv = binding.bwd(q, k, v, o, lse, torch.empty_like(q), causal=False)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)
    # no keys: dQ = 0
    q = synth.normal(rng, (1, 2, 33, 64), "bf16").cuda()
    k = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = binding.fwd(q, k, k, causal=False)
    dq, dk, dv = binding.bwd(q, k, k, o, lse, synth.normal(rng, (1, 2, 33, 64), "bf16").cuda())
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0


def test_bwd_deterministic():
    """No atomics: two calls give bitwise equal gradients."""
    from exact_attention_04_amd import binding
    q, k, v = synth.random_qkv(9, 1, 4, 1, 300, 300, 128, "bf16", device="cuda")
    do = synth.normal(np.random.default_rng(10), (1, 4, 300, 128), "bf16").cuda()
    o, lse = binding.fwd(q, k, v, causal=True)
    a = binding.bwd(q, k, v, o, lse, do, causal=True)
    b = binding.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


_full = {}


def full_size_grads():
    """GPU gradients at the prefill workload's shape (B=4, H=32, S=8192,
    d=128, causal) in the launch configuration the benchmark times, with the
    inputs, all as float64 arrays (computed once)."""
    if not _full:
        from exact_attention_04_amd import binding
        B, H, S, d = 4, 32, 8192, 128
        P.log(f"[bwd] full size B={B} H={H} S={S} d={d} causal")
        q, k, v = synth.random_qkv(21, B, H, H, S, S, d, "bf16", device="cuda")
        do = synth.normal(np.random.default_rng(22), (B, H, S, d), "bf16").cuda()
        scale = float(np.float32(1.0 / np.sqrt(d)))
        o, lse = binding.fwd(q, k, v, causal=True, scale=scale)
        dq, dk, dv = binding.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
        torch.cuda.synchronize()
        _full.update(scale=scale, inputs=tuple(synth.to_f64(t) for t in (q, k, v, do)),
                     grads=tuple(synth.to_f64(t) for t in (dq, dk, dv)))
        del q, k, v, do, o, lse, dq, dk, dv
        torch.cuda.empty_cache()
    return _full


@pytest.mark.parametrize("part", range(4))
def test_bwd_full_size_every_head(part):
    """Every gradient of every head at the full size, a quarter of the
    (batch, head) pairs per case: the oracle recomputes each pair's
    gradients (independent of every other head) on 16 threads."""
    f = full_size_grads()
    qn, kn, vn, don = f["inputs"]
    dq, dk, dv = f["grads"]
    pairs = [(b, h) for b in range(4) for h in range(32)][part * 32:(part + 1) * 32]
    P.log(f"[bwd] full size, heads {pairs[0]}..{pairs[-1]}")
    rq, rk, rv = ref.attention_backward(qn, kn, vn, don, True, f["scale"], kv_heads=pairs, workers=P.workers())
    worst = {}
    for b, h in pairs:  # the tolerance applies to each head's gradient tensors
        for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            for key, val in compare_grad(g[b, h], r[b, h], name, f"full b={b} h={h}").items():
                worst[key] = max(worst.get(key, 0.0), val)
    P.log(f"    ok {len(pairs)} heads, worst {worst}")


@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 8)])
def test_bwd_dynamic_tail_equals_captured_fixed_order(H, Hkv):
    """With 32+ query blocks of 256 rows and 16+ key blocks of 256 keys the
    lightest quarter of each kernel's blocks is claimed at run time (S = 8192
    qualifies for both); a call captured into a graph runs the fixed order.
    Same arithmetic per block, so the gradients must agree bit for bit, on
    every replay, with eager calls between the replays."""
    from exact_attention_04_amd import binding
    rng = np.random.default_rng(70 + H)
    S, d = 8192, 128
    q = synth.normal(rng, (1, H, S, d), "bf16").cuda()
    k = synth.normal(rng, (1, Hkv, S, d), "bf16").cuda()
    v = synth.normal(rng, (1, Hkv, S, d), "bf16").cuda()
    do = synth.normal(rng, (1, H, S, d), "bf16").cuda()
    scale = float(np.float32(d ** -0.5))
    o, lse = binding.fwd(q, k, v, causal=True, scale=scale)
    ref = binding.bwd(q, k, v, o, lse, do, causal=True, scale=scale)  # eager: the dynamic tails
    torch.cuda.synchronize()
    binding.bwd(q, k, v, o, lse, do, causal=True, scale=scale)  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = binding.bwd(q, k, v, o, lse, do, causal=True, scale=scale)  # captured: the fixed order
    for rep in range(3):
        for t in got:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        P.log(f"[bwd] H={H} Hkv={Hkv} graph replay {rep}")
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), rep
        again = binding.bwd(q, k, v, o, lse, do, causal=True, scale=scale)  # eager work between replays
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(again, ref)), rep
