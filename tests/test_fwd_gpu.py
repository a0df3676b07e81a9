"""GPU parity of attn_fwd against the CPU fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from exact_attention_04_amd import synth
from oracle import ref_attention as ref
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from exact_attention_04_amd import binding  # raises if the library is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding


# ------------------------------------------------------------------ named workloads, every output
def test_noncausal_f32_s256_full():
    w = synth.NONCAUSAL_F32_S256
    q, k, v = synth.prefill_inputs(w, "cuda")
    P.log(f"[fwd] {w.name}")
    o, lse = P.run_fwd(q, k, v, w.causal, w.scale)
    P.check_fwd(q, k, v, o, lse, w.causal, w.scale, "f32", what=w.name)


@pytest.mark.parametrize("w", [synth.CAUSAL_BF16_S2048, synth.CAUSAL_BF16_S2048_Q8], ids=lambda w: w.name)
def test_causal_bf16_s2048_full(w):
    q, k, v = synth.prefill_inputs(w, "cuda")
    P.log(f"[fwd] {w.name}")
    o, lse = P.run_fwd(q, k, v, w.causal, w.scale)
    res = P.check_fwd(q, k, v, o, lse, w.causal, w.scale, "bf16", what=w.name)
    P.log(f"    max logit {float((synth.to_f64(q[0, 0]) @ synth.to_f64(k[0, 0]).T).max() * w.scale):.2f} {res}")


def test_q_times_16_stress():
    """Logits up to ~100 overflow fp32 exp without the max subtraction."""
    P.fwd_case(16, 1, 4, 4, 1024, 1024, 128, True, "bf16", q_mult=16.0, what="qx16")


# ------------------------------------------------------------------ full-size workloads, every output
# The 8192- and 32768-token workloads in the launch configuration the
# benchmark times.  The GPU result is computed once per workload; the oracle
# then recomputes every row of every head, a group of heads per test case so
# that each case stays well under a minute of host time (the oracle needs
# about 6 s for all 128 heads of the 8192 workload on 16 threads, and 25-50 s
# for each 32768 workload).
FULL = {w.name: w for w in (synth.CAUSAL_BF16_S8192, synth.CAUSAL_BF16_S32768_D128, synth.CAUSAL_BF16_S32768_D64)}
FULL_GROUPS = {synth.CAUSAL_BF16_S8192.name: 1, synth.CAUSAL_BF16_S32768_D128.name: 2,
               synth.CAUSAL_BF16_S32768_D64.name: 4}
_full_cache = {}


def full_result(name):
    """(q, k, v as float64 arrays, O and LSE of the GPU as float64) for one
    workload; only the latest workload is kept."""
    if name not in _full_cache:
        _full_cache.clear()
        w = FULL[name]
        q, k, v = synth.prefill_inputs(w, "cuda")
        P.log(f"[fwd] {w.name} (every row)")
        o, lse = P.run_fwd(q, k, v, w.causal, w.scale)
        # properties at every output: finite, |O| bounded by max |V| (convex combination)
        o32 = o.float()
        assert torch.isfinite(o32).all() and torch.isfinite(lse).all()
        assert float(o32.abs().max()) <= float(v.float().abs().max()) + 2e-2
        _full_cache[name] = tuple(synth.to_f64(t) for t in (q, k, v, o, lse))
        del q, k, v, o, lse, o32
        torch.cuda.empty_cache()
    return _full_cache[name]


@pytest.mark.parametrize("name,part", [(n, i) for n, c in FULL_GROUPS.items() for i in range(c)])
def test_full_size_every_row(name, part):
    w = FULL[name]
    qn, kn, vn, og, lg = full_result(name)
    per = -(-w.B * w.H // FULL_GROUPS[name])
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)][part * per:(part + 1) * per]
    P.log(f"[fwd] {w.name} heads {pairs[0]}..{pairs[-1]}: oracle on every row")
    o_ref, l_ref = ref.attention(qn, kn, vn, w.causal, w.scale, heads=pairs, workers=P.workers())
    bi = [b for b, _ in pairs]
    hi = [h for _, h in pairs]
    res = P.compare(og[bi, hi], lg[bi, hi], o_ref[bi, hi], l_ref[bi, hi], "bf16", w.name)
    P.log(f"    ok {len(pairs)} heads x {w.Sq} rows {res}")


@pytest.mark.parametrize("d", [64, 128])
def test_long_sequence_plain_order_every_row(d):
    """Long causal rows whose block count (3 heads x 31 blocks) is not a
    multiple of the XCD count: no head pairs, no dynamic tail, workgroups in
    launch order.  Every row of every head against the oracle."""
    P.fwd_case(7900 + d, 1, 3, 1, 7900, 7900, d, True, "bf16", what="plain order")


@pytest.mark.parametrize("Sq,Sk", [(8192, 8192), (8000, 8192)])
def test_head_pairs_order_every_row(Sq, Sk):
    """32+ query blocks per head: the workgroups run two heads at a time in
    groups of four ids (the order the 8192 and 32768 workloads use), here
    with d = 64, grouped-query heads, a ragged last block and Sq != Sk.
    Every row of every head against the oracle."""
    P.fwd_case(Sq + 64, 1, 32, 8, Sq, Sk, 64, True, "bf16", what="head-pairs order")


# ------------------------------------------------------------------ the dynamic tail
# With 32+ query blocks per head the lightest quarter of the blocks is claimed
# from a per-GPU counter at run time; a call captured into a graph uses the
# fixed order instead.  Which workgroup computes a block changes nothing in
# its arithmetic, so the two orders must agree bit for bit.
def _dyn_case(seed, H=32):
    q, k, v = synth.random_qkv(seed, 1, H, H, 8192, 8192, 128, "bf16", device="cuda")
    return q, k, v, float(np.float32(128 ** -0.5))


def test_dynamic_tail_equals_captured_fixed_order():
    from exact_attention_04_amd import binding
    q, k, v, scale = _dyn_case(31)
    o_d, l_d = binding.fwd(q, k, v, causal=True, scale=scale)  # eager: the dynamic tail
    torch.cuda.synchronize()
    o_g = torch.full_like(q, float("nan"))
    l_g = torch.full((1, 32, 8192), float("nan"), dtype=torch.float32, device="cuda")
    binding.fwd(q, k, v, causal=True, scale=scale, out=o_g, lse=l_g)  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.fwd(q, k, v, causal=True, scale=scale, out=o_g, lse=l_g)  # captured: the fixed order
    for rep in range(3):
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        P.log(f"[fwd] graph replay {rep}")
        assert torch.equal(o_g, o_d) and torch.equal(l_g, l_d), rep
        o_e, l_e = binding.fwd(q, k, v, causal=True, scale=scale)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_d) and torch.equal(l_e, l_d), rep
    P.check_fwd(q, k, v, o_d, l_d, True, scale, "bf16", rows=list(range(0, 8192, 97)) + [8191],
                what="dynamic tail")


def test_dynamic_tail_concurrent_streams():
    """Calls on two streams at once, more calls than the counter has slots:
    every result equals that of a call made alone."""
    from exact_attention_04_amd import binding
    cases = [_dyn_case(41, H=16), _dyn_case(42, H=16)]
    refs = []
    for q, k, v, scale in cases:
        o, l = binding.fwd(q, k, v, causal=True, scale=scale)
        torch.cuda.synchronize()
        refs.append((o, l))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[(torch.empty_like(c[0]), torch.empty((1, 16, 8192), dtype=torch.float32, device="cuda"))
             for _ in range(4)] for c in cases]
    n = 80
    torch.cuda.synchronize()
    for i in range(n):
        for j in (0, 1):
            q, k, v, scale = cases[j]
            o, l = outs[j][i % 4]
            with torch.cuda.stream(streams[j]):
                binding.fwd(q, k, v, causal=True, scale=scale, out=o, lse=l)
        if i % 4 == 3:
            torch.cuda.synchronize()
            for j in (0, 1):
                for o, l in outs[j]:
                    assert torch.equal(o, refs[j][0]) and torch.equal(l, refs[j][1]), (i, j)
                    o.fill_(float("nan"))
            torch.cuda.synchronize()  # the fills are done before the next calls write
    P.log(f"[fwd] {2 * n} calls on two streams, every result bitwise equal to a lone call")


# ------------------------------------------------------------------ ragged and edge shapes
EDGE_S = [1, 2, 17, 63, 64, 65, 127, 129, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_square_edges(dtype, d, causal):
    for S in EDGE_S:
        P.fwd_case(S, 1, 2, 1, S, S, d, causal, dtype, what=f"square S={S}")


@pytest.mark.parametrize("Sq,Sk", [(1, 300), (5, 1029), (17, 64), (200, 129), (300, 70), (129, 4097), (64, 1)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rectangular_bottom_right(Sq, Sk, causal, dtype):
    P.fwd_case(Sq + Sk, 2, 4, 2, Sq, Sk, 128, causal, dtype, what="rect")


@pytest.mark.parametrize("H,Hkv", [(8, 1), (8, 2), (8, 8)])
def test_gqa_ratios(H, Hkv):
    P.fwd_case(H * 10 + Hkv, 2, H, Hkv, 300, 300, 128, True, "bf16", what="gqa")


def test_sk_zero_gives_empty_rows():
    q, k, v = synth.random_qkv(1, 1, 2, 2, 40, 1, 128, "bf16", device="cuda")
    k0, v0 = k[:, :, :0].contiguous(), v[:, :, :0].contiguous()
    from exact_attention_04_amd import binding
    o, lse = binding.fwd(q, k0, v0, causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


# ------------------------------------------------------------------ hygiene
def test_repeat_is_bitwise_deterministic():
    w = synth.CAUSAL_BF16_S2048
    q, k, v = synth.prefill_inputs(w, "cuda")
    o1, l1 = P.run_fwd(q, k, v, True, w.scale)
    o2, l2 = P.run_fwd(q, k, v, True, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_guard_bands_untouched_and_tail_not_read():
    """O/LSE live inside larger buffers whose guard bands must stay as filled;
    K/V are followed by NaN, so an over-read past the last key would poison O."""
    from exact_attention_04_amd import binding
    B, H, Hkv, Sq, Sk, d = 1, 4, 2, 190, 190, 128
    q, k, v = synth.random_qkv(5, B, H, Hkv, Sq, Sk, d, "bf16", device="cuda")
    g = 4096
    kbuf = torch.full((k.numel() + g,), float("nan"), dtype=torch.bfloat16, device="cuda")
    vbuf = torch.full((v.numel() + g,), float("nan"), dtype=torch.bfloat16, device="cuda")
    kbuf[:k.numel()] = k.reshape(-1)
    vbuf[:v.numel()] = v.reshape(-1)
    kk, vv = kbuf[:k.numel()].view(k.shape), vbuf[:v.numel()].view(v.shape)
    obuf = torch.full((q.numel() + 2 * g,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * Sq + 2 * g,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[g:g + q.numel()].view(q.shape)
    lse = lbuf[g:g + B * H * Sq].view(B, H, Sq)
    for causal in (False, True):
        binding.fwd(q, kk, vv, causal=causal, scale=float(np.float32(d ** -0.5)), out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(obuf[:g] == 7.0) and torch.all(obuf[g + q.numel():] == 7.0)
        assert torch.all(lbuf[:g] == 7.0) and torch.all(lbuf[g + B * H * Sq:] == 7.0)
        P.check_fwd(q, k, v, o, lse, causal, float(np.float32(d ** -0.5)), "bf16", what="guard")


def test_lse_optional():
    from exact_attention_04_amd import binding
    q, k, v = synth.random_qkv(9, 1, 2, 2, 100, 100, 64, "bf16", device="cuda")
    o1, _ = binding.fwd(q, k, v, causal=True, want_lse=False)
    o2, _ = binding.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
