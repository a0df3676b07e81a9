"""GPU parity of attn_verify (split-KV + merge) against the CPU fp64 oracle."""
import numpy as np
import pytest
import torch

from exact_attention_04_amd import synth
from oracle import ref_attention as ref
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from exact_attention_04_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding


def poison_tail(k, v, seqlens):
    """Cache rows at or beyond seqlens[b] become NaN: any over-read shows up."""
    for b, s in enumerate(seqlens.tolist()):
        k[b, :, max(s, 0):] = float("nan")
        v[b, :, max(s, 0):] = float("nan")


def run_verify(q, k, v, sl, max_len, scale):
    from exact_attention_04_amd import binding
    o, lse = binding.verify(q, k, v, sl, max_len, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def check_verify(q, k, v, sl_host, o, lse, scale, what):
    qn, kn, vn = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    kn = np.nan_to_num(kn, nan=0.0)  # the oracle never reads past seqlens either
    vn = np.nan_to_num(vn, nan=0.0)
    o_ref, l_ref = ref.verify(qn, kn, vn, sl_host, scale)
    res = P.compare(synth.to_f64(o), synth.to_f64(lse), o_ref, l_ref, "bf16", what)
    P.log(f"    ok {res}")
    return res


def verify_case(seed, lengths, H, Hkv, kq, d, what=""):
    """lengths = total keys per sequence (including the kq new ones)."""
    B = len(lengths)
    rng = np.random.default_rng(seed)
    sl = np.asarray(lengths, dtype=np.int32)
    stride = max(1, int(sl.max()) + 3)
    q = synth.normal(rng, (B, H, kq, d), "bf16").cuda()
    k = synth.normal(rng, (B, Hkv, stride, d), "bf16").cuda()
    v = synth.normal(rng, (B, Hkv, stride, d), "bf16").cuda()
    poison_tail(k, v, torch.from_numpy(sl))
    slt = torch.from_numpy(sl).cuda()
    scale = float(np.float32(d ** -0.5))
    P.log(f"[verify] {what} seed={seed} lengths={lengths} H={H} Hkv={Hkv} kq={kq} d={d}")
    o, lse = run_verify(q, k, v, slt, int(sl.max()), scale)
    return check_verify(q, k, v, sl, o, lse, scale, what)


def test_verify_workload_full():
    w = synth.VERIFY_BF16
    q, k, v, sl = synth.verify_inputs(w, "cuda")
    poison_tail(k, v, sl)
    P.log(f"[verify] {w.name} lengths={sl.tolist()}")
    o, lse = run_verify(q, k, v, sl, int(sl.max()), w.scale)
    check_verify(q, k, v, sl.cpu().numpy(), o, lse, w.scale, w.name)


@pytest.mark.parametrize("kq", [1, 5, 6])
def test_chunk_boundaries(kq):
    C = 1024
    lengths = [C - 1, C, C + 1, 2 * C, 2 * C + kq, kq, 1, 3 * C - 2]
    verify_case(kq, lengths, 32, 8, kq, 128, what="chunk-boundaries")


def test_fewer_keys_than_queries_and_empty():
    verify_case(11, [0, 1, 2, 4, 5, 6], 8, 2, 5, 128, what="short")


@pytest.mark.parametrize("H,Hkv,kq", [(8, 8, 5), (16, 2, 4), (32, 4, 4), (4, 1, 8), (32, 1, 1)])
def test_gqa_packing(H, Hkv, kq):
    verify_case(H + Hkv + kq, [700, 3000, 5], H, Hkv, kq, 128, what="gqa")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv,kq", [(32, 4, 5), (32, 4, 8), (64, 8, 6), (16, 1, 4), (8, 8, 64), (4, 2, 32),
                                      (64, 1, 1), (24, 3, 7)])
def test_two_query_tiles(H, Hkv, kq, d):
    """(H/Hkv)*kq between 33 and 64: the rows that share a KV head fill two
    32-row tiles, both fed from the same K/V operands (a GQA-8 model
    verifying up to 8 drafts, a 64-token chain on one KV head, ...)."""
    verify_case(H * 3 + Hkv + kq + d, [2500, 40, kq, 1025, 700 + kq], H, Hkv, kq, d, what="two-tiles")


@pytest.mark.parametrize("kq", [5, 8])
def test_gqa8_on_workload_lengths(kq):
    """GQA-8 (64 query heads over the 8 KV heads) with the verify workload's
    cache lengths: 8*kq packed rows per KV head."""
    w = synth.VERIFY_BF16
    L = synth.verify_lengths(w)
    verify_case(800 + kq, [int(x) + kq for x in L], 64, 8, kq, 128, what=f"gqa8-kq{kq}")


def test_head_dim_64():
    verify_case(64, [2500, 17, 1024], 16, 4, 5, 64, what="d64")


def test_device_lengths_clamped_to_max():
    """Device lengths above max_seqlen_k are clamped to it (documented)."""
    rng = np.random.default_rng(3)
    B, H, Hkv, kq, d, stride = 2, 8, 2, 5, 128, 1500
    q = synth.normal(rng, (B, H, kq, d), "bf16").cuda()
    k = synth.normal(rng, (B, Hkv, stride, d), "bf16").cuda()
    v = synth.normal(rng, (B, Hkv, stride, d), "bf16").cuda()
    sl = torch.tensor([1400, 9999], dtype=torch.int32, device="cuda")
    o, lse = run_verify(q, k, v, sl, 1200, float(np.float32(d ** -0.5)))
    check_verify(q, k, v, np.array([1200, 1200]), o, lse, float(np.float32(d ** -0.5)), "clamp")


def test_verify_deterministic():
    w = synth.VERIFY_BF16
    q, k, v, sl = synth.verify_inputs(w, "cuda")
    o1, l1 = run_verify(q, k, v, sl, int(sl.max()), w.scale)
    o2, l2 = run_verify(q, k, v, sl, int(sl.max()), w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_verify_workspace_uninitialised_and_shared():
    """The workspace needs no initialisation and may be shared by calls of
    different shapes: starting from random bytes, and from all-ones bytes,
    two workloads alternate on one workspace, and every call must equal the
    first result of its workload bit for bit (a merge that used a stale piece
    count or a slot its split did not write would change it)."""
    from exact_attention_04_amd import binding
    w = synth.VERIFY_BF16
    qa, ka, va, sla = synth.verify_inputs(w, "cuda")
    rng = np.random.default_rng(21)
    lb = [700, 3000, 5, 1]
    qb = synth.normal(rng, (4, 32, 4, 128), "bf16").cuda()
    kb = synth.normal(rng, (4, 4, 3000, 128), "bf16").cuda()
    vb = synth.normal(rng, (4, 4, 3000, 128), "bf16").cuda()
    slb = torch.tensor(lb, dtype=torch.int32, device="cuda")
    need = max(binding.attn_verify_workspace_bytes(8, 32, 8, 5, 128),
               binding.attn_verify_workspace_bytes(4, 32, 4, 4, 128))
    calls = [(qa, ka, va, sla, int(sla.max()), w.scale), (qb, kb, vb, slb, 3000, float(np.float32(128 ** -0.5)))]
    refs = []
    for q, k, v, sl, ml, sc in calls:
        o, lse = binding.verify(q, k, v, sl, ml, scale=sc,
                                workspace=torch.zeros(need, dtype=torch.uint8, device="cuda"))
        refs.append((o.clone(), lse.clone()))
    P.log("[verify] shared workspace: refs of two workloads done")
    for fill in ("random", "ones"):
        if fill == "random":
            ws = torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)).cuda()
        else:
            ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
        for it in range(12):
            i = it % 2
            q, k, v, sl, ml, sc = calls[i]
            o, lse = binding.verify(q, k, v, sl, ml, scale=sc, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o, refs[i][0]) and torch.equal(lse, refs[i][1]), (fill, it)
    P.log("    ok 24 calls bitwise equal")
    o, lse = refs[1]
    check_verify(qb, kb, vb, np.array(lb), o, lse, float(np.float32(128 ** -0.5)), "shared-ws-b")


def test_many_sequences():
    """More than 64 sequences: the split kernel reads the lengths 64 at a
    time (slice plan, segment walk, empty-sequence rows), so 150 ragged
    sequences, some empty and some shorter than kq, cross those rounds."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 400, 150)]
    for i in (0, 63, 64, 65, 127, 128, 149):
        lengths[i] = int(rng.integers(0, 4))  # empty or fewer keys than queries
    verify_case(78, lengths, 8, 2, 3, 128, what="many-sequences")
