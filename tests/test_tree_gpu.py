"""GPU parity of attn_verify_tree (draft-tree verify) against the CPU fp64
oracle, and bitwise agreement with attn_verify for the chain mask.

Draft trees: "Making Decode Fast", §3 (trees beat chains: the candidates are
proposed as a tree and scored in one verify pass with tree attention).
"""
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


def ancestor_mask(parents):
    out = []
    for i in range(len(parents)):
        m, j = 0, i
        while j >= 0:
            m |= 1 << j
            j = parents[j]
        out.append(m)
    return out


def random_tree_masks(rng, B, kq):
    """Per sequence, a random tree in topological order (node i's parent is
    uniform in [0, i)) as ancestor-and-self bitmasks."""
    rows = []
    for _ in range(B):
        parents = [-1] + [int(rng.integers(0, i)) for i in range(1, kq)]
        rows.append(ancestor_mask(parents))
    return np.array(rows, dtype=np.int64)


def as_i32(masks):
    return torch.from_numpy((np.asarray(masks, dtype=np.int64) & 0xFFFFFFFF).astype(np.uint32).view(np.int32))


def tree_case(seed, lengths, H, Hkv, kq, d, masks=None, what=""):
    from exact_attention_04_amd import binding
    rng = np.random.default_rng(seed)
    B = len(lengths)
    sl = np.asarray(lengths, dtype=np.int32)
    stride = max(1, int(sl.max()) + 2)
    q = synth.normal(rng, (B, H, kq, d), "bf16").cuda()
    k = synth.normal(rng, (B, Hkv, stride, d), "bf16").cuda()
    v = synth.normal(rng, (B, Hkv, stride, d), "bf16").cuda()
    for b, n in enumerate(sl.tolist()):  # over-read canary
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    if masks is None:
        masks = random_tree_masks(rng, B, kq)
    scale = float(np.float32(d ** -0.5))
    P.log(f"[tree] {what} seed={seed} lengths={lengths} H={H} Hkv={Hkv} kq={kq} d={d} masks={np.asarray(masks).tolist()}")
    o, lse = binding.verify_tree(q, k, v, torch.from_numpy(sl).cuda(), int(sl.max()), as_i32(masks).cuda(),
                                 scale=scale)
    torch.cuda.synchronize()
    kn = np.nan_to_num(synth.to_f64(k), nan=0.0)
    vn = np.nan_to_num(synth.to_f64(v), nan=0.0)
    o_ref, l_ref = ref.verify_tree(synth.to_f64(q), kn, vn, sl, masks, scale)
    res = P.compare(synth.to_f64(o), synth.to_f64(lse), o_ref, l_ref, "bf16", what)
    P.log(f"    ok {res}")
    return q, k, v, sl, o, lse


@pytest.mark.parametrize("H,Hkv,kq", [(32, 8, 5), (32, 8, 8), (8, 8, 16), (8, 8, 32), (16, 1, 2),
                                      (32, 8, 16), (16, 8, 32), (64, 8, 8), (8, 1, 7)])
@pytest.mark.parametrize("d", [64, 128])
def test_random_trees(H, Hkv, kq, d):
    tree_case(kq * 7 + d, [3000, 40, kq, 1025, 700], H, Hkv, kq, d, what="random-trees")


def test_arbitrary_masks_and_empty_rows():
    """Masks that are not trees, rows that see nothing (no cache, mask 0)."""
    kq = 6
    masks = np.array([[0, 1, 2, 0b110000, 0x3F, 0b100001],
                      [0x3F] * 6,
                      [1, 2, 4, 8, 16, 32]])
    tree_case(9, [6, 300, 7], 8, 2, kq, 128, masks=masks, what="arbitrary-masks")


def test_chain_mask_bitwise_equals_verify():
    from exact_attention_04_amd import binding
    kq = 5
    lengths = [5000, 33, 2049, 5]
    masks = np.array([[(1 << (i + 1)) - 1 for i in range(kq)]] * len(lengths))
    q, k, v, sl, o_t, l_t = tree_case(4, lengths, 32, 8, kq, 128, masks=masks, what="chain")
    o_c, l_c = binding.verify(q, k, v, torch.from_numpy(sl).cuda(), int(sl.max()), scale=float(np.float32(128 ** -0.5)))
    torch.cuda.synchronize()
    assert torch.equal(o_t, o_c)
    assert torch.equal(l_t, l_c)


def test_tree_on_verify_workload():
    """Seed-4 verify workload with a random 5-node tree per sequence."""
    from exact_attention_04_amd import binding
    w = synth.VERIFY_BF16
    q, k, v, sl = synth.verify_inputs(w, "cuda")
    sl_h = sl.cpu().numpy()
    masks = random_tree_masks(np.random.default_rng(44), w.B, w.kq)
    P.log(f"[tree] {w.name} masks={masks.tolist()}")
    o, lse = binding.verify_tree(q, k, v, sl, int(sl_h.max()), as_i32(masks).cuda(), scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.verify_tree(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), sl_h, masks, w.scale)
    P.log(f"    ok {P.compare(synth.to_f64(o), synth.to_f64(lse), o_ref, l_ref, 'bf16', w.name)}")


def test_tree_many_sequences():
    """More than 64 sequences, each with its own random draft tree."""
    rng = np.random.default_rng(93)
    kq = 6
    lengths = [int(x) for x in rng.integers(kq, 600, 90)]
    tree_case(94, lengths, 8, 2, kq, 64, what="tree-many-sequences")
