"""Randomized GPU parity across every entry point, from a fixed seed.

Shapes, grouped-query ratios, ragged lengths, head dims, causal flags, tree
masks, page sizes and vocabulary sizes are drawn at random (sizes kept small
so the oracle finishes in seconds) and each case goes through the same
oracle comparison as the hand-picked tests.  The draws are deterministic;
the case list is printed before each step so a failure names its case.
"""
import numpy as np
import pytest

from tests import parity as P
from tests import test_bwd_gpu as TB
from tests import test_paged_gpu as TP
from tests import test_spec_gpu as TS
from tests import test_tree_gpu as TT
from tests import test_verify_gpu as TV

pytestmark = pytest.mark.gpu

N = 12  # cases per entry point


def heads(rng, kq=1, cap=64):
    """(H, Hkv) with (H / Hkv) * kq <= cap."""
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if g * kq <= cap]))
    if G * kq > 32:
        P.log(f"    ({G * kq} packed rows: two query tiles)")
    return Hkv * G, Hkv


@pytest.mark.parametrize("i", range(N))
def test_random_fwd(i):
    rng = np.random.default_rng(100 + i)
    H, Hkv = heads(rng, cap=8)
    B, d = int(rng.integers(1, 3)), int(rng.choice([64, 128]))
    Sq = int(rng.integers(1, 700))
    Sk = Sq if rng.random() < 0.4 else int(rng.integers(1, 700))
    causal = bool(rng.random() < 0.6)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    q_mult = 8.0 if dtype == "bf16" and rng.random() < 0.25 else 1.0
    P.fwd_case(1000 + i, B, H, Hkv, Sq, Sk, d, causal, dtype, q_mult=q_mult, what=f"random{i}")


@pytest.mark.parametrize("i", range(N))
def test_random_verify(i):
    rng = np.random.default_rng(200 + i)
    kq = int(rng.integers(1, 9))
    H, Hkv = heads(rng, kq)
    B, d = int(rng.integers(1, 5)), int(rng.choice([64, 128]))
    lengths = [int(x) for x in rng.integers(0, 4000, B)]
    if rng.random() < 0.3:
        lengths[0] = int(rng.integers(0, kq + 2))  # fewer keys than new queries, or none
    TV.verify_case(2000 + i, lengths, H, Hkv, kq, d, what=f"random{i}")


@pytest.mark.parametrize("i", range(N))
def test_random_tree(i):
    rng = np.random.default_rng(300 + i)
    kq = int(rng.integers(1, 9))
    H, Hkv = heads(rng, kq)
    B, d = int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    lengths = [int(x) for x in rng.integers(kq, 3000, B)]
    TT.tree_case(3000 + i, lengths, H, Hkv, kq, d, what=f"random{i}")


@pytest.mark.parametrize("i", range(N))
def test_random_paged(i):
    rng = np.random.default_rng(400 + i)
    kq = int(rng.integers(1, 9))
    H, Hkv = heads(rng, kq)
    B, d = int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    page = int(rng.choice([16, 32, 64, 128, 256, 1024]))
    lengths = [int(x) for x in rng.integers(0, 3000, B)]
    shared = int(rng.integers(0, 3)) if B > 1 and min(lengths) > 3 * page else 0
    TP.paged_case(4000 + i, lengths, H, Hkv, kq, d, page, shared=shared, what=f"random{i}")


@pytest.mark.parametrize("i", range(N))
def test_random_spec_accept(i):
    rng = np.random.default_rng(500 + i)
    B, k, V = int(rng.integers(1, 17)), int(rng.integers(0, 9)), int(rng.integers(1, 40000))
    TS.run_and_check(*TS.make_case(5000 + i, B, k, V, mix=float(rng.random())), what=f"random{i}")


@pytest.mark.parametrize("i", range(N))
def test_random_bwd(i):
    rng = np.random.default_rng(600 + i)
    H, Hkv = heads(rng, cap=8)
    H = min(H, 8)
    Hkv = Hkv if H % Hkv == 0 else 1
    B, d = int(rng.integers(1, 3)), int(rng.choice([64, 128]))
    Sq = int(rng.integers(1, 500))
    Sk = Sq if rng.random() < 0.4 else int(rng.integers(1, 500))
    TB.bwd_case(6000 + i, B, H, Hkv, Sq, Sk, d, bool(rng.random() < 0.6), what=f"random{i}")
