"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the smoke check and the benchmark, and by
both sides of every parity check (the HIP path and the CPU oracle).  It holds
none of the attention arithmetic: it only draws i.i.d. standard-normal tensors
from a seed, rounds them to the storage dtype, and draws the ragged KV-cache
lengths of the speculative-verify workload.

Recipe (the same for every workload):
  * ``rng = numpy.random.default_rng(seed)``;
  * verify workloads draw the per-sequence pre-existing cache lengths first,
    ``rng.integers(lo, hi + 1, B)`` (inclusive bounds), then Q, K, V;
  * Q, K, V are ``rng.standard_normal(shape, dtype=float32)`` in that order;
  * bf16 tensors are the fp32 draws rounded to nearest-even by
    ``torch.Tensor.to(torch.bfloat16)``; the oracle receives exactly these
    rounded values, widened to float64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Prefill:
    """A self-attention / cross-attention forward workload."""
    name: str
    seed: int
    B: int
    H: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    causal: bool
    dtype: str
    q_mult: float = 1.0  # Q is multiplied by this after rounding (exact for powers of two)

    @property
    def scale(self) -> float:
        # 1/sqrt(d) rounded to fp32, the value handed to the library.
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def flops(self) -> float:
        """Matmul FLOPs: 4*B*H*Sq*Sk*d, halved for a causal mask (Sq == Sk)."""
        f = 4.0 * self.B * self.H * self.Sq * self.Sk * self.d
        return f / 2 if self.causal else f


@dataclasses.dataclass(frozen=True)
class Verify:
    """Speculative-verify workload: kq new queries per sequence against a ragged cache."""
    name: str
    seed: int
    B: int
    H: int
    Hkv: int
    kq: int
    d: int
    len_lo: int
    len_hi: int
    dtype: str = BF16

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The workloads the library is measured and checked on.
NONCAUSAL_F32_S256 = Prefill("noncausal_f32_b1h2s256d64", 1, 1, 2, 2, 256, 256, 64, False, F32)
CAUSAL_BF16_S2048 = Prefill("causal_bf16_b4h32s2048d128", 2, 4, 32, 32, 2048, 2048, 128, True, BF16)
CAUSAL_BF16_S2048_Q8 = dataclasses.replace(CAUSAL_BF16_S2048, name="causal_bf16_b4h32s2048d128_qx8", q_mult=8.0)
CAUSAL_BF16_S8192 = Prefill("causal_bf16_b4h32s8192d128", 3, 4, 32, 32, 8192, 8192, 128, True, BF16)
VERIFY_BF16 = Verify("verify_bf16_b8h32kv8_kq5_d128", 4, 8, 32, 8, 5, 128, 1024, 16384)
CAUSAL_BF16_S32768_D128 = Prefill("causal_bf16_b1h32s32768d128", 5, 1, 32, 32, 32768, 32768, 128, True, BF16)
CAUSAL_BF16_S32768_D64 = Prefill("causal_bf16_b1h64s32768d64", 5, 1, 64, 64, 32768, 32768, 64, True, BF16)

PREFILL_WORKLOADS = [NONCAUSAL_F32_S256, CAUSAL_BF16_S2048, CAUSAL_BF16_S2048_Q8, CAUSAL_BF16_S8192,
                     CAUSAL_BF16_S32768_D128, CAUSAL_BF16_S32768_D64]


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t.to(_TORCH_DTYPE[dtype]).contiguous()


def normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """One i.i.d. N(0,1) draw of ``shape``, rounded to ``dtype`` (CPU tensor)."""
    return _round(rng.standard_normal(shape, dtype=np.float32), dtype)


def prefill_inputs(w: Prefill, device: str = "cpu"):
    """(q, k, v) for a prefill workload, as contiguous tensors on ``device``."""
    rng = np.random.default_rng(w.seed)
    q = normal(rng, (w.B, w.H, w.Sq, w.d), w.dtype)
    k = normal(rng, (w.B, w.Hkv, w.Sk, w.d), w.dtype)
    v = normal(rng, (w.B, w.Hkv, w.Sk, w.d), w.dtype)
    if w.q_mult != 1.0:
        q = (q * w.q_mult).to(q.dtype)
    return q.to(device), k.to(device), v.to(device)


def random_qkv(seed: int, B: int, H: int, Hkv: int, Sq: int, Sk: int, d: int, dtype: str,
               device: str = "cpu", q_mult: float = 1.0):
    """(q, k, v) for an arbitrary shape, same recipe as :func:`prefill_inputs`."""
    w = Prefill("adhoc", seed, B, H, Hkv, Sq, Sk, d, False, dtype, q_mult)
    return prefill_inputs(w, device)


def verify_lengths(w: Verify) -> np.ndarray:
    """Pre-existing per-sequence cache lengths L_b (the first draw of the seed)."""
    rng = np.random.default_rng(w.seed)
    return rng.integers(w.len_lo, w.len_hi + 1, w.B)


def verify_inputs(w: Verify, device: str = "cpu", lengths: Optional[np.ndarray] = None):
    """(q, k_cache, v_cache, seqlens_k) for a verify workload.

    ``seqlens_k[b] = L_b + kq``: the kq new tokens' keys/values are appended
    after the L_b cached ones, and the cache stride is max_b seqlens_k[b].
    Rows at or beyond ``seqlens_k[b]`` hold N(0,1) draws like the rest; tests
    overwrite them with NaN to expose over-reads.
    """
    rng = np.random.default_rng(w.seed)
    L = rng.integers(w.len_lo, w.len_hi + 1, w.B)
    if lengths is not None:
        L = np.asarray(lengths, dtype=np.int64)
    seqlens = (L + w.kq).astype(np.int32)
    smax = int(seqlens.max())
    q = normal(rng, (w.B, w.H, w.kq, w.d), w.dtype)
    k = normal(rng, (w.B, w.Hkv, smax, w.d), w.dtype)
    v = normal(rng, (w.B, w.Hkv, smax, w.d), w.dtype)
    sl = torch.from_numpy(seqlens)
    return q.to(device), k.to(device), v.to(device), sl.to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (CPU or device) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
