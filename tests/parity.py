"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on exactly the same (rounded) inputs, compare element by
element against the stated tolerances.

Tolerances (max absolute error):
  * fp32 inputs:  O and LSE <= 1e-5;
  * bf16 inputs:  O <= 2e-2, LSE <= 1e-3 (fp32 accumulation).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from exact_attention_04_amd import synth
from oracle import ref_attention as ref

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def workers() -> int:
    return min(16, ref.default_workers())


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, dtype: str,
            what: str = "") -> dict:
    """Assert parity; returns the observed errors."""
    tol_o, tol_l = TOL[dtype]
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err_o = np.abs(o_gpu - o_ref)
    empty_ref = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse_gpu), empty_ref, err_msg=f"{what}: empty-row pattern")
    fin = ~empty_ref
    err_l = np.abs(lse_gpu[fin] - lse_ref[fin]) if fin.any() else np.zeros(1)
    res = {"max_err_o": float(err_o.max()) if err_o.size else 0.0,
           "max_err_lse": float(err_l.max()) if err_l.size else 0.0}
    if err_o.size:
        i = np.unravel_index(np.argmax(err_o), err_o.shape)
        res["abs_o_at_max"] = float(abs(o_ref[i]))
    assert res["max_err_o"] <= tol_o, f"{what}: max|dO| {res} > {tol_o}"
    assert res["max_err_lse"] <= tol_l, f"{what}: max|dLSE| {res} > {tol_l}"
    # empty rows: exactly zero output
    if empty_ref.any():
        assert np.all(o_gpu[empty_ref] == 0), f"{what}: empty rows must be 0"
    return res


def run_fwd(q, k, v, causal, scale):
    from exact_attention_04_amd import binding
    o, lse = binding.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def fwd_case(seed, B, H, Hkv, Sq, Sk, d, causal, dtype, q_mult=1.0, rows=None, heads=None, what=""):
    """Full (or sampled) parity of attn_fwd on one seeded case."""
    q, k, v = synth.random_qkv(seed, B, H, Hkv, Sq, Sk, d, dtype, device="cuda", q_mult=q_mult)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    log(f"[fwd] {what} seed={seed} B={B} H={H} Hkv={Hkv} Sq={Sq} Sk={Sk} d={d} causal={causal} {dtype}")
    o, lse = run_fwd(q, k, v, causal, scale)
    return check_fwd(q, k, v, o, lse, causal, scale, dtype, rows=rows, heads=heads, what=what)


def check_fwd(q, k, v, o, lse, causal, scale, dtype, rows=None, heads=None, what=""):
    qn, kn, vn = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    o_ref, l_ref = ref.attention(qn, kn, vn, causal, scale, rows=rows, heads=heads, workers=workers())
    o_g, l_g = synth.to_f64(o), synth.to_f64(lse)
    if rows is not None:
        o_g, l_g = o_g[:, :, rows], l_g[:, :, rows]
    if heads is not None:
        bi = [b for b, _ in heads]
        hi = [h for _, h in heads]
        o_g, l_g, o_ref, l_ref = o_g[bi, hi], l_g[bi, hi], o_ref[bi, hi], l_ref[bi, hi]
    res = compare(o_g, l_g, o_ref, l_ref, dtype, what)
    log(f"    ok {res}")
    return res
