"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * attn_fwd on the causal prefill workload B=4, H=32, S=8192, d=128, bf16
    (the tiled forward with online softmax), and
  * attn_verify on the speculative-verify workload (8 sequences, 32 query
    heads over 8 KV heads, 5 new tokens each, d=128, bf16, ragged caches of
    1024..16384 + 5 keys): split-KV kernel plus merge kernel.

Inputs are resident in HBM before the timed region.  The verify cache is
rotated over 4 independent copies so that a call cannot be served from the
256 MB last-level cache left warm by the previous call.  Times come from HIP
events recorded on the stream the library launches on: each leg's time per
call is the mean over back-to-back calls timed as one block (one event pair
around all of them); the spread (p10, p50, p90) comes from an event pair
around every call, which adds a few microseconds to each, so the mean of
those per-call figures is reported separately (per_call_event_mean_us).
The timed steps themselves (prefill, then verify, events around each leg)
give ms_per_step and the in-step per-call spread.  The GPU's clocks take
tens of milliseconds to settle under a new load, so whole steps run for a
second before the warmup steps, and every other leg runs back to back for
half a second before it is timed.

Prints one JSON line: value = prefill TFLOP/s (causal FLOPs halved:
2*B*H*S^2*d per call); the verify throughput (algorithmic bytes: K and V of
every valid cache row plus Q, O and LSE, per call) rides along under
"verify".  The CPU-baseline leg times the fp64 oracle on a bounded sample of
the prefill workload (whole heads) on the host cores.

After the timed steps, the entry points beyond the step are measured on the
same verify workload, each against the HBM roofline ("extras"): attn_verify
back to back (without the prefill before each call), attn_verify_paged
(64-key pages in random physical order), attn_verify_tree (a random 5-node
draft tree per sequence) and attn_spec_accept (8 sequences, k = 5, a
131072-entry vocabulary); attn_bwd on the prefill workload against the bf16
matrix peak; and attn_fwd on the other prefill workloads (S = 2048 batch,
S = 32768 at d = 128 and d = 64, the small fp32 case).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal prefill TFLOP/s @S=8192,d=128 (% MFMA peak); verify KV GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
SETTLE_S = 0.5              # seconds of back-to-back calls before each leg is timed
STEP_SETTLE_S = 1.0         # seconds of whole steps before the warmup steps


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(leg: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f)[leg]
        h = hashlib.sha1()
        for src in entry["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != entry["sources_sha1"]:
            return None
        return entry["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def verify_algorithmic_bytes(w, seqlens: np.ndarray) -> int:
    kv = int(seqlens.sum()) * w.Hkv * w.d * 2 * 2          # K and V rows that are read, bf16
    qo = 2 * w.B * w.H * w.kq * w.d * 2                    # Q read, O written
    lse = w.B * w.H * w.kq * 4
    return kv + qo + lse


def max_errors(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray) -> dict:
    """Largest |O - O_ref| (with |O_ref| there) and |LSE - LSE_ref| over every element."""
    err_o = np.abs(o_gpu - o_ref)
    i = np.unravel_index(int(np.argmax(err_o)), err_o.shape)
    fin = np.isfinite(lse_ref)
    return {"max_abs_err_o": float(err_o[i]), "abs_o_ref_at_max": float(abs(o_ref[i])),
            "max_abs_err_lse": float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0,
            "rows_compared": int(np.prod(lse_ref.shape)), "tolerance": {"o": 2e-2, "lse": 1e-3}}


def cpu_baseline(w, o_gpu, lse_gpu) -> tuple:
    """The oracle, as it is, on every head of the prefill workload; its
    output is also compared with the GPU's (every row)."""
    from exact_attention_04_amd import synth
    from oracle import ref_attention as ref

    cores = min(16, ref.default_workers())
    n_heads = w.B * w.H
    q, k, v = synth.prefill_inputs(w, "cpu")
    heads = [(i // w.H, i % w.H) for i in range(n_heads)]
    qn, kn, vn = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    log(f"cpu baseline: oracle on {n_heads} heads x {w.Sq} rows with {cores} threads")
    t0 = time.perf_counter()
    o_ref, lse_ref = ref.attention(qn, kn, vn, w.causal, w.scale, heads=heads, workers=cores)
    dt = time.perf_counter() - t0
    flops = n_heads * (2.0 * w.Sq * w.Sk * w.d)  # causal convention: half of 4*S^2*d
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"all {n_heads} (batch, head) pairs of {w.name}, all {w.Sq} query rows, "
                      f"fp64 materialised rows, {cores} worker threads (one BLAS thread each); {dt:.1f} s wall; "
                      f"causal FLOPs halved like the GPU figure"}
    return base, max_errors(synth.to_f64(o_gpu), synth.to_f64(lse_gpu), o_ref, lse_ref)


def stats_us(us: np.ndarray, block: float = None) -> dict:
    """Time per call and the spread of per-call durations (us).

    us_per_call is `block` when given: the mean over back-to-back calls
    timed as one block (one event pair), which is the throughput figure.
    The per-call durations come from an event pair around every call; each
    such pair adds a few microseconds of its own to the call it brackets
    (about 3-5 us measured on 75-160 us calls), so their mean is kept
    separately as per_call_event_mean_us and only their spread (p10, p50,
    p90) is reported beside the block figure."""
    mean = float(us.mean()) if block is None else float(block)
    return {"us_per_call": round(mean, 2), "per_call_event_mean_us": round(float(us.mean()), 2),
            "p10_us": round(float(np.percentile(us, 10)), 2), "p50_us": round(float(np.percentile(us, 50)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2), "calls": int(len(us))}


def host_info() -> dict:
    """CPU model, threads available to this process and the ROCm version."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                rocm = f.read().strip()
                break
        except OSError:
            pass
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        threads = os.cpu_count()
    return {"cpu_model": model, "cpu_threads_available": threads, "rocm_version": rocm}


def parse_amdsmi(text: str) -> dict:
    """Socket power (W) and the GFX (XCD) clocks (MHz) from `amd-smi metric -p -c` output."""
    import re
    power = [float(x) for x in re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)]
    clocks = []
    lines = text.splitlines()
    for i, line in enumerate(lines):
        if re.match(r"\s*GFX_\d+:\s*$", line) and i + 1 < len(lines):
            m = re.match(r"\s*CLK:\s*([0-9.]+)\s*MHz", lines[i + 1])
            if m:
                clocks.append(float(m.group(1)))
    return {"power_w": power, "gfx_clk_mhz": clocks}


def sample_clocks(run_for_s: float, call, stream, sample_at=(2.0, 3.0)) -> dict:
    """Board power and XCD clocks read with amd-smi while `call` runs back to
    back for run_for_s seconds (the clocks settle under the power limit after
    a second or two), or None when amd-smi is not available."""
    import shutil
    import subprocess
    import threading
    import torch
    smi = shutil.which("amd-smi")
    if smi is None:
        return None
    texts = []

    def sampler():
        t0 = time.perf_counter()
        for t in sample_at:
            time.sleep(max(0.0, t - (time.perf_counter() - t0)))
            try:
                r = subprocess.run([smi, "metric", "-p", "-c", "-g", "0"], capture_output=True, text=True,
                                   timeout=10)
                texts.append(r.stdout)
            except (OSError, subprocess.SubprocessError):
                pass
    th = threading.Thread(target=sampler)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < run_for_s:
        for _ in range(20):
            call()
            n += 1
        stream.synchronize()
    th.join()
    torch.cuda.synchronize()
    got = [parse_amdsmi(t) for t in texts]
    clk = [c for g in got for c in g["gfx_clk_mhz"]]
    pw = [p for g in got for p in g["power_w"]]
    if not clk:
        return None
    return {"samples": len(got), "calls": n, "gfx_clk_mhz_min": min(clk), "gfx_clk_mhz_mean": round(sum(clk) / len(clk), 1),
            "gfx_clk_mhz_max": max(clk), "socket_power_w": round(sum(pw) / len(pw), 1) if pw else None}


def timed_us(fn, n: int, stream) -> np.ndarray:
    """Per-call durations (us) of fn(i) from HIP events on `stream`."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i].record(stream)
        fn(i)
    ev[n].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)])


def block_us(fn, n: int, stream) -> float:
    """Mean time per call (us) of n back-to-back calls fn(0..n-1), timed as
    one block by a HIP event pair on `stream`."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def settle(fn, seconds: float, stream) -> int:
    """Run fn(0), fn(1), ... back to back for about `seconds` of wall time.

    Under load the GPU's clocks move for tens of milliseconds: up from idle
    (the first prefill calls after a pause run 10-30% slower) and down as
    the board reaches its power limit.  Every leg runs this long before it
    is timed, so the figures describe the steady state.  Returns the number
    of calls made."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(n)
            n += 1
        stream.synchronize()
    return n


def leg_us(fn, n: int, stream):
    """(block-timed us per call, per-call durations) of n calls each."""
    return block_us(fn, n, stream), timed_us(fn, n, stream)


def paged_copy(k, v, seqlens, page, rng):
    """Pages [num_pages, Hkv, page, d] holding caches [B, Hkv, S, d] in random
    physical order, and the int32 block table."""
    import torch
    B, Hkv, S, d = k.shape
    nblk = [(int(s) + page - 1) // page for s in seqlens]
    perm = rng.permutation(sum(nblk))
    kp = torch.zeros((len(perm), Hkv, page, d), dtype=k.dtype, device=k.device)
    vp = torch.zeros_like(kp)
    table = np.full((B, max(nblk)), -1, dtype=np.int32)
    i = 0
    for b in range(B):
        for blk in range(nblk[b]):
            ph = int(perm[i])
            i += 1
            table[b, blk] = ph
            n = min(page, int(seqlens[b]) - blk * page)
            kp[ph, :, :n] = k[b, :, blk * page:blk * page + n]
            vp[ph, :, :n] = v[b, :, blk * page:blk * page + n]
    return kp, vp, torch.from_numpy(table).to(k.device)


def tree_masks(rng, B, kq):
    rows = []
    for _ in range(B):
        parents = [-1] + [int(rng.integers(0, i)) for i in range(1, kq)]
        row = []
        for i in range(kq):
            m, j = 0, i
            while j >= 0:
                m |= 1 << j
                j = parents[j]
            row.append(m)
        rows.append(row)
    return np.array(rows, dtype=np.int32)


def spec_inputs(B, k, V, dev, seed=12):
    import torch
    rng = np.random.default_rng(seed)
    g = rng.gamma(0.3, size=(B, k + 1, V)).astype(np.float32)
    p = g / g.sum(-1, keepdims=True)
    n = rng.gamma(0.3, size=(B, k, V)).astype(np.float32)
    q = (0.8 * p[:, :k] + 0.2 * n / n.sum(-1, keepdims=True)).astype(np.float32)
    x = np.argmax(q, axis=-1).astype(np.int32)
    ua = rng.random((B, k), dtype=np.float32)
    us = rng.random(B, dtype=np.float32)
    return [torch.from_numpy(a).to(dev) for a in (x, q, p, ua, us)]


def cpu_rate(fn, work: float, unit: str, sample: str, threads: int = 1) -> dict:
    """The oracle as it is, timed once on the host: work / seconds.  With
    threads == 1 its BLAS calls are held to one thread, so `cores` is what
    ran; callers that pass threads > 1 run the oracle with that many worker
    threads of one BLAS thread each."""
    from oracle.ref_attention import _blas_one_thread
    with _blas_one_thread():
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
    scale = 1e9 if unit == "GB/s" else 1e12
    return {"value": round(work / dt / scale, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{sample}; {dt:.2f} s wall on {threads} thread{'s' if threads > 1 else ''}"}


def extras(dev, wv, vq, caches, vsl, seqlens, max_len, stream, cpu: bool = False) -> dict:
    import torch
    from exact_attention_04_amd import binding, synth
    from_dev = synth.to_f64
    rng = np.random.default_rng(7)
    vbytes = verify_algorithmic_bytes(wv, seqlens)
    out = {}
    # plain verify, back to back (the timed step runs it right after the
    # prefill kernel has written its 268 MB of O)
    def plain(i):
        kc, vc = caches[i % len(caches)]
        binding.verify(vq, kc, vc, vsl, max_len, scale=wv.scale, out=o, lse=lse, workspace=ws)
    o = torch.empty_like(vq)
    lse = torch.empty((wv.B, wv.H, wv.kq), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.attn_verify_workspace_bytes(wv.B, wv.H, wv.Hkv, wv.kq, wv.d), dtype=torch.uint8,
                     device=dev)
    settle(plain, SETTLE_S, stream)
    blk, us = leg_us(plain, 200, stream)
    out["verify_back_to_back"] = {**stats_us(us, blk),
                                  "roofline": {"bound": "hbm", "achieved": round(vbytes / blk / 1e3, 1),
                                               "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                               "frac": round(vbytes / blk / 1e3 / PEAK_HBM_GBPS, 4),
                                               "traffic": None}}
    if cpu:
        from oracle import ref_attention as ref
        qn, kn, vn = from_dev(vq), from_dev(caches[0][0]), from_dev(caches[0][1])
        out["verify_back_to_back"]["cpu_baseline"] = cpu_rate(
            lambda: ref.verify(qn, kn, vn, seqlens, wv.scale), vbytes, "GB/s",
            f"the whole {wv.name} call (fp64, materialised rows), rated by the same algorithmic bytes")
    # the same shape on the other seeds' length mixes (each rotated over
    # four cache copies like the timed step); seed 0's 205 MB would fit in
    # the last-level cache without the rotation
    sweep = {}
    for seed in (0, 1, 2, 3):
        w = dataclasses.replace(wv, seed=seed, name=f"{wv.name}_seed{seed}")
        sq, sk, sv, ssl = synth.verify_inputs(w, dev)
        slen = ssl.cpu().numpy()
        rot = [(sk, sv)] + [(sk.clone(), sv.clone()) for _ in range(3)]

        def seeded(i):
            kc, vc = rot[i % len(rot)]
            binding.verify(sq, kc, vc, ssl, int(slen.max()), scale=w.scale, out=o, lse=lse, workspace=ws)
        settle(seeded, SETTLE_S, stream)
        blk, us = leg_us(seeded, 200, stream)
        sb = verify_algorithmic_bytes(w, slen)
        sweep[f"seed{seed}"] = {"sum_seqlens": int(slen.sum()), "algorithmic_bytes": int(sb),
                                **stats_us(us, blk),
                                "GB/s": round(sb / blk / 1e3, 1),
                                "frac": round(sb / blk / 1e3 / PEAK_HBM_GBPS, 4)}
        del sq, sk, sv, ssl, rot
        torch.cuda.empty_cache()
    out["verify_seeds"] = sweep
    # paged verify: two page pools in different random orders, alternated
    pools = [paged_copy(kc, vc, seqlens, 64, rng) for kc, vc in caches[:2]]

    def paged(i):
        kp, vp, table = pools[i % 2]
        binding.verify_paged(vq, kp, vp, table, vsl, max_len, scale=wv.scale, out=o, lse=lse, workspace=ws)
    settle(paged, SETTLE_S, stream)
    blk, us = leg_us(paged, 200, stream)
    pbytes = vbytes + int(sum((int(s) + 63) // 64 for s in seqlens)) * 4
    out["verify_paged"] = {"page": 64, **stats_us(us, blk),
                           "roofline": {"bound": "hbm", "achieved": round(pbytes / blk / 1e3, 1),
                                        "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                        "frac": round(pbytes / blk / 1e3 / PEAK_HBM_GBPS, 4),
                                        "traffic": None}}
    if cpu:
        kp, vp, table = pools[0]
        kpn, vpn, tabn = from_dev(kp), from_dev(vp), table.cpu().numpy()
        out["verify_paged"]["cpu_baseline"] = cpu_rate(
            lambda: ref.verify_paged(qn, kpn, vpn, tabn, seqlens, 64, wv.scale), pbytes, "GB/s",
            "the whole paged call: gather of the logical cache, then verify (fp64)")
        del kpn, vpn
    del pools
    # tree verify: a random 5-node tree per sequence
    tm = torch.from_numpy(tree_masks(rng, wv.B, wv.kq)).to(dev)

    def tree(i):
        kc, vc = caches[i % len(caches)]
        binding.verify_tree(vq, kc, vc, vsl, max_len, tm, scale=wv.scale, out=o, lse=lse, workspace=ws)
    settle(tree, SETTLE_S, stream)
    blk, us = leg_us(tree, 200, stream)
    out["verify_tree"] = {**stats_us(us, blk),
                          "roofline": {"bound": "hbm", "achieved": round(vbytes / blk / 1e3, 1),
                                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                       "frac": round(vbytes / blk / 1e3 / PEAK_HBM_GBPS, 4),
                                       "traffic": None}}
    if cpu:
        tmn = tm.cpu().numpy()
        out["verify_tree"]["cpu_baseline"] = cpu_rate(
            lambda: ref.verify_tree(qn, kn, vn, seqlens, tmn, wv.scale), vbytes, "GB/s",
            "the whole tree-verify call (fp64, explicit visibility per row)")
        del qn, kn, vn
    # acceptance rule: 8 sequences, k = 5, V = 131072; two input copies
    B, k, V = wv.B, wv.kq, 131072
    sets = [spec_inputs(B, k, V, dev, seed) for seed in (12, 13)]
    sws_bytes = binding.attn_spec_accept_workspace_bytes(B, V)
    sws = torch.empty(sws_bytes, dtype=torch.uint8, device=dev)
    outs = [(torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, k + 1), dtype=torch.int32, device=dev))
            for _ in sets]
    for s_, (n_, t_) in zip(sets, outs):  # through the tensor binding once (its checks), then raw calls
        binding.spec_accept(*s_, workspace=sws, n_accepted=n_, out_tokens=t_)
    raw = [tuple(t.data_ptr() for t in s_) + (n_.data_ptr(), t_.data_ptr(), B, k, V, sws.data_ptr(), sws_bytes,
                                              stream.cuda_stream) for s_, (n_, t_) in zip(sets, outs)]

    def spec(i):
        # the C entry point directly: the kernels take about 11 us, close to the
        # tensor binding's own host time per call, which would otherwise be
        # what a block of back-to-back calls measures
        rc = binding.attn_spec_accept(*raw[i % 2])
        assert rc == binding.ATTN_OK, binding.attn_strerror(rc)
    settle(spec, SETTLE_S, stream)
    blk, us = leg_us(spec, 200, stream)
    # bytes: the sampled row of p (and of q after a rejection) for every
    # sequence, plus the k looked-up entries; averaged over the two sets
    acc = [n_.cpu().numpy() for n_, _ in outs]
    sbytes = float(np.mean([sum(V * 4 * (2 if j < k else 1) + k * 16 for j in a.tolist()) for a in acc]))
    out["spec_accept"] = {"B": B, "k": k, "V": V, **stats_us(us, blk),
                          "roofline": {"bound": "hbm", "achieved": round(sbytes / blk / 1e3, 1),
                                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                       "frac": round(sbytes / blk / 1e3 / PEAK_HBM_GBPS, 4),
                                       "traffic": None}}
    if cpu:
        from oracle import ref_spec
        xs, qs, ps, uas, uss = (t.cpu().numpy() for t in sets[0])
        out["spec_accept"]["cpu_baseline"] = cpu_rate(
            lambda: ref_spec.spec_accept(xs, qs, ps, uas, uss), float(sbytes), "GB/s",
            "one call on the first input set (numpy; fixed-point sums in int64)")
    return out


def backward_leg(dev, wp, q, k, v, o, lse, stream, cpu: bool = False) -> dict:
    """attn_bwd on the prefill workload: the forward's O and LSE, a seeded
    N(0,1) dO.  Algorithmic FLOPs: the five S-sized products (S, dP, dV, dQ,
    dK) at 2*S*S*d each per head, halved for the causal mask -- 2.5 times the
    forward's count; the kernels recompute S and dP once more, which is not
    counted."""
    import torch
    from exact_attention_04_amd import binding, synth
    do = synth.normal(np.random.default_rng(wp.seed + 1), (wp.B, wp.H, wp.Sq, wp.d), "bf16").to(dev)
    ws = torch.empty(binding.attn_bwd_workspace_bytes(wp.B, wp.H, wp.Sq), dtype=torch.uint8, device=dev)

    def bwd(i):
        binding.bwd(q, k, v, o, lse, do, causal=True, scale=wp.scale, workspace=ws)
    settle(bwd, SETTLE_S, stream)
    blk, us = leg_us(bwd, 10, stream)
    flops = 2.5 * wp.flops()
    tf = flops / (blk * 1e-6) / 1e12
    out = {"workload": wp.name, **stats_us(us, blk),
           "algorithmic_flops": flops,
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("backward")}}
    if cpu:
        from oracle import ref_attention as ref
        n = min(16, ref.default_workers())
        part = (slice(0, 1), slice(0, n))  # the first n heads of batch 0
        qn, kn, vn, dn = (synth.to_f64(t[part]) for t in (q, k, v, do))
        out["cpu_baseline"] = cpu_rate(
            lambda: ref.attention_backward(qn, kn, vn, dn, True, wp.scale, workers=n), flops * n / (wp.B * wp.H),
            "TFLOP/s",
            f"{n} (batch, head) pairs of {wp.name}: all {wp.Sq} rows, fp64 materialised S, P, dP, dS; rated by "
            f"those heads' share of the algorithmic FLOPs", threads=n)
    return out


def other_prefill(dev, stream) -> dict:
    """attn_fwd on the other prefill workloads (each timed alone, inputs
    resident): the 2048-token batch, the 32768-token single sequences at
    d = 128 and d = 64, and the small fp32 case (launch-bound: time only)."""
    import torch
    from exact_attention_04_amd import binding, synth
    out = {}
    for w in (synth.CAUSAL_BF16_S2048, synth.CAUSAL_BF16_S32768_D128, synth.CAUSAL_BF16_S32768_D64,
              synth.NONCAUSAL_F32_S256):
        q, k, v = synth.prefill_inputs(w, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)

        def call(i):
            binding.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        settle(call, SETTLE_S, stream)
        blk, us = leg_us(call, 20, stream)
        tf = w.flops() / (blk * 1e-6) / 1e12
        e = {**stats_us(us, blk), "TFLOP/s": round(tf, 2)}
        if w.dtype == "bf16":
            e["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None}
        out[w.name] = e
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return out


def profile_leg(args, dev) -> int:
    """Run one leg warmup+steps times with no timing or output (for rocprofv3)."""
    import torch
    from exact_attention_04_amd import binding, synth

    n = args.warmup + args.steps
    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(n):
            dst.copy_(src)
    elif args.only == "prefill":
        w = {x.name: x for x in synth.PREFILL_WORKLOADS}[args.workload]
        q, k, v = synth.prefill_inputs(w, dev)
        for _ in range(n):
            binding.fwd(q, k, v, causal=w.causal, scale=w.scale)
    elif args.only == "backward":
        w = synth.CAUSAL_BF16_S8192
        q, k, v = synth.prefill_inputs(w, dev)
        o, lse = binding.fwd(q, k, v, causal=True, scale=w.scale)
        do = synth.normal(np.random.default_rng(w.seed + 1), (w.B, w.H, w.Sq, w.d), "bf16").to(dev)
        for _ in range(n):
            binding.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    else:
        w = synth.VERIFY_BF16
        q, kc, vc, sl = synth.verify_inputs(w, dev)
        caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(3)]
        m = int(sl.max())
        for i in range(n):
            binding.verify(q, caches[i % 4][0], caches[i % 4][1], sl, m, scale=w.scale)
    torch.cuda.synchronize()
    log(f"profile leg {args.only}: {n} calls done")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "verify", "backward", "copy"], default=None,
                    help="profiling aid: run just one leg (no JSON line); 'copy' runs a plain "
                         "1 GiB device-to-device copy used to calibrate the HBM byte counters")
    ap.add_argument("--workload", default="causal_bf16_b4h32s8192d128",
                    help="with --only prefill: the prefill workload to run (by name)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the attention path "
              f"shards by head with no exchange, so N GPUs run N independent copies)", file=sys.stderr)
        return 2

    import torch
    from exact_attention_04_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.only is not None:
        return profile_leg(args, dev)
    props = torch.cuda.get_device_properties(dev)
    wp = synth.CAUSAL_BF16_S8192
    wv = synth.VERIFY_BF16

    # ---- inputs resident in HBM
    q, k, v = synth.prefill_inputs(wp, dev)
    o = torch.empty_like(q)
    lse = torch.empty((wp.B, wp.H, wp.Sq), dtype=torch.float32, device=dev)
    vq, vk, vv, vsl = synth.verify_inputs(wv, dev)
    seqlens = vsl.cpu().numpy()
    max_len = int(seqlens.max())
    n_rot = 4
    caches = [(vk, vv)] + [(vk.clone(), vv.clone()) for _ in range(n_rot - 1)]
    vo = torch.empty_like(vq)
    vlse = torch.empty((wv.B, wv.H, wv.kq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, binding.attn_verify_workspace_bytes(wv.B, wv.H, wv.Hkv, wv.kq, wv.d)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def prefill():
        binding.fwd(q, k, v, causal=True, scale=wp.scale, out=o, lse=lse)

    def verify(i):
        kc, vc = caches[i % n_rot]
        binding.verify(vq, kc, vc, vsl, max_len, scale=wv.scale, out=vo, lse=vlse, workspace=ws)

    def step(i):
        prefill()
        verify(i)
    settle(step, STEP_SETTLE_S, stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        e[2].record(stream)
        verify(i)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    ver_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    # each leg's throughput: the same calls back to back, timed as one block
    # (the event pairs around every call in the step add a few us to each)
    pre_blk_us = block_us(lambda i: prefill(), args.steps, stream)
    ver_blk_us = block_us(verify, 200, stream)
    # clocks and board power while the prefill runs back to back (amd-smi)
    clocks = sample_clocks(4.0, prefill, stream)
    flops = wp.flops()
    tflops = flops / (pre_blk_us * 1e-6) / 1e12
    vbytes = verify_algorithmic_bytes(wv, seqlens)
    gbps = vbytes / (ver_blk_us * 1e-6) / 1e9
    log(f"device {props.name} CUs={props.multi_processor_count}")
    log(f"prefill: {pre_blk_us / 1e3:.3f} ms per call back to back; in the step mean {pre_ms.mean():.3f} ms "
        f"(p10 {np.percentile(pre_ms, 10):.3f}, p90 {np.percentile(pre_ms, 90):.3f})"
        f" -> {tflops:.1f} TFLOP/s = {100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")
    log(f"verify: {ver_blk_us:.1f} us per call back to back; in the step mean {ver_ms.mean() * 1e3:.1f} us "
        f"(p10 {np.percentile(ver_ms, 10) * 1e3:.1f}, p90 {np.percentile(ver_ms, 90) * 1e3:.1f})"
        f" -> {gbps:.0f} GB/s = {100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM")

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": STEP_SETTLE_S,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wp.name} + {wv.name}",
                   "prefill": {"B": wp.B, "H": wp.H, "Hkv": wp.Hkv, "S": wp.Sq, "d": wp.d, "causal": True,
                               "seed": wp.seed},
                   "verify": {"B": wv.B, "H": wv.H, "Hkv": wv.Hkv, "kq": wv.kq, "d": wv.d, "seed": wv.seed,
                              "seqlens_k": seqlens.tolist(), "cache_copies_rotated": n_rot}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("prefill")},
        "prefill_stats": stats_us(pre_ms * 1e3, pre_blk_us),
        "verify": {"value": round(gbps, 1), "unit": "GB/s", **stats_us(ver_ms * 1e3, ver_blk_us),
                   "block_calls": 200,
                   "algorithmic_bytes": vbytes,
                   "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic("verify")}},
        "prefill_ms": round(pre_blk_us / 1e3, 4),
        "device": {"name": props.name, "cus": props.multi_processor_count, "clocks_under_prefill": clocks},
        "host": host_info(),
    }
    out["extras"] = extras(dev, wv, vq, caches, vsl, seqlens, max_len, stream, cpu=not args.no_cpu_baseline)
    for name, e in out["extras"].items():
        if name == "verify_seeds":
            for sd, r in e.items():
                log(f"verify {sd}: {r['us_per_call']:.1f} us -> {r['GB/s']:.0f} GB/s = {100 * r['frac']:.1f}% of HBM")
            continue
        log(f"{name}: {e['us_per_call']:.1f} us -> {e['roofline']['achieved']:.0f} GB/s "
            f"= {100 * e['roofline']['frac']:.1f}% of HBM")
    out["extras"]["backward"] = b = backward_leg(dev, wp, q, k, v, o, lse, stream, cpu=not args.no_cpu_baseline)
    log(f"backward: {b['us_per_call'] / 1e3:.3f} ms -> {b['roofline']['achieved']:.1f} TFLOP/s "
        f"= {100 * b['roofline']['frac']:.1f}% of bf16 peak")
    out["extras"]["prefill_other"] = po = other_prefill(dev, stream)
    for name, e in po.items():
        log(f"{name}: {e['us_per_call']:.1f} us -> {e['TFLOP/s']:.1f} TFLOP/s")
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(wp, o, lse)
        from oracle import ref_attention as ref
        vo_ref, vl_ref = ref.verify(synth.to_f64(vq), synth.to_f64(vk), synth.to_f64(vv), seqlens, wv.scale)
        out["verify"]["parity"] = max_errors(synth.to_f64(vo), synth.to_f64(vlse), vo_ref, vl_ref)
        log(f"parity (every row): prefill {out['parity']}; verify {out['verify']['parity']}")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
