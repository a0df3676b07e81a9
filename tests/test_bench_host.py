"""Host-side pieces of bench.py (no GPU): the committed HBM-counter summary
and the algorithmic byte count of the verify workload."""
import json
import os

import numpy as np

import bench
from exact_attention_04_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_summary_has_every_leg():
    """profiles/traffic.json holds a counter summary for each measured leg,
    keyed to the sha1 of the sources it was taken on."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        entries = json.load(f)
    for leg in ("prefill", "verify", "backward"):
        e = entries[leg]
        assert e["bytes_per_launch"] > 0 and len(e["sources_sha1"]) == 40 and e["sources"]


def test_traffic_is_none_for_an_unknown_leg():
    assert bench.measured_traffic("no-such-leg") is None


def test_verify_algorithmic_bytes():
    w = synth.VERIFY_BF16
    sl = np.array(synth.verify_lengths(w), dtype=np.int64) + w.kq
    b = bench.verify_algorithmic_bytes(w, sl)
    kv = int(sl.sum()) * w.Hkv * w.d * 2 * 2
    assert b == kv + 2 * w.B * w.H * w.kq * w.d * 2 + w.B * w.H * w.kq * 4
    assert b == 413766656  # the seed-4 workload's 413.77 MB
