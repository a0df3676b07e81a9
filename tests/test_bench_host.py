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


def test_parse_amdsmi_reads_power_and_every_xcd_clock():
    text = "GPU: 0\n    POWER:\n        SOCKET_POWER: 1360 W\n    CLOCK:\n" + "".join(
        f"        GFX_{i}:\n            CLK: {1800 + i} MHz\n            MIN_CLK: 500 MHz\n"
        f"            MAX_CLK: 2400 MHz\n" for i in range(8)) + "        MEM_0:\n            CLK: 1900 MHz\n"
    got = bench.parse_amdsmi(text)
    assert got["power_w"] == [1360.0]
    assert got["gfx_clk_mhz"] == [1800.0 + i for i in range(8)]  # MIN/MAX and memory clocks excluded


def test_stats_and_max_errors():
    st = bench.stats_us(np.arange(1.0, 101.0))
    assert st["calls"] == 100 and st["p50_us"] == 50.5 and st["p10_us"] < st["p50_us"] < st["p90_us"]
    # with a block-timed figure, that is the time per call; the per-call mean rides along
    sb = bench.stats_us(np.arange(1.0, 101.0), 40.0)
    assert sb["us_per_call"] == 40.0 and sb["per_call_event_mean_us"] == 50.5 and sb["p50_us"] == 50.5
    o_ref = np.zeros((1, 2, 3, 4))
    o = o_ref.copy()
    o[0, 1, 2, 3] = 0.01
    o_ref[0, 1, 2, 3] = -3.0
    lse_ref = np.array([[[0.0, -np.inf, 1.0], [2.0, 3.0, 4.0]]])
    lse = lse_ref + 1e-4
    e = bench.max_errors(o, lse, o_ref, lse_ref)
    assert abs(e["max_abs_err_o"] - 3.01) < 1e-12 and e["abs_o_ref_at_max"] == 3.0
    assert abs(e["max_abs_err_lse"] - 1e-4) < 1e-12 and e["rows_compared"] == 6


def test_host_info_names_the_cpu():
    h = bench.host_info()
    assert h["cpu_threads_available"] >= 1
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)
