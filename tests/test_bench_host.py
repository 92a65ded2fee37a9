"""Host-side logic of bench.py (CPU only): the one-GPU guard and the measured
HBM traffic it reports next to each roofline."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_every_traffic_record_matches_the_sources_it_was_measured_on():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert set(rec) == set(bench.KERNEL_SOURCES)
    for kind, r in rec.items():
        # FETCH_SIZE and WRITE_SIZE scaled by the 1 GiB copy's calibration
        assert abs(r["fetch_scale"] - 2.0) < 0.01 and abs(r["write_scale"] - 1.0) < 0.01, kind
        assert r["fetch_bytes"] > 0 and r["write_bytes"] > 0, kind
        if r["source_sha"] != bench.source_sha(kind):
            pytest.skip(f"{kind}: kernel sources changed since the counters were taken")
        assert bench.measured_traffic(kind) == r["fetch_bytes"] + r["write_bytes"], kind


def test_traffic_is_withheld_once_a_source_changes(monkeypatch):
    monkeypatch.setattr(bench, "source_sha", lambda kind: "0" * 16)
    assert all(bench.measured_traffic(kind) is None for kind in bench.KERNEL_SOURCES)


def test_traffic_within_a_few_percent_of_the_algorithmic_bytes_for_the_step():
    # the step's decode reads every cached byte once; its prefill re-reads K/V from L2 only
    dec = bench.measured_traffic("decode")
    pre = bench.measured_traffic("prefill")
    if dec is None or pre is None:
        pytest.skip("kernel sources changed since the counters were taken")
    assert 8_641_433_236 <= dec <= 1.01 * 8_641_433_236
    assert 84_410_368 <= pre <= 1.05 * 84_410_368


_SMI_SAMPLE = """GPU: 0
    POWER:
        SOCKET_POWER: 1286 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1764 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1727 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
        VCLK_0:
            CLK: 59 MHz
"""


def test_power_and_shader_clocks_are_read_from_amd_smi_text():
    watts, gfx = bench.parse_smi_metric(_SMI_SAMPLE)
    assert watts == 1286.0
    assert gfx == [1764.0, 1727.0]  # memory and video clocks are not shader clocks
    assert bench.parse_smi_metric("SOCKET_POWER: N/A\n") == (None, [])
