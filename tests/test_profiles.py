"""The committed rocprofv3 summaries are consistent with themselves: the
kernel-trace average of each timed kernel agrees with the HIP-event average
the benchmark measured in the same profiled run, and the byte counters were
scaled by the plain-copy calibration they record.  (Host only.)"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = os.path.join(ROOT, "profiles")
TRACES = ["mhsa_b128_lognormal_kernel_trace.md", "mhsa_bf16_b32_long_full_kernel_trace.md"]


def _trace_rows(text):
    rows = {}
    for line in text.splitlines():
        m = re.match(r"\| ([^|]+) \| `([^`]+)` \| (\d+) \| ([\d.]+) \|", line)
        if m:
            rows[m.group(1).strip()] = float(m.group(4))
    return rows


def _event_avgs(text):
    return {m.group(1): float(m.group(2))
            for m in re.finditer(r"^- (\w+): ([\d.]+) us", text, flags=re.M)}


@pytest.mark.parametrize("name", TRACES)
def test_trace_and_event_averages_agree(name):
    text = open(os.path.join(PROF, name)).read()
    rows, ev = _trace_rows(text), _event_avgs(text)
    assert "qkv_proj" in rows and "qkv_proj" in ev
    # the trace average includes the warm-up calls, the event average only the
    # timed ones; both are per call, a step's event time covering all its
    # launches (a projection's "last rows" launch, the attention's table)
    qkv = rows["qkv_proj"] + rows.get("qkv_proj (last rows)", 0.0)
    assert abs(qkv - ev["qkv_proj"]) <= 0.05 * ev["qkv_proj"]
    attn = rows["block_attn"] + rows.get("(attention work-unit table)", 0.0)
    assert abs(attn - ev["block_attn"]) <= 0.08 * ev["block_attn"]


@pytest.mark.parametrize("kernel", ["qkv_proj", "block_attn", "out_proj"])
def test_traffic_files_are_scaled_by_their_calibration(kernel):
    t = json.load(open(os.path.join(PROF, f"traffic_{kernel}.json")))
    fetch = (t["fetch_kib_per_dispatch"] + t["extra_dispatch_fetch_kib"]) * 1024 * t["fetch_scale"]
    write = (t["write_kib_per_dispatch"] + t["extra_dispatch_write_kib"]) * 1024 * t["write_scale"]
    assert abs(fetch + write - t["bytes_per_launch"]) <= 1e-6 * t["bytes_per_launch"]
    # a plain copy of 1 GiB each way reads back as 1 GiB each way after scaling
    m = re.search(r"FETCH_SIZE read ([\d.]+) KiB and WRITE_SIZE ([\d.]+) KiB", t["calibration"])
    assert m
    assert abs(float(m.group(1)) * t["fetch_scale"] - 1048576) < 1
    assert abs(float(m.group(2)) * t["write_scale"] - 1048576) < 1


@pytest.mark.parametrize("kernel", ["qkv_proj", "block_attn", "out_proj"])
def test_counter_files_are_consistent(kernel):
    """MFMA busy = busy cycles / (per-XCD cycles x 1024 SIMDs), clock =
    per-XCD cycles / duration, as bench.py --counter-summary derives them."""
    c = json.load(open(os.path.join(PROF, f"counters_{kernel}.json")))
    main = c["launches"][kernel]
    k = main["counters"]
    cycles = k["GRBM_GUI_ACTIVE"] / 8
    assert abs(main["cycles"] - cycles) <= 1e-9 * cycles
    assert abs(main["mfma_busy"] - k["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 1024)) < 1e-9
    assert 1500 < main["clock_mhz"] < 2600
    assert abs(main["clock_mhz"] - cycles / (main["avg_us"] * 1e3) * 1e3) < 0.05 * main["clock_mhz"]
    assert c["mfma_busy"] == main["mfma_busy"] and c["clock_mhz"] == main["clock_mhz"]
