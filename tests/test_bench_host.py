"""Host-side pieces of bench.py (no GPU): the parsing of the power readings
and the stored HBM-counter lookup."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_socket_power_reading_from_amd_smi_json():
    # amd-smi metric -p --json: a list of per-GPU records, the reading as {value, unit}.
    j = [{"gpu": 0, "power": {"socket_power": {"value": 1401, "unit": "W"}, "gfx_voltage": "N/A",
                              "power_management": "N/A"}}]
    vals = [bench._watts(v) for v in bench._json_find(j, lambda k: k == "socket_power")]
    assert vals == [1401.0]


def test_power_cap_from_rocm_smi_json():
    j = {"card0": {"Max Graphics Package Power (W)": "1400.0"}}
    caps = [bench._watts(v) for v in bench._json_find(j, lambda k: "max" in k and "power" in k)]
    assert caps == [1400.0]


def test_unreadable_power_values_are_skipped():
    assert bench._watts("N/A") is None
    assert bench._watts({"value": "N/A", "unit": "W"}) is None
    assert bench._watts(None) is None


def test_stored_traffic_only_for_matching_sources_and_workload():
    # The committed summary names the kernel sources' hash; bench.py reports
    # its bytes only for that hash and the workload it was taken on.
    path = os.path.join(ROOT, bench.COUNTERS_PROFILE)
    text = open(path).read()
    blob = json.loads(text[text.index("```json") + 7:text.index("```", text.index("```json") + 7)])
    got = bench.stored_traffic(blob["workload"])
    if blob["sources"] == bench.kernel_sources_hash():
        expect = round(blob["fetch_kib"] * 1024 * blob["fetch_scale"] + blob["write_kib"] * 1024 * blob["write_scale"])
        assert got == expect
    else:
        assert got is None
    assert bench.stored_traffic("another_workload") is None
