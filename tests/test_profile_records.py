"""The committed rocprofv3 records under profiles/ describe the kernels as they
stand: every traffic record carries the source hash of the kernel headers it
was measured on, and bench.py uses a record only while that hash matches, so
a stale record would silently drop the `traffic` figure from the bench line.
Also: each record names the summary it came from, and that summary exists and
quotes the same hash."""
import glob
import json
import os

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))


def _sources(rec):
    return bench.CHAIN_SOURCES if rec["workload"] in W.CHAIN_WORKLOADS else None


def test_there_are_records():
    assert RECORDS


@pytest.mark.parametrize("path", RECORDS, ids=os.path.basename)
def test_record_matches_current_kernel_sources(path):
    with open(path) as f:
        rec = json.load(f)
    assert rec["source_hash"] == bench.kernel_source_hash(_sources(rec)), (
        f"{os.path.basename(path)} was measured on other kernel sources: re-take the "
        f"FETCH_SIZE / WRITE_SIZE counters")
    # the stored figures are rounded (0.1 KiB, scale to 2 decimals)
    approx = rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]
    assert abs(rec["bytes_per_launch"] - approx) <= 1e-3 * approx
    summary = os.path.join(ROOT, "profiles", rec["from"])
    assert os.path.exists(summary)
    with open(summary) as f:
        assert rec["source_hash"] in f.read()
