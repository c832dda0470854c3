"""The committed HBM-traffic records of the split kernel against the byte accounting (CPU only).

Each `profiles/traffic_split_kernel_<workload>.json` holds what FETCH_SIZE, WRITE_SIZE and the
memory-side read counter gave per launch, scaled by a device copy of known size. The checks below
tie those records to the workloads and to the traffic model (Ch. 10 "System Model of Throughput
and Latency" §4: each K/V element of an attended position is read once, whatever the group
size):
* the algorithmic bytes a record divides by are the accounting module's unique-KV bytes for that
  workload's seeded lengths;
* the measured traffic is those bytes within one percent, so no query head re-reads its KV
  head's tiles. The windowed workload is the exception: it reads whole 16-position tiles at the
  window's edges and around the sinks, a few percent of its 67 MB;
* the memory-side read counter agrees with the calibrated FETCH_SIZE.
"""
import glob
import json
import os

import pytest

from kv_cache_decode_split_amd import accounting as A
from kv_cache_decode_split_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_split_kernel_*.json")))


def _spec_of(workload: str):
    """The workload spec a record's name stands for: C<n>, then _g<γ>, _token_major or
    _w<W>_s<sinks> as the bench options that produced it."""
    parts = workload.split("_")
    over = {}
    i = 1
    while i < len(parts):
        p = parts[i]
        if p.startswith("g") and p[1:].isdigit():
            over["num_queries"] = int(p[1:])
        elif p == "token" and i + 1 < len(parts) and parts[i + 1] == "major":
            over["layout"] = "token_major"
            i += 1
        elif p.startswith("w") and p[1:].isdigit():
            over["window"] = int(p[1:])
        elif p.startswith("s") and p[1:].isdigit():
            over["num_sinks"] = int(p[1:])
        else:
            raise ValueError(f"unknown record suffix {p!r} in {workload}")
        i += 1
    return W.preset(parts[0], **over)


def test_every_long_context_workload_has_a_record():
    names = {json.load(open(p))["workload"] for p in RECORDS}
    assert {"C2", "C3", "C4", "C5"} <= names


@pytest.mark.parametrize("path", RECORDS, ids=lambda p: os.path.basename(p)[:-5])
def test_record_matches_the_accounting(path):
    rec = json.load(open(path))
    spec = _spec_of(rec["workload"])
    lens = [int(t) for t in W.workload_structure(spec)["ctx"]]
    gamma = max(spec.num_queries, 1)
    att = [A.attended_length(t, spec.window, spec.num_sinks, gamma) for t in lens]
    elem = 2 if spec.kv_dtype == "bf16" else 4
    assert rec["algorithmic_bytes_per_launch"] == A.unique_kv_read_bytes(
        att, spec.num_kv_heads, spec.head_dim, elem)


@pytest.mark.parametrize("path", RECORDS, ids=lambda p: os.path.basename(p)[:-5])
def test_measured_traffic_is_the_unique_kv_bytes(path):
    rec = json.load(open(path))
    ratio = rec["traffic_over_algorithmic"]
    bound = 1.05 if _spec_of(rec["workload"]).window else 1.01
    assert 0.995 <= ratio <= bound, ratio
    assert rec["hbm_bytes_per_launch"] == pytest.approx(ratio * rec["algorithmic_bytes_per_launch"], rel=1e-9)


@pytest.mark.parametrize("path", RECORDS, ids=lambda p: os.path.basename(p)[:-5])
def test_memory_side_reads_agree_with_the_calibrated_fetch(path):
    rec = json.load(open(path))
    assert abs(rec["dram_read_over_calibrated_fetch"] - 1.0) < 0.005
    cal = rec["calibration"]
    # The copy's own bytes fix the scales: FETCH_SIZE reads half the copied bytes on this device.
    assert cal["fetch_scale"] == pytest.approx(cal["copy_bytes"] / (cal["fetch_kib"] * 1024), rel=1e-12)
    assert cal["write_scale"] == pytest.approx(cal["copy_bytes"] / (cal["write_kib"] * 1024), rel=1e-12)
    assert rec["commands"] and all("bench.py" in c for c in rec["commands"])
