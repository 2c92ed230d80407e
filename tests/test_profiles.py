"""The committed profile summaries (host only): every summary names the
command that produced it, and the HBM-traffic record matches the current
sources of the kernels it measured, so that bench.py reports measured
traffic rather than null."""
import glob
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_summary_gives_its_command():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))
    assert files
    for f in files:
        text = open(f).read()
        assert "command" in text and "rocprofv3" in text, f


def test_traffic_record_matches_the_sources():
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic_shared_expert_decode.json")))
    mlp = bench.measured_traffic("mlp_forward")
    assert isinstance(mlp, dict) and set(mlp) == {"1", "8", "32", "64"}, "re-take the counters: sources changed"
    for m, b in mlp.items():
        assert b == int(rec["mlp_forward"]["bytes_per_launch"][m])
    gather = bench.measured_traffic("reassemble_into_slot")
    assert isinstance(gather, int) and abs(gather - 528_482_304) < 528_482_304 * 0.01
