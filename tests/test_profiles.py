"""The committed rocprofv3 summaries agree with one another: the kernel-trace
summary and the calibrated HBM counters name the same library build, carry the
commands that produced them, and cover every kernel of the step."""
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = os.path.join(ROOT, "profiles")
STEP = ["per_token", "swiglu", "per_block", "per_channel_T", "e2m1"]


def load():
    with open(os.path.join(PROF, "casts_deepseek_v3_shapes.md")) as f:
        md = f.read()
    with open(os.path.join(PROF, "traffic.json")) as f:
        traffic = json.load(f)
    return md, traffic


def test_summary_and_counters_name_the_same_build():
    md, traffic = load()
    m = re.search(r"Library source digest: `([0-9a-f]{64})`", md)
    assert m, "the summary states the library digest it was taken on"
    assert m.group(1) == traffic["library_digest"]


def test_commands_are_given():
    md, _ = load()
    assert "rocprofv3 --kernel-trace --stats" in md
    assert "rocprofv3 --pmc FETCH_SIZE" in md and "rocprofv3 --pmc WRITE_SIZE" in md
    assert "bench.py" in md


def test_every_step_kernel_is_covered():
    md, traffic = load()
    for k in STEP:
        assert re.search(rf"^\| {k} \| \d+ \| [\d.]+ \|", md, re.M), f"{k} missing from the trace"
        entry = traffic["kernels"][k]
        # calibrated HBM bytes within 1% of what the cast must move
        assert 0.99 < entry["bytes_per_launch"] / entry["algorithmic_bytes"] < 1.01, k
    # the calibration factors come from the copy kernel and sit near their
    # known values (FETCH_SIZE reads half the bytes fetched, WRITE_SIZE all)
    assert 0.45 < traffic["fetch_factor"] < 0.55
    assert 0.95 < traffic["write_factor"] < 1.05
