"""bench.py's host-side contract, without a GPU: the one-GPU guard, the CPU-baseline
record (the oracle timed on a bounded sample) and the counter records it reads from
profiles/."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from layer_streamed_qlora_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_record_on_the_toy_stack():
    rec = bench.cpu_baseline(synth.WORKLOADS["toy"])
    json.dumps(rec)                                   # serialisable as part of the JSON line
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "batch 1 x seq 512" in rec["sample"]
    more = rec["more"]
    assert more["host"]["logical_cpus"] >= 1
    assert more["one_thread"]["value"] > 0
    assert more["toy_step"]["seconds"] > 0 and more["toy_step"]["seconds_one_thread"] > 0
    assert more["packer"]["MB_per_s"] > 0


@pytest.mark.parametrize("name", ["llama8b_gemm_traffic.md", "llama8b_gemm_mfma_counters.md"])
def test_counter_records_are_readable(name):
    """A record is returned only while its kernel source is unchanged; either way the
    file holds one machine-readable line naming an existing source."""
    lines = [l for l in open(os.path.join(ROOT, "profiles", name)).read().splitlines()
             if l.startswith("machine-readable: ")]
    assert len(lines) == 1
    raw = json.loads(lines[0][len("machine-readable: "):])
    assert os.path.exists(os.path.join(ROOT, raw["kernel_source"]))
    rec = bench.profile_record(name)
    assert rec is None or rec == raw
