"""Host-side checks of the benchmark and its committed measurement records
(no GPU): the machine-readable record of every profile summary carries the
fields the benchmark reads, and a run asked for more than one GPU exits with
its message before touching a device."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WORKLOADS = ["tiny_fp32", "vitb_fc1", "vitl_fc1", "vitl_fc2", "monarch", "lm_blast", "lm_blast_diag"]


@pytest.mark.parametrize("w", WORKLOADS)
def test_profile_records_parse(w):
    path = os.path.join(ROOT, "profiles", f"forward_{w}.md")
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    assert m, path
    rec = json.loads(m.group(1))
    assert rec["workload"] == w and re.fullmatch(r"[0-9a-f]{16}", rec["kernel_source_hash"])
    out = rec["fused_output"]
    for key in ("kernel", "avg_us", "traffic_bytes", "algorithmic_bytes", "algorithmic_flop", "mfma_busy_frac"):
        assert key in out, (w, key)
    assert out["avg_us"] > 0 and out["traffic_bytes"] > 0 and 0 < out["mfma_busy_frac"] < 1
    assert 0.4 < rec["fetch_factor"] < 1.1 and 0.4 < rec["write_factor"] < 1.1
    # the commands that made the summary run committed files only
    assert "rocprofv3 --kernel-trace --stats" in text and "_work" not in text


def test_more_than_one_gpu_exits_with_its_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and not p.stdout.strip()
