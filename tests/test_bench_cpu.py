"""Host-side checks of bench.py: its multi-GPU refusal and the counter-traffic lookup."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_traffic_lookup():
    # the committed summary belongs to the decode workload and its listed sources
    assert bench.counter_traffic("no_such_workload", "sparse_token") is None
    assert bench.counter_traffic("decode_7b_32k", "no_such_stage") is None
    path = os.path.join(ROOT, "profiles", "decode_7b_32k_hbm_counters.md")
    for stage in ("sparse_token", "full_attn"):
        t = bench.counter_traffic("decode_7b_32k", stage)
        if t is not None:
            text = open(path).read()
            meta = json.loads(text.split("```json\n")[1].split("\n```")[0])
            assert t == meta["traffic_bytes_per_launch"][stage]
            # traffic can only exceed the algorithmic bytes (re-reads), never undercut them much
            assert t >= 0.99 * meta["algorithmic_bytes_per_launch"][stage]
