"""bench.py's command line on the host: one GPU only, and a clear refusal otherwise."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU only" in res.stdout + res.stderr


def test_committed_profiles_name_one_kernel_source_hash():
    """Every committed counter summary carries the kernel-source hash it was taken on, and they
    agree with each other (bench.py reports counter traffic only while that hash is current)."""
    import json
    prof = os.path.join(ROOT, "profiles")
    shas = {json.load(open(os.path.join(prof, f)))["kernel_sha"]
            for f in os.listdir(prof) if f.endswith(".json")}
    assert len(shas) == 1
