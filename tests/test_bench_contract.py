"""bench.py's command-line contract, checked without a GPU: more than one GPU
is refused with a message before any device work, and the argument parser
knows every workload the bench line can be taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_workloads_are_known():
    sys.path.insert(0, ROOT)
    import bench
    import synth
    for wl in bench.PREFILL + bench.DECODE + bench.SCAN:
        assert wl in synth.WORKLOADS, wl
