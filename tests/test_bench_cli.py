"""bench.py's command line without a GPU: more than one GPU is refused with a
message, and the help text documents the modes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_help_lists_modes():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0
    for flag in ("--steps", "--warmup", "--ladder", "--op", "--copy-probe-mib", "--row", "--format",
                 "--all-workloads", "--shape-sweep"):
        assert flag in proc.stdout
