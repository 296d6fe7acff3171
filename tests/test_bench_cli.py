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


def test_kernel_source_digest_ignores_comments_only():
    """The HBM-traffic record is tied to the kernel's code: a comment or
    whitespace edit keeps the digest's input, a code edit changes it."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, bench.KERNEL_SOURCES[0]), encoding="utf-8") as f:
        text = f.read()
    code = bench.source_code(text)
    assert "//" not in code and "/*" not in code
    edited = "// a new header line\n/* and a block\n   comment */\n" + text.replace("\n", "\n    ", 3)
    assert bench.source_code(edited) == code
    assert bench.source_code(text.replace("kSBK = 32", "kSBK = 16", 1)) != code
    assert len(bench.source_digest()) == 16
