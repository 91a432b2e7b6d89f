"""bench.py's command line on the CPU: more than one GPU is refused with a
message (this build measures one GPU), and the help lists every secondary
leg that the full run launches."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_help_lists_every_secondary_leg():
    sys.path.insert(0, ROOT)
    import bench
    p = _run("--help")
    assert p.returncode == 0
    for leg in bench.SECONDARY_LEGS:
        assert leg in p.stdout
