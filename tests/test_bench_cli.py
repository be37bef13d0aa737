"""bench.py's command-line contract on the CPU: more than one GPU is refused with
a message (the path is measured on one GPU), and the flags the profiling
commands use parse."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_help_lists_the_modes():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0
    for flag in ("--steps", "--warmup", "--no-cpu", "--only", "--ceilings", "skewed"):
        assert flag in p.stdout
