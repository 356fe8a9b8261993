"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    """Only one GPU is measured: --gpus N with N > 1 exits (status 2) before
    touching the device and says why."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 2" in res.stderr
    assert res.stdout == ""
