"""Host-side logic of bench.py (no GPU): the one-GPU guard and the argument
checks that run before any GPU work."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
    assert bench.main(["--gpus", "1", "--steps", "0"]) == 2

