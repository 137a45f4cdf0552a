"""The benchmark's command-line contract, checked on the CPU: asked for more than one GPU it
prints one explanation on stderr, nothing on stdout, and exits with status 2 before it touches
a device (the aggregation stage and the Top-K stage alike); with no flags it runs one GPU,
20 timed steps after 3 warm-ups, on the largest workload."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.join(os.path.dirname(__file__), "..")
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("extra", [[], ["--stage", "topk"]])
@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n, extra):
    r = subprocess.run([sys.executable, BENCH, "--gpus", str(n), *extra],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr


def test_defaults():
    src = open(BENCH).read()
    want = {"--gpus": "1", "--steps": "20", "--warmup": "3", "--workload": '"large"'}
    for flag, default in want.items():
        m = re.search(r'add_argument\("' + re.escape(flag) + r'"[^)]*?default=([^,)\s]+)', src)
        assert m is not None and m.group(1) == default, flag
