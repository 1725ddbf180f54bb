"""bench.py's command-line contract that needs no GPU: a request for more
than one GPU is refused with a message (the sampling path runs on one GPU;
rows shard across GPUs with no communication)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""   # no result line
