"""bench.py's command line contract on the host: more than one GPU is refused with a message, before
any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)


def test_density_needs_a_fraction_and_a_topk_workload():
    for extra in (["--density", "1.5"], ["--workload", "chunked_window", "--density", "0.5"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0"] + extra,
                           capture_output=True, text=True, timeout=300, cwd=ROOT)
        assert r.returncode == 2, (extra, r.stderr[-300:])
        assert "--density needs" in r.stderr
