"""bench.py's command line on the host: more than one GPU is refused with a
message before anything touches a device, and the workload names resolve."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_workloads():
    r = _bench("--help")
    assert r.returncode == 0
    for name in ("llama3-8b-gqa-1m-striped-share", "causal-256k-striped-share", "causal-32k-contiguous-ring",
                 "noncausal-4k-ring"):
        assert name in r.stdout
