"""bench.py's command-line contract on the CPU: it measures one GPU only, so
a request for more (--gpus N > 1, or a WORLD_SIZE above 1 from a launcher)
ends at once with exit status 2 and a message that says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=e, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_launcher_world_size_is_refused():
    r = _bench([], env={"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
