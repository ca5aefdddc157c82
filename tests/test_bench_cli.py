"""bench.py's command line, checked without a GPU: it runs on exactly one GPU
and says so (one JSON line, exit status 2) when asked for more, before it
touches a device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          timeout=120, env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2, r.stderr
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])
