"""bench.py's command line on the CPU: the options that cannot run exit with
status 2 and a JSON error message before touching a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "8")
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stderr.strip().splitlines()[-1])["error"]


def test_write_back_needs_the_bucket_workload():
    r = _run("--write-back", "--workload", "llama7b")
    assert r.returncode == 2
    assert "buckets" in json.loads(r.stderr.strip().splitlines()[-1])["error"]


def test_inject_every_needs_whole_steps():
    for k in ("1", "-3"):
        r = _run("--inject-every", k)
        assert r.returncode == 2
        assert "inject-every" in json.loads(r.stderr.strip().splitlines()[-1])["error"]


def test_graph_needs_device_control():
    r = _run("--graph", "--host-control")
    assert r.returncode == 2
    assert "host-control" in json.loads(r.stderr.strip().splitlines()[-1])["error"]
