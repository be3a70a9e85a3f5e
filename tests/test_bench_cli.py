"""bench.py's command line on the host: it measures one GPU only and refuses more (by flag
or by a launcher's WORLD_SIZE) with status 2 and a message, before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_bench_refuses_a_multi_rank_launch():
    env = dict(os.environ, WORLD_SIZE="4", RANK="0", LOCAL_RANK="0")
    r = _run(["--gpus", "1"], env=env)
    assert r.returncode == 2, r.stderr
    assert "WORLD_SIZE=4" in r.stderr
