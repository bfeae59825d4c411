"""bench.py's command-line contract on the host: the library has one-GPU paths only, so a
request for several GPUs (by flag or by a launcher's WORLD_SIZE) ends with a message and a
non-zero status before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_bench_refuses_several_gpus_by_flag():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_bench_refuses_several_ranks_from_launcher():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2", "RANK": "1", "LOCAL_RANK": "1"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
