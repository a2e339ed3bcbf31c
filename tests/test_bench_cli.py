"""bench.py's command-line contract on the CPU: it measures one rank's layer on one GPU, so
a request for several GPUs (flag or launcher environment) exits with status 2 and says so,
before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env, cwd=ROOT)


def test_several_gpus_flag_is_refused():
    r = run_bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_several_ranks_from_the_launcher_are_refused():
    r = run_bench(["--steps", "1"], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "WORLD_SIZE=2" in r.stderr
