"""bench.py's contract on the host: more than one GPU is refused with a message before any
device work (one GPU measures this path), and the multi-GPU launcher's variables do not
change that."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, extra_env=None):
    env = dict(os.environ)
    env.update(extra_env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run(["--gpus", n])
        out = r.stdout + r.stderr
        assert "not supported" in out and "single GPU" in out, out
        assert "{" not in r.stdout, r.stdout            # no benchmark line


def test_refused_under_the_distributed_launcher_variables():
    r = _run(["--gpus", "2"], {"RANK": "0", "LOCAL_RANK": "0", "WORLD_SIZE": "2", "MASTER_ADDR": "127.0.0.1",
                               "MASTER_PORT": "29555"})
    assert "not supported" in r.stdout + r.stderr
