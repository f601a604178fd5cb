"""bench.py's command line, on the CPU: it measures one GPU only, so any other
GPU count (or a multi-rank launch) exits at once with a message and status 2,
before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments():
    """Stored counters are keyed by the sources' code: a comment or blank-space
    edit keeps the key, a code edit changes it."""
    import bench
    a = "int f(int x) {  // doubles\n  return 2 * x; /* plain */\n}\n"
    b = "int f(int x) {\n  // doubles its argument\n  return 2 * x;\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
