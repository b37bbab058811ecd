"""bench.py's command line on a host without a GPU: more than one GPU is
refused with a message before any GPU work, and the options it documents
parse (argparse's --help)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        r = run("--gpus", str(n))
        assert r.returncode != 0
        assert "one GPU" in r.stdout + r.stderr
        assert "{" not in r.stdout   # no JSON line


def test_help_lists_the_contract_options():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--no-cpu-baseline"):
        assert opt in r.stdout, opt
