"""bench.py's command-line contract on the host (no GPU needed): more than one GPU is refused
with a message and exit status 2, as are --direct-p without MXFP4, --kv16 without NVFP4 or with
--backward, an unknown sweep format and an N that is not a multiple of 256; the help text lists
the options."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    r = run(env=dict(os.environ, WORLD_SIZE="4"))
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("args", [["--fmt", "nvfp4", "--direct-p"], ["--fmt", "mx4_pv8", "--direct-p"]])
def test_direct_p_needs_mxfp4(args):
    r = run(*args)
    assert r.returncode == 2 and "--direct-p needs --fmt mxfp4" in r.stderr


@pytest.mark.parametrize("args", [["--fmt", "mxfp4", "--kv16"], ["--kv16", "--backward"]])
def test_kv16_needs_the_nvfp4_forward(args):
    r = run(*args)
    assert r.returncode == 2 and "--kv16 needs --fmt nvfp4" in r.stderr


def test_unknown_sweep_format_is_refused():
    r = run("--sweep", os.devnull, "--sweep-formats", "nvfp4,fp8")
    assert r.returncode == 2 and "unknown sweep formats" in r.stderr


def test_sequence_length_must_be_a_multiple_of_256():
    r = run("--seq-len", "1000")
    assert r.returncode == 2 and "multiple of 256" in r.stderr


def test_help_lists_the_options():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--causal", "--fmt", "--direct-p", "--seq-len", "--workload",
                "--sweep", "--sweep-formats", "--backward", "--kv16"):
        assert opt in r.stdout
