"""bench.py's command-line contract, checked on the CPU: one GPU only (any
other count, or a WORLD_SIZE above 1, exits 2 with a message before anything
touches a device), and the profile modes the committed rocprofv3 summaries
name all exist."""
import os
import pathlib
import re
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=e, cwd=ROOT)


@pytest.mark.parametrize("gpus", ["2", "8", "0"])
def test_other_gpu_counts_are_refused(gpus):
    r = _run("--gpus", gpus)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


def test_world_size_above_one_is_refused():
    r = _run(env={"WORLD_SIZE": "2"})
    assert r.returncode == 2


def test_profile_modes_named_by_the_summaries_exist():
    import bench
    src = (ROOT / "bench.py").read_text()
    choices = re.search(r'"--profile", choices=\[([^\]]*)\]', src, re.S).group(1)
    modes = set(re.findall(r'"(\w+)"', choices))
    named = set()
    for p in (ROOT / "profiles").iterdir():
        named |= set(re.findall(r"bench\.py --profile (\w+)", p.read_text()))
    assert named and named <= modes, named - modes
    assert bench.PROFILE_WARM_GEMM > 0 and bench.PROFILE_WARM_MFMA > 0
