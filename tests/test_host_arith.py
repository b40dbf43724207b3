"""Host checks of the fp32 arithmetic identities that the fast activation
quantizer (rotate_quant_fast.hip) relies on: Markstein's corrected quotient
equals IEEE division over the scales the kernel admits, and
trunc(q + copysign(0.49999997, q)) rounds half away from zero.  The checker
is a C program (tests/host/quotient_identities.c) built with gcc; two builds
with a planted mistake must be rejected by it."""
import pathlib
import shutil
import subprocess

import pytest

SRC = pathlib.Path(__file__).parent / "host" / "quotient_identities.c"
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _build(tmp_path, name, defines=()):
    exe = tmp_path / name
    subprocess.run(["gcc", *CFLAGS, *[f"-D{d}" for d in defines], "-o", str(exe), str(SRC), "-lm"],
                   check=True, capture_output=True, text=True)
    return exe


def _run(exe):
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)


def test_quotient_identities_hold(tmp_path):
    res = _run(_build(tmp_path, "qid"))
    assert res.returncode == 0, res.stdout + res.stderr
    assert "markstein random: 200000000 pairs, 0 mismatches" in res.stdout


@pytest.mark.parametrize("plant", ["PLANT_PLAIN_HALF", "PLANT_NO_CORRECTION"])
def test_checker_rejects_planted_mistake(tmp_path, plant):
    res = _run(_build(tmp_path, plant.lower(), [plant]))
    assert res.returncode != 0, res.stdout
