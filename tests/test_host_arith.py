"""Host checks of the fp32 arithmetic the fast activation quantizer
(rotate_quant_fast.hip) relies on: the int8 code is the low byte of
fma(v, rb, 1.5 * 2^23) with rb = RN(1/scale) raised by two units in the
last place, which rounds every exact tie away from zero and differs from
round_half_away(v / scale) only just below a rounding boundary.  The
checker is a C program (tests/host/quotient_identities.c) built with gcc;
builds with a planted mistake must be rejected by it."""
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


def test_quantizer_identities_hold(tmp_path):
    res = _run(_build(tmp_path, "qid"))
    assert res.returncode == 0, res.stdout + res.stderr
    assert "byte identity: every |p| <= 128, 0 mismatches" in res.stdout
    assert "not away from zero" in res.stdout and ", 0 not away from zero" in res.stdout
    assert "decision random: 200000000 pairs, 0 off the definition away from a boundary" in res.stdout


@pytest.mark.parametrize("plant", ["PLANT_MAGIC_2P23", "PLANT_NO_BUMP"])
def test_checker_rejects_planted_mistake(tmp_path, plant):
    res = _run(_build(tmp_path, plant.lower(), [plant]))
    assert res.returncode != 0, res.stdout
