"""The oracle's pins catch plausible mistakes: every mutant of
tests/oracle_mutants.py (one planted mistake in a copy of
oracle/a2av_oracle.c, built with gcc here on the CPU) must fail at least one
pin of tests/test_oracle_pins.py or tests/test_signal_model.py, run against
it in a process of its own; the unmutated copy must pass them all."""
import os
import subprocess
import sys

import pytest

from tests import oracle_mutants as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_pins(lib):
    return subprocess.run([sys.executable, "-m", "tests.oracle_mutants", lib], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_unmutated_copy_passes_every_pin(tmp_path):
    lib = str(tmp_path / "liba2av_oracle_copy.so")
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-w", "-shared", "-fPIC", "-o", lib,
                           om.SRC])
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "survived" in r.stdout


@pytest.mark.parametrize("name", [m[0] for m in om.MUTANTS])
def test_mutant_is_caught(name, tmp_path):
    lib = om.build(name, str(tmp_path))
    r = _run_pins(lib)
    assert r.returncode != 0, f"no pin notices the mutant {name}"
    assert "survived" not in r.stdout
