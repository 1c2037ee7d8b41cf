"""The library's C ABI driven from a C program: tests/c_abi/a2av_c_driver.c
allocates the operands with hipMalloc, runs plain (FP32 and INT8, one block,
cooperative, chunked, P = 64), blocked, bias (BF16 with an FP32 bias, FP16
with an FP16 bias, chunked) and indexed exchanges twice each on a stream of
its own, and compares target, signal and recv_counts byte for byte with the C
oracle.  The driver is built with the library; it runs here as a
child process.

On ROCm, once a process has made a cooperative launch, another process's
cooperative launch on the same GPU fails until the first process exits.
The driver's runs with B > 1 therefore need a pytest process that has made
none yet: this file's name sorts before the other GPU tests, and the test is
skipped, with that reason, when it runs after one.""" 
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "a2av_c_driver")


def test_c_driver_matches_the_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        from tests.c_abi import build
        build.build()
    print("running", EXE, flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    sys.stdout.write(res.stdout)
    sys.stderr.write(res.stderr)
    if "present state" in res.stderr:
        # The platform's rule, not a fault of the library: see the module docstring.
        pytest.skip("the driver's cooperative launches were refused because this pytest "
                    "process made one before the driver ran; run this file first or alone")
    assert res.returncode == 0, f"driver exit status {res.returncode}"
    assert "all cases match the oracle" in res.stdout
