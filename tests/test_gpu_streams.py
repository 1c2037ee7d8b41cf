"""Two handles on two streams at once: each handle owns its workspace, so
exchanges enqueued alternately on two torch streams (no ordering between
them) must each match the oracle.  B = 1 on both (regular launches, no
cooperative residency needed); B > 1 on both, so that the two runs' final
launches are cooperative launches enqueued while the other stream's work is
in flight; and B > 1 beside B = 1.  Several runs each, different shapes and
dtypes; the signal of each counts its own runs, and every run must succeed
(no TIMEOUT from a barrier that could not gather its blocks)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import Case, exchange_for, say  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _workload(P, dtype, hi, seed, core_num=1):
    rng = np.random.default_rng(seed)
    C = wl.uniform_counts(rng, P, hi, 0.2)
    return wl.custom(P, dtype, C, core_num=core_num, seed=seed)


# (core_num of the first handle, of the second): B = 1 and 1; B = 8 and 64
# (both cooperative); B = 64 and 1 (cooperative beside a regular launch).
@pytest.mark.parametrize("L1,L2", [(1, 1), (8, 64), (64, 1)])
@pytest.mark.parametrize("runs", [1, 4])
def test_two_handles_on_two_streams(runs, L1, L2):
    w1 = _workload(8, wl.FP32, 1 << 16, 21, core_num=L1)      # ~10 MiB, 4-byte ragged
    w2 = _workload(4 if L2 > 1 else 5, wl.INT8, 1 << 20, 22, core_num=L2)  # ~8-10 MiB, odd phases
    say("streams", runs, "core_num", L1, L2, "payload", w1.payload_bytes, w2.payload_bytes,
        "blocks", a2av.a2av_blocks(w1.P, L1), a2av.a2av_blocks(w2.P, L2))
    c1, c2 = Case(w1), Case(w2)
    # A short barrier bound: if the two launches could not gather their
    # blocks, the runs end with TIMEOUT well within the test's time limit.
    e1, e2 = exchange_for(w1, spin_limit=1 << 18), exchange_for(w2, spin_limit=1 << 18)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    try:
        torch.cuda.synchronize()
        for _ in range(runs):
            with torch.cuda.stream(s1):
                e1.run(c1.input, c1.target, c1.signal, c1.send, c1.recv, w1.core_num, w1.dtype)
            with torch.cuda.stream(s2):
                e2.run(c2.input, c2.target, c2.signal, c2.send, c2.recv, w2.core_num, w2.dtype)
        torch.cuda.synchronize()
        for c, e in ((c1, e1), (c2, e2)):
            st = e.query_error()
            exp = None
            for _ in range(runs):
                exp = c.run_oracle()
                c.signal_np0 = exp[2].copy()
            c.assert_matches(st, exp)
    finally:
        torch.cuda.synchronize()
        e1.close()
        e2.close()
