"""The library's profiling events: tallies of runs and K2 launches, times
that bracket the kernels, sampling of one run in N, and no events under
graph capture."""
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


def _runs(case, ex, n):
    w = case.w
    for _ in range(n):
        ex.run(case.input, case.target, case.signal, case.send, case.recv, w.core_num, w.dtype)
    torch.cuda.synchronize()
    assert ex.query_error() == a2av.OK


@pytest.mark.parametrize("chunk", [0, 1 << 16])
def test_profile_tallies_runs_and_launches(chunk):
    w = wl.workload(2)
    say("profile tally, chunk", chunk)
    case = Case(w)
    ex = exchange_for(w, chunk_limit_bytes=chunk, profile=True)
    try:
        launches = ex.launch_info(w.core_num).chunk_launches
        _runs(case, ex, 5)
        k1, k2, n, runs = ex.profile()
        assert runs == 5 and n == 5 * launches
        assert k1 > 0 and k2 > 0
        # A new tally starts after each read.
        assert ex.profile() == (0.0, 0.0, 0, 0)
    finally:
        ex.close()


@pytest.mark.parametrize("every,n,expect", [(1, 4, 4), (3, 7, 3), (4, 4, 1), (5, 11, 3)])
def test_profile_sample_records_one_run_in_every(every, n, expect):
    w = wl.workload(1)
    case = Case(w)
    ex = exchange_for(w, profile=True)
    try:
        _runs(case, ex, 2)
        ex.profile()
        ex.profile_sample(every)
        _runs(case, ex, n)
        _, _, launches, runs = ex.profile()
        assert runs == expect and launches == expect
    finally:
        ex.close()


def test_profile_sample_rejects_bad_periods_and_unprofiled_handles():
    w = wl.workload(1)
    ex = exchange_for(w, profile=True)
    plain = exchange_for(w)
    try:
        with pytest.raises(ValueError):
            ex.profile_sample(0)
        with pytest.raises(ValueError):
            plain.profile_sample(1)
        assert a2av.a2av_profile_sample(None, 1) == a2av.ERR_NULLPTR
    finally:
        ex.close()
        plain.close()


def test_no_events_are_recorded_under_graph_capture():
    w = wl.workload(1)
    case = Case(w)
    ex = exchange_for(w, profile=True)
    g = None
    try:
        _runs(case, ex, 1)
        ex.profile()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ex.run(case.input, case.target, case.signal, case.send, case.recv, w.core_num,
                   w.dtype)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK
        assert ex.profile()[3] == 0
        _runs(case, ex, 2)                 # eager runs are still recorded
        assert ex.profile()[3] == 2
    finally:
        del g
        torch.cuda.synchronize()
        ex.close()
