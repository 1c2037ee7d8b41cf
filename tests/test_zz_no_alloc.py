"""a2av_run_noalloc (the entry point that allocates nothing: its workspace is
the library's per-device array) against a2av_run (a handle's workspace) on
the same inputs, through the C ABI: two calls in a row, the second with a
smaller input (fewer ranks, fewer blocks, another dtype), then a device-side
failure and a valid run after it.  Target, signal, recv_counts and the
status word must match what a2av_run gives, byte for byte, and the oracle.
Also a run captured into a HIP graph and replayed, against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, exchange_for, say  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _noalloc(c: Case, core_num: int, status: torch.Tensor) -> int:
    w = c.w
    stream = torch.cuda.current_stream(DEV).cuda_stream
    return a2av.a2av_run_noalloc(c.input.data_ptr(), c.target.data_ptr(), c.signal.data_ptr(),
                                 c.send.data_ptr(), c.recv.data_ptr(), status.data_ptr(), w.P,
                                 w.in_slab, w.tgt_slab, w.S, core_num, w.dtype, stream)


def _compare(w: wl.Workload, status: torch.Tensor):
    """One a2av_run_noalloc call and one a2av_run on copies of the same operands."""
    ref = Case(w)
    ex = exchange_for(w)
    try:
        st_ref = ref.run_gpu(ex)
    finally:
        ex.close()
    c = Case(w)
    status.fill_(-99)
    assert _noalloc(c, w.core_num, status) == a2av.OK
    torch.cuda.synchronize()
    got_status = int(status.item())
    assert got_status == st_ref, (got_status, st_ref)
    np.testing.assert_array_equal(c.target.cpu().numpy(), ref.target.cpu().numpy())
    np.testing.assert_array_equal(c.signal.cpu().numpy(), ref.signal.cpu().numpy())
    np.testing.assert_array_equal(c.recv.cpu().numpy(), ref.recv.cpu().numpy())
    c.assert_matches(got_status, c.run_oracle())
    return got_status


def test_noalloc_matches_a2av_run_twice_then_error_then_valid():
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(5)
    big = wl.custom(8, wl.FP32, wl.uniform_counts(rng, 8, 1 << 15, 0.1), core_num=64, seed=51)
    small = wl.custom(5, wl.INT8, wl.uniform_counts(rng, 5, 3000, 0.2), core_num=3, seed=52)
    assert small.payload_bytes < big.payload_bytes
    say("noalloc call 1", big.P, big.payload_bytes, "call 2", small.P, small.payload_bytes)
    assert _compare(big, status) == a2av.OK
    assert _compare(small, status) == a2av.OK

    # A negative count: the status word reports INVALID_ARGS, nothing is
    # written; the next valid run reports OK again.
    C = small.counts.copy()
    C[1, 3] = -2
    bad = wl.custom(5, wl.INT8, C, core_num=3, seed=53, in_slab=small.in_slab,
                    tgt_slab=small.tgt_slab)
    say("noalloc device-side error")
    assert _compare(bad, status) == a2av.ERR_INVALID_ARGS
    assert _compare(small, status) == a2av.OK


@pytest.mark.parametrize("core_num", [64, 1])
def test_noalloc_run_captured_into_a_graph_and_replayed(core_num):
    # Code under HIP graph capture is among the callers this entry point is
    # for: a run is captured once (after an eager run, so the device's array
    # address is already known) and replayed three times, with a new payload
    # before each replay; the status word, target, signal and recv_counts
    # match the oracle after every replay.  core_num 64: a cooperative final
    # launch (B = 64); 1: a regular one.
    rng = np.random.default_rng(7 + core_num)
    w = wl.custom(8, wl.INT8, wl.uniform_counts(rng, 8, 20000, 0.2), core_num=core_num, seed=61)
    inp0 = wl.input_bytes_np(w)
    c = Case(w, input_np=inp0)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def check():
        exp = c.run_oracle()
        assert int(status.item()) == a2av.OK
        c.assert_matches(a2av.OK, exp)
        c.signal_np0 = exp[2].copy()

    assert _noalloc(c, w.core_num, status) == a2av.OK
    torch.cuda.synchronize()
    check()
    g = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(g):
            assert _noalloc(c, w.core_num, status) == a2av.OK
        torch.cuda.synchronize()
        np.testing.assert_array_equal(c.signal.cpu().numpy(), c.signal_np0)  # nothing ran
        for rep in range(3):
            say("noalloc replay", rep, "core_num", core_num)
            new = np.roll(inp0, 1 + rep)
            c.input.copy_(torch.from_numpy(new).to(DEV))
            c.input_np = new
            c.target.fill_(wl.SENTINEL)
            c.recv.fill_(-7)
            status.fill_(-99)
            g.replay()
            torch.cuda.synchronize()
            check()
    finally:
        del g
        torch.cuda.synchronize()


def test_noalloc_host_errors():
    w = wl.custom(4, wl.FP32, np.ones((4, 4), np.int32), core_num=4)
    c = Case(w)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = lambda t: t.data_ptr()  # noqa: E731
    run = lambda **o: a2av.a2av_run_noalloc(  # noqa: E731
        o.get("inp", p(c.input)), p(c.target), p(c.signal), p(c.send), p(c.recv),
        o.get("status", p(status)), o.get("P", 4), w.in_slab, w.tgt_slab, w.S,
        o.get("L", 4), o.get("dtype", wl.FP32), None)
    assert run(status=None) == a2av.ERR_NULLPTR
    assert run(inp=None) == a2av.ERR_NULLPTR
    assert run(dtype=wl.BF16) == a2av.ERR_UNSUPPORTED_DTYPE
    assert run(P=65) == a2av.ERR_INVALID_ARGS
    assert run(L=0) == a2av.ERR_INVALID_ARGS
    assert run(status=p(c.recv)) == a2av.ERR_INVALID_ARGS         # overlaps recv_counts
    torch.cuda.synchronize()
    assert (c.target.cpu().numpy() == wl.SENTINEL).all()
    assert (c.signal.cpu().numpy() == 0).all()
