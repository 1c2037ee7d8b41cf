"""The exchanges with a host copy of the counts (a2av_run_host_counts and the
blocked, bias and indexed *_host_counts entry points).  Count errors come back
from the call itself, before anything is enqueued, and the chunk plan follows
the payload (ceil(T / limit) launches) instead of the geometry bound.  Results
against the oracle, byte for byte."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, exchange_for, say, upload  # noqa: E402
from tests.test_gpu_random import _case  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run_hc(w, host_counts=None, runs=1, **kw):
    """Run with host counts on a profiled handle; (case, launches per run, status)."""
    c = Case(w)
    ex = exchange_for(w, profile=True, **kw)
    try:
        hc = np.ascontiguousarray(w.counts if host_counts is None else host_counts, np.int32)
        for _ in range(runs):
            ex.run(c.input, c.target, c.signal, c.send, c.recv, w.core_num, w.dtype,
                   host_counts=hc)
        torch.cuda.synchronize()
        st = ex.query_error()
        _, _, launches, n = ex.profile()
        exp = None
        for _ in range(runs):
            exp = c.run_oracle()
            c.signal_np0 = exp[2].copy()
        c.assert_matches(st, exp)
        return c, launches // max(n, 1), st
    finally:
        ex.close()


@pytest.mark.parametrize("scale", [64, 1])
def test_c4_shape_one_launch(scale):
    # c4's slabs bound the payload at 2 GiB (two launches by geometry); its
    # payload is about 0.8 GiB, so the host counts plan one launch.
    w = wl.workload(4, scale=scale)
    say(w.name, "scale", scale, "payload", w.payload_bytes)
    c, launches, st = _run_hc(w)
    assert st == a2av.OK and launches == 1


@pytest.mark.parametrize("limit", [1 << 20, 65536, 4096])
def test_small_limits_follow_the_payload(limit):
    rng = np.random.default_rng(limit)
    P = 8
    C = rng.integers(0, 5000, size=(P, P)).astype(np.int32)
    for dtype in (wl.FP32, wl.INT8):
        w = wl.custom(P, dtype, C, core_num=16, seed=3)
        w.in_slab += 4096
        w.tgt_slab += 4096
        T = w.payload_bytes
        c, launches, st = _run_hc(w, runs=2, chunk_limit_bytes=limit)
        say("limit", limit, "dtype", dtype, "payload", T, "launches", launches)
        assert st == a2av.OK and launches == max(1, -(-T // limit))


def test_p64_large_slabs_small_payload():
    # 64 ranks with 64 MiB slabs: 64 launches would cover the geometry bound
    # at 64 MiB per launch; the payload needs one.
    P = 64
    rng = np.random.default_rng(9)
    C = rng.integers(0, 100, size=(P, P)).astype(np.int32)
    w = wl.custom(P, wl.INT8, C, core_num=128, in_slab=64 << 20, tgt_slab=64 << 20, seed=4)
    c, launches, st = _run_hc(w, chunk_limit_bytes=64 << 20)
    assert st == a2av.OK and launches == 1


@pytest.mark.parametrize("kind", ["negative", "over_capacity"])
def test_count_errors_are_returned_by_the_call(kind):
    P = 4
    C = np.full((P, P), 16, np.int32)
    if kind == "negative":
        C[2, 1] = -1
    else:
        C[0, 3] += 1
    w = wl.custom(P, wl.FP32, C, core_num=8, in_slab=64 * 4, tgt_slab=64 * 4)
    c = Case(w)
    ex = exchange_for(w)
    try:
        want = "INVALID_ARGS" if kind == "negative" else "OVER_CAPACITY"
        with pytest.raises(ValueError, match=want):
            ex.run(c.input, c.target, c.signal, c.send, c.recv, 8, wl.FP32, host_counts=C)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK           # nothing was enqueued
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
        assert (c.recv.cpu().numpy() == -7).all()
    finally:
        ex.close()


def test_device_counts_decide_when_the_host_copy_differs():
    # Host copy all zeros: one launch is planned at a 4 KiB limit, while the
    # device counts move ~60 KiB.  The device refuses the run
    # (OVER_CAPACITY, latched) and writes nothing.
    P = 4
    rng = np.random.default_rng(3)
    C = rng.integers(100, 1000, size=(P, P)).astype(np.int32)
    w = wl.custom(P, wl.FP32, C, core_num=8, seed=6)
    w.in_slab += 64
    w.tgt_slab += 64
    c = Case(w)
    ex = exchange_for(w, chunk_limit_bytes=4096)
    try:
        ex.run(c.input, c.target, c.signal, c.send, c.recv, 8, wl.FP32,
               host_counts=np.zeros((P, P), np.int32))
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.ERR_OVER_CAPACITY
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
        assert (c.recv.cpu().numpy() == -7).all()
        # A host copy whose plan covers the device payload: the device counts
        # are the ones exchanged.
        hc = C.copy()
        hc[0, 0] -= 1
        T = int(C.sum()) * 4
        assert -(-T // 4096) == -(-(T - 4) // 4096)      # the same plan
        ex.run(c.input, c.target, c.signal, c.send, c.recv, 8, wl.FP32, host_counts=hc)
        torch.cuda.synchronize()
        c.assert_matches(ex.query_error(), c.run_oracle())
    finally:
        ex.close()


def _kind_kwargs(c):
    """The GPU and oracle arguments of one random case's exchange."""
    w, kind = c["w"], c["kind"]
    if kind == "blocked":
        return dict(nblk=c["nblk"]), dict(nblk=c["nblk"])
    if kind == "bias":
        b = c["bias"]
        bt = torch.from_numpy(b.view(np.float16) if w.dtype == wl.FP16 else b).to(DEV)
        return (dict(nblk=c["nblk"], bias=bt, hidden=c["hidden"]),
                dict(nblk=c["nblk"], bias=b, hidden=c["hidden"]))
    return (dict(index=upload(c["index"]), row_elems=c["R"]),
            dict(index=c["index"], row_elems=c["R"]))


# Seeds of the random mixtures whose exchange is blocked, bias or indexed
# (seed % 4 = 1, 2, 3), at every chunk limit they draw.
@pytest.mark.parametrize("seed", [s for s in range(60) if s % 4 != 0])
def test_every_exchange_with_host_counts(seed):
    c = _case(seed)
    w, kind = c["w"], c["kind"]
    T = w.payload_bytes
    limit = c["chunk"] or (1 << 30)
    say(seed, kind, "P", w.P, "dtype", w.dtype, "payload", T, "limit", limit)
    inp = wl.input16_np(w) if kind == "bias" else wl.input_bytes_np(w)
    case = Case(w, input_np=inp)
    ex = exchange_for(w, wg_per_block=c["G"], chunk_limit_bytes=c["chunk"], profile=True)
    try:
        gkw, okw = _kind_kwargs(c)
        st = case.run_gpu(ex, host_counts=np.ascontiguousarray(w.counts, np.int32), **gkw)
        _, _, launches, runs = ex.profile()
        case.assert_matches(st, case.run_oracle(**okw))
        assert st == a2av.OK and launches == runs * max(1, -(-T // limit))
    finally:
        ex.close()


@pytest.mark.parametrize("kind", ["blocked", "bias", "indexed"])
@pytest.mark.parametrize("what", ["negative", "not_whole", "over_capacity"])
def test_count_errors_of_every_exchange_are_returned_by_the_call(kind, what):
    seed = {"blocked": 1, "bias": 2, "indexed": 3}[kind] + 4 * 3
    c = _case(seed)
    w = c["w"]
    unit = {"blocked": c["nblk"], "bias": c["nblk"] * c["hidden"], "indexed": c["R"]}[kind]
    if what == "not_whole" and unit == 1:
        pytest.skip("every count is whole at a unit of one")
    hc = np.ascontiguousarray(w.counts, np.int32).copy()
    if what == "negative":
        hc[0, 0] = -unit
    elif what == "not_whole":
        hc[0, 0] += 1
    else:
        hc[0, 0] += (w.tgt_slab // wl.ELEM_SIZE[w.dtype] // unit + 1) * unit   # column 0 over
    case = Case(w, input_np=wl.input16_np(w) if kind == "bias" else wl.input_bytes_np(w))
    ex = exchange_for(w, wg_per_block=c["G"], chunk_limit_bytes=c["chunk"])
    try:
        gkw, _ = _kind_kwargs(c)
        want = "OVER_CAPACITY" if what == "over_capacity" else "INVALID_ARGS"
        with pytest.raises(ValueError, match=want):
            case.run_gpu(ex, host_counts=hc, **gkw)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK           # nothing was enqueued
        assert (case.target.cpu().numpy() == wl.SENTINEL).all()
        np.testing.assert_array_equal(case.signal.cpu().numpy(), case.signal_np0)
        assert (case.recv.cpu().numpy() == -7).all()
    finally:
        ex.close()
