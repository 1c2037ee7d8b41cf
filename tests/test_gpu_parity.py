"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bit-exact comparison (as bytes) of the whole target allocation (received
prefixes and untouched tails), the signal and recv_counts, plus the status.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, check_case, exchange_for, say, upload  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("k", [1, 2])
def test_small_workloads_full_size(k):
    w = wl.workload(k)
    say("workload", w.name)
    check_case(w)


@pytest.mark.parametrize("k,scale", [(3, 64), (4, 256), (5, 1024), (3, 8), (4, 16)])
def test_large_workloads_scaled(k, scale):
    w = wl.workload(k, scale=scale)
    say("workload", w.name, "scale", scale, "payload", w.payload_bytes)
    check_case(w)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_repeated_runs_raise_signal_each_time(k):
    w = wl.workload(k, scale=64 if k >= 3 else 1)
    check_case(w, runs=3)


# ------------------------------------------------------------------ sweeps

def _sweep_Ls(P):
    return sorted({L for L in [1, P - 1, P, P + 1, 2 * P - 1, 10, 256] if L >= 1})


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 32, 64])
@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_sweep_P_and_core_num(P, dtype):
    rng = np.random.default_rng(1000 * P + dtype)
    hi = 3000 if P <= 8 else 300
    C = rng.integers(0, hi + 1, size=(P, P)).astype(np.int32)
    C[rng.random((P, P)) < 0.15] = 0
    for L in _sweep_Ls(P):
        B = oracle.blocks(P, L)
        w = wl.custom(P, dtype, C, core_num=L, S=max(B, 1) + 3, seed=L)
        w.in_slab += 48          # ragged tails past every row / column
        w.tgt_slab += 36
        say("P", P, "dtype", dtype, "L", L, "B", B)
        check_case(w)


def test_int8_every_phase_and_ragged_rows():
    # Counts that put source and destination at every offset mod 16, with
    # bodies from under one word to several 64-word rows.
    rng = np.random.default_rng(77)
    P = 6
    for trial in range(6):
        C = rng.integers(0, 40000, size=(P, P)).astype(np.int32)
        C += rng.integers(0, 16, size=(P, P)).astype(np.int32)
        if trial == 0:
            C[:] = rng.integers(0, 40, size=(P, P))
        w = wl.custom(P, wl.INT8, C, core_num=P * 3, seed=trial)
        w.in_slab += 5
        w.tgt_slab += 11
        check_case(w)


@pytest.mark.parametrize("in_off,tgt_off", [(1, 0), (0, 3), (7, 13), (4, 8), (12, 4)])
def test_unaligned_operand_addresses(in_off, tgt_off):
    rng = np.random.default_rng(in_off * 31 + tgt_off)
    P = 4
    for dtype in (wl.INT8, wl.FP32):
        C = rng.integers(0, 9000, size=(P, P)).astype(np.int32)
        w = wl.custom(P, dtype, C, core_num=8, seed=in_off)
        c = Case(w, in_offset=in_off, tgt_offset=tgt_off)
        ex = exchange_for(w)
        try:
            c.assert_matches(c.run_gpu(ex), c.run_oracle())
        finally:
            ex.close()


@pytest.mark.parametrize("G", [1, 2, 3, 7])
def test_workgroups_per_block_invariance(G):
    # core_num 32 on P=32 admits 32 blocks, leaving room for several
    # workgroups per block.
    w = wl.workload(4, scale=64)
    w.core_num = 32
    c = check_case(w, wg_per_block=G)
    assert (c.signal.cpu().numpy()[:, :32] == 1).all()


@pytest.mark.parametrize("limit", [1 << 20, 65536, 4096, 1000, 16])
def test_chunk_limit_invariance(limit):
    rng = np.random.default_rng(limit)
    P = 8
    C = rng.integers(0, 5000, size=(P, P)).astype(np.int32)
    for dtype in (wl.FP32, wl.INT8):
        w = wl.custom(P, dtype, C, core_num=16, seed=3)
        say("chunk limit", limit, "dtype", dtype)
        check_case(w, chunk_limit_bytes=limit)


# ------------------------------------------------------------------ count categories

def _category(name, P=4, dtype=wl.FP32):
    e = wl.ELEM_SIZE[dtype]
    slab = 64 * e
    if name == "zeros":
        C = np.zeros((P, P), np.int32)
    elif name == "ones":
        C = np.ones((P, P), np.int32)
    elif name == "capacity":
        C = np.full((P, P), 64 // P, np.int32)        # every row and column exactly full
    elif name == "over_capacity":
        C = np.full((P, P), 64 // P, np.int32)
        C[1, P - 1] += 1
    elif name == "negative":
        C = np.ones((P, P), np.int32)
        C[P - 1, 0] = -3
    return wl.custom(P, dtype, C, core_num=P, in_slab=slab, tgt_slab=slab, seed=5)


@pytest.mark.parametrize("name", ["zeros", "ones", "capacity", "over_capacity", "negative"])
@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
@pytest.mark.parametrize("P", [2, 4])
def test_count_categories(name, dtype, P):
    w = _category(name, P, dtype)
    c = check_case(w)
    if name in ("over_capacity", "negative"):
        # Nothing written: sentinel target, untouched signal and recv_counts.
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
        assert (c.recv.cpu().numpy() == -7).all()


def test_unequal_signal_is_rejected_and_nothing_written():
    P = 4
    w = wl.custom(P, wl.INT8, np.ones((P, P), np.int32), core_num=4, S=6)
    sig = np.zeros((P, 6), np.int32)
    sig[2, 3] = 1
    c = Case(w, signal_np=sig)
    ex = exchange_for(w)
    try:
        st = c.run_gpu(ex)
        c.assert_matches(st, c.run_oracle())
        assert st == a2av.ERR_INVALID_ARGS
        # The latched error was cleared by the query; a valid run is clean.
        sig[2, 3] = 0
        c2 = Case(w, signal_np=sig)
        c2.assert_matches(c2.run_gpu(ex), c2.run_oracle())
    finally:
        ex.close()


def test_error_then_valid_run_reports_first_error_once():
    P = 4
    good = wl.custom(P, wl.FP32, np.ones((P, P), np.int32), core_num=4)
    C = np.ones((P, P), np.int32)
    C[0, 0] = -1
    bad = wl.custom(P, wl.FP32, C, core_num=4, in_slab=good.in_slab, tgt_slab=good.tgt_slab)
    ex = exchange_for(good)
    try:
        cb, cg = Case(bad), Case(good)
        cb.run_gpu(ex, sync=False)
        cg.run_gpu(ex, sync=False)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.ERR_INVALID_ARGS
        assert ex.query_error() == a2av.OK
        cg.assert_matches(a2av.OK, cg.run_oracle())
    finally:
        ex.close()


def test_run_with_check_raises_on_device_side_errors():
    # Exchange.run(check=True) waits for the run and raises on the latched
    # device-side status: a negative count (INVALID_ARGS) and an over-full
    # column (OVER_CAPACITY) raise ValueError with nothing written; a valid
    # run returns normally and matches the oracle.
    P = 4
    good = wl.custom(P, wl.FP32, np.full((P, P), 2, np.int32), core_num=8)
    ex = exchange_for(good)
    try:
        C = good.counts.copy()
        C[1, 2] = -3
        bad = wl.custom(P, wl.FP32, C, core_num=8, in_slab=good.in_slab, tgt_slab=good.tgt_slab)
        cb = Case(bad)
        with pytest.raises(ValueError, match="INVALID_ARGS"):
            ex.run(cb.input, cb.target, cb.signal, cb.send, cb.recv, 8, wl.FP32, check=True)
        C2 = good.counts.copy()
        C2[3, 0] += 1                                   # column 0 past the target slab
        over = wl.custom(P, wl.FP32, C2, core_num=8, in_slab=good.in_slab + 16,
                         tgt_slab=good.tgt_slab)
        assert int(C2[:, 0].sum()) * 4 > good.tgt_slab
        co = Case(over)
        ex2 = exchange_for(over)
        try:
            with pytest.raises(ValueError, match="OVER_CAPACITY"):
                ex2.run(co.input, co.target, co.signal, co.send, co.recv, 8, wl.FP32, check=True)
        finally:
            ex2.close()
        for c in (cb, co):
            torch.cuda.synchronize()
            assert (c.target.cpu().numpy() == wl.SENTINEL).all()
            assert (c.signal.cpu().numpy() == 0).all()
        cg = Case(good)
        ex.run(cg.input, cg.target, cg.signal, cg.send, cg.recv, 8, wl.FP32, check=True)
        cg.assert_matches(a2av.OK, cg.run_oracle())
    finally:
        ex.close()


def test_tiny_spin_limit_latches_timeout_and_the_run_still_completes():
    # The arrival wait is bounded by the handle's spin limit.  With a limit of
    # 1 the first workgroups to arrive give up after two polls (they finish
    # microseconds apart) and latch TIMEOUT; every workgroup still leaves the
    # kernel, and the payload and the flags are complete, since a workgroup
    # copies and arrives before it waits.  The next run reports cleanly.
    P = 8
    rng = np.random.default_rng(17)
    C = rng.integers(1 << 18, 1 << 19, size=(P, P)).astype(np.int32)
    w = wl.custom(P, wl.FP32, C, core_num=8, S=8)
    c = Case(w)
    ex = exchange_for(w, spin_limit=1, wg_per_block=32)
    try:
        assert ex.launch_info(w.core_num).workgroups == 256
        assert c.run_gpu(ex) == a2av.ERR_TIMEOUT
        exp = c.run_oracle()
        c.assert_matches(a2av.OK, exp)
        assert ex.query_error() == a2av.OK              # the latch was cleared by the read
    finally:
        ex.close()
    ex2 = exchange_for(w)
    try:
        c.signal_np0 = exp[2].copy()
        c.target.fill_(wl.SENTINEL)
        c.assert_matches(c.run_gpu(ex2), c.run_oracle())
    finally:
        ex2.close()


# ------------------------------------------------------------------ host-side errors

def test_launch_capacity_refused_not_partial():
    P = 4
    w = wl.custom(P, wl.FP32, np.ones((P, P), np.int32), core_num=8, S=8)
    ex = exchange_for(w, capacity_override=4)
    c = Case(w)
    try:
        with pytest.raises(ValueError, match="LAUNCH_CAPACITY"):
            c.run_gpu(ex)
        torch.cuda.synchronize()
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
        # B = 4 fits.
        c.assert_matches(c.run_gpu(ex, core_num=4), c.run_oracle(core_num=4, capacity=4))
    finally:
        ex.close()


def test_refused_launch_writes_nothing():
    # A launch the runtime refuses: the handle is told the device holds 8,192
    # workgroups at once (capacity_override), so 2,048 blocks pass the host
    # check, but the cooperative launch of 2,048 one-per-CU workgroups cannot
    # be resident together and the runtime refuses it before anything runs.
    # The run has one K2 launch; the count kernel before it writes only the
    # workspace, so a2av_run returns A2AV_ERR_HIP and target, signal and
    # recv_counts keep their contents.  The handle works normally afterwards.
    P = 8
    w = wl.custom(P, wl.FP32, np.full((P, P), 64, np.int32), core_num=2048, S=2048)
    # A short barrier bound, so that even a launch the runtime did not refuse
    # would end at once (with TIMEOUT) rather than wait on absent blocks.
    ex = exchange_for(w, capacity_override=8192, wg_per_block=1, spin_limit=1 << 12)
    c = Case(w)
    try:
        info = ex.launch_info(2048)
        assert info.blocks == 2048 and info.workgroups == 2048 and info.cooperative == 1
        assert info.chunk_launches == 1
        say("refused launch", info.workgroups, "workgroups")
        with pytest.raises(a2av.A2avError, match="A2AV_ERR_HIP"):
            c.run_gpu(ex)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
        assert (c.recv.cpu().numpy() == -7).all()
        c.assert_matches(c.run_gpu(ex, core_num=8), c.run_oracle(core_num=8))
    finally:
        ex.close()


@pytest.mark.parametrize("P,L", [(8, 64), (32, 256), (5, 7), (64, 256)])
def test_no_block_wait_matches_the_oracle(P, L):
    # A2AV_FLAG_NO_BLOCK_WAIT: B > 1 runs end in a regular launch with no wait
    # for the other blocks; target, flags and recv_counts are those of the
    # cooperative run (the oracle's), over two runs and with chunked launches.
    rng = np.random.default_rng(P * 1000 + L)
    C = rng.integers(0, 20000 if P <= 8 else 2000, size=(P, P)).astype(np.int32)
    C[rng.random((P, P)) < 0.15] = 0
    for dtype in (wl.FP32, wl.INT8):
        w = wl.custom(P, dtype, C, core_num=L, seed=L + dtype)
        for limit in (0, 1 << 16):
            ex = exchange_for(w, block_wait=False, chunk_limit_bytes=limit)
            try:
                info = ex.launch_info(L)
                assert info.blocks > 1 and info.cooperative == 0
            finally:
                ex.close()
            say("no block wait: P", P, "L", L, "dtype", dtype, "limit", limit)
            check_case(w, runs=2, block_wait=False, chunk_limit_bytes=limit)


def test_host_errors_raise_before_enqueue():
    P = 4
    w = wl.custom(P, wl.FP32, np.ones((P, P), np.int32), core_num=4)
    ex = exchange_for(w)
    c = Case(w)
    try:
        with pytest.raises(ValueError, match="INVALID_ARGS"):       # S < B
            c.run_gpu(ex, core_num=64)
        with pytest.raises(ValueError, match="UNSUPPORTED_DTYPE"):
            ex.run(c.input, c.target, c.signal, c.send, c.recv, 4, 2)
        with pytest.raises(ValueError, match="INVALID_ARGS"):       # core_num 0
            c.run_gpu(ex, core_num=0)
        st = a2av.a2av_run(ex.h, c.input.data_ptr(), c.input.data_ptr(), c.signal.data_ptr(),
                           c.send.data_ptr(), c.recv.data_ptr(), P, 4, wl.FP32, None)
        assert st == a2av.ERR_INVALID_ARGS                          # input aliases target
        st = a2av.a2av_run(ex.h, c.input.data_ptr(), c.target.data_ptr(), None,
                           c.send.data_ptr(), c.recv.data_ptr(), P, 4, wl.FP32, None)
        assert st == a2av.ERR_NULLPTR
        with pytest.raises(ValueError, match="contiguous"):
            ex.run(c.input, c.target, c.signal, c.send.t(), c.recv, 4, wl.FP32)
        with pytest.raises(ValueError, match="at most one"):       # two exchanges named
            ex.run(c.input, c.target, c.signal, c.send, c.recv, 4, wl.FP32,
                   index=torch.zeros((P, 4), dtype=torch.int32, device=DEV), row_elems=1,
                   bias=torch.zeros((P, 1, 8), dtype=torch.float32, device=DEV), hidden=8)
        with pytest.raises(ValueError, match="no nblk"):
            ex.run(c.input, c.target, c.signal, c.send, c.recv, 4, wl.FP32, nblk=2,
                   index=torch.zeros((P, 4), dtype=torch.int32, device=DEV), row_elems=1)
        torch.cuda.synchronize()
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
        assert ex.query_error() == a2av.OK
    finally:
        ex.close()


# ------------------------------------------------------------------ properties

@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_round_trip_on_gpu(dtype):
    rng = np.random.default_rng(12)
    P = 8
    e = wl.ELEM_SIZE[dtype]
    C = rng.integers(0, 7000, size=(P, P)).astype(np.int32)
    slab = 7000 * P * e + 64
    w = wl.custom(P, dtype, C, core_num=P, in_slab=slab, tgt_slab=slab)
    c = Case(w)
    ex = exchange_for(w)
    try:
        assert c.run_gpu(ex) == a2av.OK
        back = torch.zeros_like(c.input)
        sig2 = torch.zeros((P, w.S), dtype=torch.int32, device=DEV)
        rc2 = torch.zeros((P, P), dtype=torch.int32, device=DEV)
        ex.run(c.target, back, sig2, c.recv, rc2, P, dtype)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK
        b = back.view(P, slab).cpu().numpy()
        a = c.input.view(P, slab).cpu().numpy()
        for s in range(P):
            n = int(C[s].sum()) * e
            np.testing.assert_array_equal(b[s, :n], a[s, :n])
        np.testing.assert_array_equal(rc2.cpu().numpy(), C)
    finally:
        ex.close()


def test_generator_on_gpu_matches_numpy():
    t = torch.empty(10_000_003, dtype=torch.uint8, device=DEV)
    wl.fill_random_(t, 4242, chunk_words=1 << 18)
    np.testing.assert_array_equal(t.cpu().numpy(), wl.random_bytes_np(4242, 0, t.numel()))


def test_block_count_changes_between_runs_on_one_handle():
    # One handle, runs with core_num giving B = 64, 1, 8, 3, 64, 16 in turn: the
    # per-block counters and the arrival counter copies are reset by every
    # run's count kernel, whatever B the run before used.  The signal is set
    # back to zeros before each run, so each run's precondition holds.
    P = 8
    C = np.random.default_rng(77).integers(0, 1 << 18, size=(P, P)).astype(np.int32)
    w = wl.custom(P, wl.FP32, C, core_num=64, S=80, seed=77)
    c = Case(w)
    ex = exchange_for(w)
    try:
        for L in (64, 1, 8, 3, 64, 16):
            c.signal.zero_()
            c.signal_np0 = np.zeros_like(c.signal_np0)
            c.target.fill_(wl.SENTINEL)
            c.recv.fill_(-7)
            say("core_num", L, "B", oracle.blocks(P, L))
            c.assert_matches(c.run_gpu(ex, core_num=L), c.run_oracle(core_num=L))
    finally:
        ex.close()


@pytest.mark.parametrize("core_num", [1, 16])
def test_signal_wraps_at_int32_max(core_num):
    # Every admitted entry at INT32_MAX: one run takes it to INT32_MIN (32-bit
    # wraparound), the next to INT32_MIN + 1; columns past the admitted
    # blocks hold other values and stay untouched.  B = 1 (regular launch)
    # and B = 16 (cooperative).
    P = 4
    rng = np.random.default_rng(31)
    C = rng.integers(0, 300, size=(P, P)).astype(np.int32)
    w = wl.custom(P, wl.FP32, C, core_num=core_num, S=24, seed=31)
    B = a2av.a2av_blocks(P, core_num)
    sig = np.full((P, w.S), -5, np.int32)
    sig[:, :B] = np.iinfo(np.int32).max
    c = Case(w, signal_np=sig)
    ex = exchange_for(w)
    try:
        for expect in (np.iinfo(np.int32).min, np.iinfo(np.int32).min + 1):
            st = c.run_gpu(ex)
            exp = c.run_oracle()
            c.assert_matches(st, exp)
            got = c.signal.cpu().numpy()
            assert (got[:, :B] == expect).all() and (got[:, B:] == -5).all()
            c.signal_np0 = exp[2].copy()
    finally:
        ex.close()
