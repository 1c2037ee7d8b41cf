"""GPU parity of the blocked exchange (a2av_run_blocked): each segment read as
nblk sub-blocks of the source's block-rows -- the AllToAll of the CANN
BatchMatMulReduceScatterAllToAll op on temp3 in its own (E/ep, ep*C, H/tp)
layout.  Bit-exact against the oracle's blocked exchange."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, check_case, exchange_for, say  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P", [1, 2, 3, 8, 32])
@pytest.mark.parametrize("nblk", [1, 2, 3, 8])
@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_blocked_sweep(P, nblk, dtype):
    rng = np.random.default_rng(100 * P + 10 * nblk + dtype)
    hi = 900 if P <= 8 else 60
    C = (rng.integers(0, hi + 1, size=(P, P)) * nblk).astype(np.int32)
    C[rng.random((P, P)) < 0.15] = 0
    for L in sorted({1, P, 2 * P + 1, 256}):
        w = wl.custom(P, dtype, C, core_num=L, seed=L + nblk)
        w.in_slab += 40
        w.tgt_slab += 52
        say("P", P, "nblk", nblk, "dtype", dtype, "L", L)
        check_case(w, nblk=nblk)


@pytest.mark.parametrize("P,nblk", [(16, 16), (16, 17), (8, 64), (64, 1), (64, 2)])
def test_blocked_segment_per_sub_block_bound(P, nblk):
    # A handle's tables hold 4,096 entries: up to P * P * nblk = 4,096 the
    # blocked byte copy takes one segment per sub-block (P = 16 with 16
    # sub-blocks, P = 8 with 64), past it K2 walks the sub-blocks of each
    # segment (P = 16 with 17, P = 64 with 2).  Both against the oracle, two
    # runs each, with small chunks as well.
    rng = np.random.default_rng(P * 1000 + nblk)
    C = (rng.integers(0, 7, size=(P, P)) * nblk).astype(np.int32)
    C[rng.random((P, P)) < 0.2] = 0
    w = wl.custom(P, wl.INT8, C, core_num=2 * P + 1, seed=nblk)
    w.in_slab += 24
    say("P", P, "nblk", nblk, "entries", P * P * nblk)
    check_case(w, nblk=nblk, runs=2)
    check_case(w, nblk=nblk, chunk_limit_bytes=1000)


@pytest.mark.parametrize("limit", [4096, 1000])
def test_blocked_small_chunks(limit):
    rng = np.random.default_rng(limit)
    P, nblk = 4, 4
    C = (rng.integers(0, 3000, size=(P, P)) * nblk).astype(np.int32)
    w = wl.custom(P, wl.INT8, C, core_num=8, seed=9)
    check_case(w, nblk=nblk, chunk_limit_bytes=limit)


def test_blocked_equal_counts_is_a_permute():
    # Equal counts: source slab s is (A, P, Q); target slab d must be (P, A, Q)
    # with target[d][s][a] = input[s][a][d]: torch's permute, compared on the GPU.
    P, A, Q = 8, 8, 4096 + 12
    C = np.full((P, P), A * Q, np.int32)
    w = wl.custom(P, wl.FP32, C, core_num=256, S=256)
    c = Case(w, host_input=False)
    ex = exchange_for(w)
    try:
        assert c.run_gpu(ex, nblk=A) == a2av.OK
        src = c.input.view(torch.int32).view(P, A, P, Q)
        want = src.permute(2, 0, 1, 3).contiguous().view(-1)
        assert torch.equal(c.target.view(torch.int32), want)
        assert (c.signal.cpu().numpy() == 1).all()
    finally:
        ex.close()


def test_blocked_indivisible_count_is_rejected_on_device():
    P, nblk = 4, 4
    C = np.full((P, P), 8, np.int32)
    C[2, 1] = 6
    w = wl.custom(P, wl.FP32, C, core_num=4)
    c = Case(w)
    ex = exchange_for(w)
    try:
        st = c.run_gpu(ex, nblk=nblk)
        assert st == a2av.ERR_INVALID_ARGS
        c.assert_matches(st, c.run_oracle(nblk=nblk))
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        with pytest.raises(ValueError, match="INVALID_ARGS"):
            c.run_gpu(ex, nblk=0)
    finally:
        ex.close()


def test_c5_blocked_full_size():
    # c5's counts with the source in the CANN temp3 layout: (E/ep=8, ep*C=8*2048,
    # H/tp=2048) per rank, nblk = E/ep = 8, 8 GiB of payload.
    w = wl.workload(5)
    P, A = w.P, w.extra["E_over_ep"]
    Q = int(w.counts[0, 0]) // A
    c = Case(w, host_input=False)
    ex = exchange_for(w)
    try:
        assert c.run_gpu(ex, nblk=A) == a2av.OK
        src = c.input.view(torch.int32).view(P, A, P, Q)
        tgt = c.target.view(torch.int32).view(P, P, A, Q)
        for d in range(P):
            assert torch.equal(tgt[d], src[:, :, d, :]), d
        np.testing.assert_array_equal(c.recv.cpu().numpy(), w.counts.T)
        assert (c.signal.cpu().numpy() == 1).all()
    finally:
        ex.close()
