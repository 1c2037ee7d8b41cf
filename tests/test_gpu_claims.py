"""GPU parity of K2's claimed tiles: a launch deals the first eighth of its
tile rounds statically and hands the rest out from a counter, two counters
alternating between the launches of a run and reused by the next run.  These
cases make every launch large enough to claim (more than one round of tiles
per workgroup: 64 KiB for the byte copy, 128 KiB for the bias and gather
bodies), with odd and even numbers of launches, several runs on
one handle, several workgroups per block, and every body (plain, blocked,
bias, row gather).  Bit-exact against the oracle after every run."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import Case, exchange_for, say, upload  # noqa: E402

MiB = 1 << 20


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _counts(P, mean_bytes, elem, seed, multiple=1):
    rng = np.random.default_rng(seed)
    C = rng.integers(mean_bytes // (2 * elem), 3 * mean_bytes // (2 * elem), size=(P, P))
    return (C // multiple * multiple).astype(np.int32)


@pytest.mark.parametrize("launch_mib,runs", [(48, 3), (64, 2), (100, 3)])
def test_claimed_tiles_many_launches_many_runs(launch_mib, runs):
    # P=4 fp32, ~192 MiB of payload: 48 MiB chunks give 4 launches + empty
    # ones, 64 MiB gives 3, 100 MiB gives 2; each launch holds 1.5-3 rounds.
    P = 4
    C = _counts(P, 12 * MiB, 4, seed=launch_mib)
    w = wl.custom(P, wl.FP32, C, core_num=256, S=256, seed=launch_mib)
    c = Case(w)
    ex = exchange_for(w, chunk_limit_bytes=launch_mib * MiB)
    try:
        info = ex.launch_info(w.core_num)
        say("launches", info.chunk_launches, "workgroups", info.workgroups, "runs", runs)
        for run in range(runs):
            st = c.run_gpu(ex)
            exp = c.run_oracle()
            c.assert_matches(st, exp)
            c.signal_np0 = exp[2].copy()
            c.target.fill_(wl.SENTINEL)
            c.recv.fill_(-7)
    finally:
        ex.close()


@pytest.mark.parametrize("G", [2, 5])
def test_claimed_tiles_with_several_workgroups_per_block(G):
    P = 8
    C = _counts(P, 3 * MiB, 1, seed=G) | 1              # odd sizes: realigned pieces too
    w = wl.custom(P, wl.INT8, C, core_num=8, S=8, seed=G)
    c = Case(w)
    ex = exchange_for(w, wg_per_block=G)
    try:
        assert ex.launch_info(w.core_num).workgroups == 8 * G
        for _ in range(2):
            st = c.run_gpu(ex)
            exp = c.run_oracle()
            c.assert_matches(st, exp)
            c.signal_np0 = exp[2].copy()
    finally:
        ex.close()


def test_claimed_tiles_blocked_and_bias_bodies():
    # Blocked fp32 and BF16 + bias, both ~3 rounds per launch and two runs.
    P, A = 4, 4
    C = _counts(P, 16 * MiB, 4, seed=11, multiple=A * 64)
    w = wl.custom(P, wl.FP32, C, core_num=256, S=256, seed=12)
    c = Case(w)
    ex = exchange_for(w, chunk_limit_bytes=96 * MiB)
    try:
        for _ in range(2):
            st = c.run_gpu(ex, nblk=A)
            exp = c.run_oracle(nblk=A)
            c.assert_matches(st, exp)
            c.signal_np0 = exp[2].copy()
    finally:
        ex.close()

    H = 256
    Cb = _counts(P, 16 * MiB, 2, seed=13, multiple=A * H)
    wb = wl.custom(P, wl.BF16, Cb, core_num=256, S=256, seed=14)
    cb = Case(wb, input_np=wl.input16_np(wb))
    bn = wl.bias_np(wb, A, H)
    bt = torch.from_numpy(bn).to(cb.target.device)
    exb = exchange_for(wb, chunk_limit_bytes=96 * MiB)
    try:
        for _ in range(2):
            st = cb.run_gpu(exb, nblk=A, bias=bt, hidden=H)
            exp = cb.run_oracle(nblk=A, bias=bn, hidden=H)
            cb.assert_matches(st, exp)
            cb.signal_np0 = exp[2].copy()
    finally:
        exb.close()


@pytest.mark.parametrize("R,chunk_mib", [(1792, 0), (1792, 40), (1000, 40)])
def test_claimed_tiles_row_gather_body(R, chunk_mib):
    # int8 rows of R bytes gathered through the lists (1792: the 16-byte word
    # path; 1000: whole rows through the byte-exact copy), about 4 rounds of
    # tiles in one launch, or 1-2 rounds in each of several 40 MiB launches.
    P, table_rows = 8, 4096
    rng = np.random.default_rng(R + chunk_mib)
    rows = rng.integers(800, 1600, size=(P, P))
    C = (rows * R).astype(np.int32)
    in_slab = (table_rows * R + 15) // 16 * 16
    w = wl.custom(P, wl.INT8, C, core_num=64, S=64, in_slab=in_slab, seed=R)
    stride = int(rows.sum(axis=1).max()) + 3
    index = rng.integers(0, table_rows, size=(P, stride)).astype(np.int32)
    c = Case(w)
    ex = exchange_for(w, chunk_limit_bytes=chunk_mib * MiB)
    try:
        say("R", R, "payload", w.payload_bytes, "launches", ex.launch_info(w.core_num).chunk_launches)
        for _ in range(2):
            st = c.run_gpu(ex, index=upload(index), row_elems=R)
            exp = c.run_oracle(index=index, row_elems=R)
            c.assert_matches(st, exp)
            c.signal_np0 = exp[2].copy()
    finally:
        ex.close()
