"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default Exchange settings, the workload's own core_num).

c3 and c4 are compared with the whole C oracle on the host.  c5 (8 GiB of
payload) is checked by a property that holds at any size -- with equal counts
the exchange is the block transpose target[d][s] = input[s][d], compared on
the GPU with torch slicing -- plus sampled bytes located one by one by the
oracle's per-byte view from regenerated input bytes.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from oracle import locate  # noqa: E402
from tests.gpu_harness import DEV, Case, exchange_for, say  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [3, 4])
def test_full_size_against_oracle(k):
    w = wl.workload(k)
    say("full size", w.name, "payload bytes", w.payload_bytes)
    c = Case(w, host_input=False)          # input generated on the GPU by the workload module
    ex = exchange_for(w)
    try:
        info = ex.launch_info(w.core_num)
        say("launch", info.blocks, info.wg_per_block, info.workgroups, info.chunk_launches)
        st = c.run_gpu(ex)
        c.assert_matches(st, c.run_oracle())
    finally:
        ex.close()


def test_p64_against_oracle():
    # The largest P: 64 ranks (4,096 segments), FP32 counts uniform in
    # [0, 2^17] with a fifth zeroed, 32 MiB slabs (4 GiB of allocations),
    # core_num 256 (B = 256, cooperative); whole oracle on the host.
    rng = np.random.default_rng(64)
    C = wl.uniform_counts(rng, 64, 1 << 17, 0.2)
    w = wl.custom(64, wl.FP32, C, core_num=256, S=256, in_slab=32 << 20, tgt_slab=32 << 20,
                  seed=64)
    say("P=64", w.payload_bytes)
    c = Case(w, host_input=False)
    ex = exchange_for(w)
    try:
        info = ex.launch_info(w.core_num)
        assert info.blocks == 256
        c.assert_matches(c.run_gpu(ex), c.run_oracle())
    finally:
        ex.close()


@pytest.mark.parametrize("seed", [41, 42])
def test_c4_shape_other_counts_against_oracle(seed):
    # c4's shape (P = 32 FP32, counts uniform in [0, 2^19] with 205 of 1024
    # zeroed, 64 MiB slabs, B = 256) with other count matrices and payloads.
    rng = np.random.default_rng(seed)
    C = wl.uniform_counts(rng, 32, 1 << 19, 205 / 1024)
    w = wl.custom(32, wl.FP32, C, core_num=256, S=256, in_slab=64 << 20, tgt_slab=64 << 20,
                  seed=seed)
    say("c4 shape, seed", seed, w.payload_bytes)
    c = Case(w, host_input=False)
    ex = exchange_for(w)
    try:
        c.assert_matches(c.run_gpu(ex), c.run_oracle())
    finally:
        ex.close()


def test_c4_with_small_chunks_against_oracle():
    # The chunked path the c4 text intends: 256 MiB per launch (about 4 launches).
    w = wl.workload(4)
    c = Case(w, host_input=False)
    ex = exchange_for(w, chunk_limit_bytes=256 << 20)
    try:
        assert ex.launch_info(w.core_num).chunk_launches == 8
        c.assert_matches(c.run_gpu(ex), c.run_oracle())
    finally:
        ex.close()


def test_c5_full_size_block_transpose_and_samples():
    w = wl.workload(5)
    P = w.P
    n = int(w.counts[0, 0]) * 4
    say("full size", w.name, "payload bytes", w.payload_bytes)
    c = Case(w, host_input=False)
    ex = exchange_for(w)
    try:
        info = ex.launch_info(w.core_num)
        assert info.chunk_launches == 8 and info.blocks == 256
        assert c.run_gpu(ex) == a2av.OK
        inp = c.input.view(P, P, n)
        tgt = c.target.view(P, P, n)
        for d in range(P):
            for s in range(P):
                assert torch.equal(tgt[d, s], inp[s, d]), (d, s)
        assert (c.signal.cpu().numpy() == 1).all()
        np.testing.assert_array_equal(c.recv.cpu().numpy(), w.counts.T)
        # Sampled bytes, located by the oracle and regenerated from the seed.
        rng = np.random.default_rng(55)
        d_idx = rng.integers(0, P, 4000)
        offs = rng.integers(0, w.tgt_slab, 4000)
        offs[:8] = [0, 1, 15, 16, n - 1, n, w.tgt_slab - 1, w.tgt_slab - 16]
        got = c.target.view(P, w.tgt_slab)[torch.as_tensor(d_idx, device=DEV),
                                           torch.as_tensor(offs, device=DEV)].cpu().numpy()
        for j in range(len(d_idx)):
            src = locate.source_of(w.counts, int(d_idx[j]), int(offs[j]), 4, w.in_slab)
            want = wl.SENTINEL if src is None else wl.random_bytes_np(w.payload_seed, src, 1)[0]
            assert got[j] == want, (int(d_idx[j]), int(offs[j]))
    finally:
        ex.close()


def test_largest_count_int8():
    # The largest int32 count: 2^31 - 1 int8 elements in one segment, beside
    # segments of 3 and 5 bytes, P = 2 with core_num 2 (B = 2, cooperative).
    # The payload, 2^31 + 7 bytes, spans chunks of 1 GiB, 1 GiB and 7 bytes
    # (segments cut at odd offsets), plus one launch past it.  Checked
    # on the GPU against the source bytes and at sampled bytes located by the
    # oracle from regenerated input.
    P, big = 2, (1 << 31) - 1
    C = np.array([[big, 0], [3, 5]], np.int32)
    w = wl.custom(P, wl.INT8, C, core_num=2, S=2, in_slab=big + 1, tgt_slab=big + 9, seed=77)
    say("largest count", w.payload_bytes)
    c = Case(w, host_input=False)
    ex = exchange_for(w)
    try:
        info = ex.launch_info(w.core_num)
        assert info.chunk_launches == 4 and info.blocks == 2
        assert c.run_gpu(ex) == a2av.OK
        inp = c.input.view(P, w.in_slab)
        tgt = c.target.view(P, w.tgt_slab)
        assert torch.equal(tgt[0, :big], inp[0, :big])          # segment 0 -> 0
        assert torch.equal(tgt[0, big:big + 3], inp[1, :3])     # segment 1 -> 0
        assert (tgt[0, big + 3:] == wl.SENTINEL).all()
        assert torch.equal(tgt[1, :5], inp[1, 3:8])             # segment 1 -> 1
        assert (tgt[1, 5:] == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 1).all()
        np.testing.assert_array_equal(c.recv.cpu().numpy(), C.T)
        rng = np.random.default_rng(7)
        d_idx = np.concatenate([np.zeros(300, np.int64), np.ones(20, np.int64)])
        offs = np.concatenate([rng.integers(0, w.tgt_slab, 300), np.arange(20)])
        offs[:6] = [0, (1 << 30) - 1, 1 << 30, big - 1, big, big + 2]
        got = tgt[torch.as_tensor(d_idx, device=DEV), torch.as_tensor(offs, device=DEV)].cpu().numpy()
        for j in range(len(d_idx)):
            src = locate.source_of(C, int(d_idx[j]), int(offs[j]), 1, w.in_slab)
            want = wl.SENTINEL if src is None else wl.random_bytes_np(w.payload_seed, src, 1)[0]
            assert got[j] == want, (int(d_idx[j]), int(offs[j]))
    finally:
        ex.close()


@pytest.mark.parametrize("k,variant", [(3, "no_block_wait"), (4, "host_counts_no_block_wait"),
                                       (3, "core_num_1"), (4, "core_num_1"), (4, "host_counts")])
def test_full_size_bench_variants_against_oracle(k, variant):
    # The other configurations the benchmark times on c3 and c4: a handle
    # with A2AV_FLAG_NO_BLOCK_WAIT, the run with a host copy of the counts,
    # and core_num 1 (B = 1, a regular launch); whole oracle on the host.
    w = wl.workload(k)
    if variant == "core_num_1":
        w.core_num = 1
    say("full size", w.name, variant, "payload bytes", w.payload_bytes)
    c = Case(w, host_input=False)
    ex = exchange_for(w, block_wait="no_block_wait" not in variant)
    try:
        if "host_counts" in variant:
            ex.run(c.input, c.target, c.signal, c.send, c.recv, w.core_num, w.dtype,
                   host_counts=w.counts)
            torch.cuda.synchronize()
            st = ex.query_error()
        else:
            st = c.run_gpu(ex)
        c.assert_matches(st, c.run_oracle())
    finally:
        ex.close()
