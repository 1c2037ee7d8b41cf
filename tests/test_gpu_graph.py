"""Runs captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

A run enqueues only kernels (K1 and the K2 launches, the last one
cooperative when B > 1), so it can be captured once and replayed: every
replay is one more run over the buffers' current contents.  Each case
captures one run, then replays it three times; before each replay the input
is changed in place and the target and recv_counts are reset, and an eager
run on the same handle follows each replay.  After every replay and every
eager run the whole target allocation, the signal (one more per run) and
recv_counts are compared bit for bit with the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, exchange_for, say, upload  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _counts(P, hi, unit, seed):
    rng = np.random.default_rng(seed)
    C = rng.integers(0, hi + 1, size=(P, P)) * unit
    C[rng.random((P, P)) < 0.2] = 0
    return C.astype(np.int32)


# name: (kind, P, dtype, core_num, max count per segment in units, unit, chunk limit)
CASES = {
    "plain_cooperative": ("plain", 8, wl.FP32, 64, 3000, 1, 0),
    "plain_one_block": ("plain", 4, wl.INT8, 1, 5000, 1, 0),
    "plain_chunked": ("plain", 5, wl.INT8, 10, 40000, 1, 65536),
    "blocked": ("blocked", 8, wl.FP32, 16, 300, 4, 0),
    "bias_bf16": ("bias", 8, wl.BF16, 8, 20, 2 * 64, 0),
    "indexed": ("indexed", 8, wl.INT8, 64, 12, 448, 0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_the_oracle(name):
    kind, P, dtype, L, hi, unit, chunk = CASES[name]
    say("graph case", name, "P", P, "dtype", dtype, "L", L, "chunk", chunk)
    C = _counts(P, hi, unit, seed=sum(map(ord, name)))
    gkw, okw = {}, {}
    in_slab = None
    if kind == "indexed":
        rows = C.astype(np.int64).sum(axis=1) // unit
        table_rows = int(rows.max()) + 3
        in_slab = table_rows * unit
    w = wl.custom(P, dtype, C, core_num=L, in_slab=in_slab, seed=11)
    if kind == "blocked":
        gkw = okw = dict(nblk=unit)
    elif kind == "bias":
        nblk, hidden = 2, 64
        b = wl.bias_values(5, P, nblk, hidden, dtype)
        gkw = dict(nblk=nblk, hidden=hidden, bias=torch.from_numpy(b).to(DEV))
        okw = dict(nblk=nblk, hidden=hidden, bias=b)
    elif kind == "indexed":
        stride = int((C.astype(np.int64).sum(axis=1) // unit).max()) + 2
        idx = np.random.default_rng(3).integers(0, w.in_slab // unit, size=(P, stride))
        idx = idx.astype(np.int32)
        gkw = dict(index=upload(idx), row_elems=unit)
        okw = dict(index=idx, row_elems=unit)
    inp0 = wl.input16_np(w) if kind == "bias" else wl.input_bytes_np(w)
    case = Case(w, input_np=inp0)
    ex = exchange_for(w, chunk_limit_bytes=chunk)
    g = None
    try:
        def check(st):
            exp = case.run_oracle(**okw)
            case.assert_matches(st, exp)
            case.signal_np0 = exp[2].copy()

        check(case.run_gpu(ex, **gkw))                 # an eager run first
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ex.run(case.input, case.target, case.signal, case.send, case.recv, w.core_num,
                   w.dtype, **gkw)
        torch.cuda.synchronize()
        # Capturing runs nothing: the signal is still that of the eager run.
        np.testing.assert_array_equal(case.signal.cpu().numpy(), case.signal_np0)
        for rep in range(3):
            say("  replay", rep)
            new = np.roll(inp0, 16 * (rep + 1))       # new payload, same value set
            case.input.copy_(upload(new))
            case.input_np = new
            case.target.fill_(wl.SENTINEL)
            case.recv.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            check(ex.query_error())
            say("  eager", rep)
            case.target.fill_(wl.SENTINEL)
            case.recv.fill_(-7)
            check(case.run_gpu(ex, **gkw))
    finally:
        del g
        torch.cuda.synchronize()
        ex.close()
