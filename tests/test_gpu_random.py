"""Seeded random mixtures of everything the library takes -- P, dtype,
core_num, signal stride, workgroups per block, chunk limits, and the plain,
blocked, bias and indexed exchanges -- each compared bit for bit with the
oracle (whole target allocation, signal, recv_counts, status).  Payloads stay
under ~48 MiB; with the automatic workgroups-per-block choice many of these
launches span several tile rounds, so they claim tiles too."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, exchange_for, say, upload  # noqa: E402

N_CASES = 400


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _case(seed):
    rng = np.random.default_rng(90_000 + seed)
    kind = ["plain", "blocked", "bias", "indexed"][seed % 4]
    P = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 64]))
    L = int(rng.choice([1, max(1, P - 1), P, 2 * P + 1, 64, 256]))
    B = oracle.blocks(P, L)
    S = B + int(rng.integers(0, 3))
    G = int(rng.choice([0, 0, 1, 2, 3]))
    budget = int(rng.choice([1 << 20, 8 << 20, 48 << 20]))      # payload bytes, roughly
    unit_bytes, nblk, hidden, R, dtype = 1, 1, 0, 0, wl.INT8
    if kind in ("plain", "blocked"):
        dtype = int(rng.choice([wl.FP32, wl.INT8]))
        nblk = 1 if kind == "plain" else int(rng.choice([2, 3, 4, 8]))
        unit = nblk
    elif kind == "bias":
        dtype = int(rng.choice([wl.BF16, wl.FP16]))
        nblk = int(rng.choice([1, 2, 4]))
        hidden = int(rng.choice([8, 16, 40, 2048]))
        unit = nblk * hidden
    else:
        dtype = int(rng.choice([wl.FP32, wl.INT8]))
        R = int(rng.choice([1, 3, 4, 16, 448, 1792]))
        unit = R
    e = wl.ELEM_SIZE[dtype]
    per_seg = max(1, budget // (P * P * e * unit))
    C = (rng.integers(0, 2 * per_seg + 1, size=(P, P)) * unit).astype(np.int64)
    C[rng.random((P, P)) < 0.2] = 0
    C = C.astype(np.int32)
    align = 16 if kind in ("bias", "indexed") else 1
    pad = int(rng.integers(0, 4)) * 16 if align == 16 else int(rng.integers(0, 40)) * e
    if kind == "indexed":
        table_rows = max(1, int(rng.integers(1, 3 * per_seg * P + 2)))
        in_slab = ((table_rows * R * e + 15) // 16 * 16) + pad
    else:
        in_slab = None
    w = wl.custom(P, dtype, C, core_num=L, S=S, in_slab=in_slab, seed=seed)
    if kind != "indexed":
        w.in_slab += pad
    w.tgt_slab += pad
    # Chunk limits: tiny ones (many launches) only on small payloads.
    if rng.random() < 0.5:
        chunk = 0
    elif align == 16:
        chunk = int(rng.choice([4096, 1 << 16, 1 << 20, 3 << 20]))
    else:
        chunk = int(rng.choice([1000, 4096, 12345, 1 << 20, 5 << 20]))
    if 0 < chunk < (1 << 20) and budget > (1 << 20):
        chunk = 1 << 20
    extra = {}
    if kind == "indexed":
        rows = C.astype(np.int64).sum(axis=1) // R
        stride = int(rows.max(initial=0)) + int(rng.integers(1, 5))
        tr = w.in_slab // (R * e)
        extra["index"] = rng.integers(0, tr, size=(P, stride)).astype(np.int32)
    if kind == "bias":
        extra["bias"] = wl.bias_values(seed + 5, P, nblk, hidden, dtype)
    return dict(kind=kind, w=w, nblk=nblk, hidden=hidden, R=R, G=G, chunk=chunk, **extra)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_mixture(seed):
    c = _case(seed)
    w, kind = c["w"], c["kind"]
    say(seed, kind, "P", w.P, "dtype", w.dtype, "L", w.core_num, "S", w.S, "G", c["G"], "chunk",
        c["chunk"], "payload", w.payload_bytes, "nblk", c["nblk"], "hidden", c["hidden"], "R", c["R"])
    inp = wl.input16_np(w) if kind == "bias" else wl.input_bytes_np(w)
    case = Case(w, input_np=inp)
    ex = exchange_for(w, wg_per_block=c["G"], chunk_limit_bytes=c["chunk"])
    try:
        gkw, okw = {}, {}
        if kind == "blocked":
            gkw = okw = dict(nblk=c["nblk"])
        elif kind == "bias":
            b = c["bias"]
            bt = torch.from_numpy(b.view(np.float16) if w.dtype == wl.FP16 else b).to(DEV)
            gkw = dict(nblk=c["nblk"], bias=bt, hidden=c["hidden"])
            okw = dict(nblk=c["nblk"], bias=b, hidden=c["hidden"])
        elif kind == "indexed":
            gkw = dict(index=upload(c["index"]), row_elems=c["R"])
            okw = dict(index=c["index"], row_elems=c["R"])
        st = case.run_gpu(ex, **gkw)
        case.assert_matches(st, case.run_oracle(**okw))
    finally:
        ex.close()
