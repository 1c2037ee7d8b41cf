"""CPU tests of the HIP library's host side: it loads, exports every symbol the
header declares, and its fold and host-side argument checks agree with the
oracle's on every diagnostic row that the host decides.  No kernel runs here.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from all_movement_amd import a2av
from all_movement_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="a2av.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(a2av_[a-z_]+)\s*\(", text)))


@pytest.mark.parametrize("header,exports", [("a2av.h", "EXPORTS"),
                                            ("a2av_probe.h", "PROBE_EXPORTS")])
def test_library_exports_every_declared_symbol(header, exports):
    names = _declared_functions(header)
    assert set(names) == set(getattr(a2av, exports))
    L = a2av.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", a2av.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (a2av_[a-z_]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_library_has_gfx950_code_object():
    # The offload bundle names its target triple and processor.
    blob = open(a2av.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings():
    for code, name in [(0, "A2AV_OK"), (1, "A2AV_ERR_NULLPTR"), (2, "A2AV_ERR_INVALID_ARGS"),
                       (3, "A2AV_ERR_UNSUPPORTED_DTYPE"), (4, "A2AV_ERR_OVER_CAPACITY"),
                       (5, "A2AV_ERR_LAUNCH_CAPACITY"), (6, "A2AV_ERR_HIP"),
                       (7, "A2AV_ERR_TIMEOUT"), (99, "A2AV_ERR_UNKNOWN")]:
        assert a2av.a2av_status_string(code) == name
    # Same numbers as the oracle reports.
    assert (oracle.OK, oracle.ERR_NULLPTR, oracle.ERR_INVALID_ARGS, oracle.ERR_UNSUPPORTED_DTYPE,
            oracle.ERR_OVER_CAPACITY, oracle.ERR_LAUNCH_CAPACITY) == (
        a2av.OK, a2av.ERR_NULLPTR, a2av.ERR_INVALID_ARGS, a2av.ERR_UNSUPPORTED_DTYPE,
        a2av.ERR_OVER_CAPACITY, a2av.ERR_LAUNCH_CAPACITY)


def test_blocks_fold_matches_oracle_and_golden():
    for P in range(1, 65):
        for L in list(range(1, 300)) + [2**31 - 1]:
            assert a2av.a2av_blocks(P, L) == oracle.blocks(P, L)
    assert a2av.a2av_blocks(8, 10) == 8
    assert a2av.a2av_blocks(0, 3) == -1 and a2av.a2av_blocks(3, 0) == -1


def _cfg(P, S, in_slab, tgt_slab):
    return a2av.a2av_config(0, P, in_slab, tgt_slab, S, 0, 0, 0, 0, 0)


def _both(bufs, P, S, in_slab, tgt_slab, core_num=1, dtype=wl.INT8, capacity=0, override=None):
    ptrs = [b.ctypes.data for b in bufs]
    if override:
        for i, v in override.items():
            ptrs[i] = v
    lib_st = a2av.a2av_check_args(_cfg(P, S, in_slab, tgt_slab), capacity, *ptrs, P, core_num,
                                  dtype)
    or_st = oracle.check(*ptrs, P=P, S=S, in_slab=in_slab, tgt_slab=tgt_slab, core_num=core_num,
                         dtype=dtype, capacity=capacity)
    return lib_st, or_st


def _buffers(P, S, in_slab, tgt_slab):
    return (np.zeros(P * in_slab, np.uint8), np.full(P * tgt_slab, wl.SENTINEL, np.uint8),
            np.zeros((P, S), np.int32), np.ones((P, P), np.int32), np.zeros((P, P), np.int32))


HOST_ROWS = [
    # (description, P, S, in_slab, tgt_slab, kwargs)
    ("ok", 4, 4, 16, 16, {}),
    ("null input", 4, 4, 16, 16, {"override": {0: None}}),
    ("null target", 4, 4, 16, 16, {"override": {1: None}}),
    ("null signal", 4, 4, 16, 16, {"override": {2: None}}),
    ("null send", 4, 4, 16, 16, {"override": {3: None}}),
    ("null recv", 4, 4, 16, 16, {"override": {4: None}}),
    ("dtype 2", 4, 4, 16, 16, {"dtype": 2}),
    ("core_num 0", 4, 4, 16, 16, {"core_num": 0}),
    ("core_num 2^31", 4, 4, 16, 16, {"core_num": 2**31}),
    ("S < B", 4, 4, 16, 16, {"core_num": 8}),
    ("S == B", 4, 4, 16, 16, {"core_num": 5}),
    ("capacity", 4, 8, 16, 16, {"core_num": 8, "capacity": 4}),
    ("capacity ok", 4, 8, 16, 16, {"core_num": 8, "capacity": 8}),
    ("B=1 ignores capacity", 4, 8, 16, 16, {"core_num": 1, "capacity": 0}),
    ("slab not whole fp32", 4, 4, 18, 16, {"dtype": wl.FP32}),
    ("slab fine for int8", 4, 4, 18, 16, {"dtype": wl.INT8}),
]


@pytest.mark.parametrize("row", HOST_ROWS, ids=[r[0] for r in HOST_ROWS])
def test_host_checks_match_oracle(row):
    name, P, S, ins, tgs, kw = row
    b = _buffers(P, S, ins, tgs)
    lib_st, or_st = _both(b, P, S, ins, tgs, **kw)
    assert lib_st == or_st, (name, lib_st, or_st)


def test_host_checks_aliasing_matches_oracle():
    P, S = 4, 4
    b = _buffers(P, S, 16, 16)
    for i in range(5):
        for j in range(5):
            if i == j:
                continue
            for delta in [0, 1, 3]:
                lib_st, or_st = _both(b, P, S, 16, 16, override={j: b[i].ctypes.data + delta})
                assert lib_st == or_st == a2av.ERR_INVALID_ARGS, (i, j, delta)
    # Adjacent but disjoint ranges are fine.
    big = np.zeros(4 * 16 + 4 * 16, np.uint8)
    lib_st, or_st = _both(b, P, S, 16, 16, override={0: big.ctypes.data,
                                                     1: big.ctypes.data + 64})
    assert lib_st == or_st == a2av.OK


def test_host_checks_leave_device_rows_to_the_device():
    # Negative counts, over-capacity counts and an unequal signal are decided
    # by the count kernel, so the host check passes them.
    P, S = 4, 4
    b = _buffers(P, S, 16, 16)
    b[3][0, 0] = -1
    lib_st, or_st = _both(b, P, S, 16, 16)
    assert lib_st == a2av.OK and or_st == a2av.ERR_INVALID_ARGS
    b = _buffers(P, S, 12, 16)
    lib_st, or_st = _both(b, P, S, 12, 16, dtype=wl.FP32)
    assert lib_st == a2av.OK and or_st == a2av.ERR_OVER_CAPACITY


def test_run_rejects_null_handle():
    assert a2av.a2av_run(None, 1, 2, 3, 4, 5, 1, 1, 0, None) == a2av.ERR_NULLPTR
    assert a2av.a2av_query_error(None) == a2av.ERR_NULLPTR
    assert a2av.a2av_destroy(None) == a2av.OK


def test_create_rejects_bad_geometry_without_touching_the_device():
    for cfg in [_cfg(0, 1, 16, 16), _cfg(65, 1, 16, 16), _cfg(4, 0, 16, 16), _cfg(4, 1, 0, 16),
                _cfg(4, 1, 16, -1)]:
        st, h = a2av.a2av_create(cfg)
        assert st == a2av.ERR_INVALID_ARGS and h is None


def test_chunk_plan_is_bounded_to_2_pow_20_launches():
    # P * min(slabs) / chunk limit: exactly 2^20 launches is the largest plan.
    P, slab = 8, 1 << 20
    ok = a2av.a2av_config(0, P, slab, slab, 1, 0, 8, 0, 0, 0)         # 2^23 / 8 = 2^20
    over = a2av.a2av_config(0, P, slab, slab, 1, 0, 7, 0, 0, 0)       # > 2^20
    # Host checks only: the five operands are distinct, non-overlapping fake addresses.
    args = lambda cfg: (ctypes.byref(cfg), 0, 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44,
                        P, 1, wl.INT8)
    assert a2av.lib().a2av_check_args(*args(ok)) == a2av.OK
    assert a2av.lib().a2av_check_args(*args(over)) == a2av.ERR_INVALID_ARGS
    st, h = a2av.a2av_create(over)
    assert st == a2av.ERR_INVALID_ARGS and h is None


# ------------------------------------------------ bias and indexed host checks

def _bias_bufs(P=4, nblk=2, hidden=8, slab=128, dtype=wl.BF16):
    C = np.full((P, P), nblk * hidden, np.int32)           # whole rows of every sub-block
    bias = np.zeros(P * nblk * hidden, np.float32 if dtype == wl.BF16 else np.uint16)
    return [np.zeros(P * slab, np.uint8), np.full(P * slab, wl.SENTINEL, np.uint8),
            np.zeros((P, 8), np.int32), C, np.zeros((P, P), np.int32), bias]


def _bias_both(bufs, P=4, S=8, slab=128, tgt_slab=None, core_num=1, dtype=wl.BF16, nblk=2,
               hidden=8, capacity=0, chunk=0, override=None):
    tgt_slab = slab if tgt_slab is None else tgt_slab
    ptrs = [b.ctypes.data for b in bufs]
    for i, v in (override or {}).items():
        ptrs[i] = v
    cfg = a2av.a2av_config(0, P, slab, tgt_slab, S, 0, chunk, 0, 0, 0)
    lib_st = a2av.a2av_check_bias_args(cfg, capacity, *ptrs, P, core_num, dtype, nblk, hidden)
    or_st = oracle.lib().a2av_oracle_run_bias(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], P, S,
                                              slab, tgt_slab, core_num, dtype, capacity, nblk,
                                              ptrs[5], hidden)
    return lib_st, or_st


BIAS_ROWS = [
    ("ok", {}),
    ("ok fp16", {"dtype": wl.FP16}),
    ("null bias", {"override": {5: None}}),
    ("null input", {"override": {0: None}}),
    ("dtype fp32", {"dtype": wl.FP32}),
    ("dtype int8", {"dtype": wl.INT8}),
    ("nblk 0", {"nblk": 0}),
    ("hidden 0", {"hidden": 0}),
    ("P differs", {"P": 5}),
    ("core_num 0", {"core_num": 0}),
    ("S < B", {"core_num": 12}),
    ("capacity", {"core_num": 8, "capacity": 4}),
    ("odd slab", {"slab": 129}),
]


@pytest.mark.parametrize("row", BIAS_ROWS, ids=[r[0] for r in BIAS_ROWS])
def test_bias_host_checks_match_oracle(row):
    name, kw = row
    kw = dict(kw)
    dtype = kw.get("dtype", wl.BF16)
    slab = kw.get("slab", 128)
    b = _bias_bufs(dtype=dtype if dtype in (wl.BF16, wl.FP16) else wl.BF16, slab=slab)
    if "P" in kw:            # the run names a P the handle was not created for
        P = kw.pop("P")
        ptrs = [x.ctypes.data for x in b]
        cfg = a2av.a2av_config(0, 4, slab, slab, 8, 0, 0, 0, 0, 0)
        st = a2av.a2av_check_bias_args(cfg, 0, *ptrs, P, 1, wl.BF16, 2, 8)
        assert st == a2av.ERR_INVALID_ARGS
        return
    lib_st, or_st = _bias_both(b, **kw)
    assert lib_st == or_st, (name, lib_st, or_st)


def test_bias_host_checks_aliasing_matches_oracle():
    b = _bias_bufs()
    for j in range(5):
        lib_st, or_st = _bias_both(b, override={5: b[j].ctypes.data})
        assert lib_st == or_st == a2av.ERR_INVALID_ARGS, j


def test_bias_host_limits_of_the_gpu_path():
    # Rows of a multiple of 8 elements, 16-byte aligned operands, slabs and
    # chunk limit: the GPU path refuses what the oracle (no such limits) runs.
    b = _bias_bufs(hidden=12, slab=192)     # buffers sized for the slab the run names
    assert _bias_both(b, hidden=12, slab=192) == (a2av.ERR_INVALID_ARGS, a2av.OK)
    b = _bias_bufs()
    buf = np.zeros(4 * 128 + 16, np.uint8)
    for off, idx in [(2, 0), (8, 1)]:
        lib_st, or_st = _bias_both(b, override={idx: buf.ctypes.data + off})
        assert (lib_st, or_st) == (a2av.ERR_INVALID_ARGS, a2av.OK), (off, idx)
    b = _bias_bufs(slab=136)
    assert _bias_both(b, slab=136) == (a2av.ERR_INVALID_ARGS, a2av.OK)
    b = _bias_bufs()
    assert _bias_both(b, chunk=1000) == (a2av.ERR_INVALID_ARGS, a2av.OK)
    assert _bias_both(b, chunk=4096) == (a2av.OK, a2av.OK)


def _idx_bufs(P=4, R=4, rows=2, slab=64, stride=8, dtype=wl.INT8):
    C = np.full((P, P), rows * R, np.int32)
    table_rows = slab // (R * wl.ELEM_SIZE[dtype])
    index = (np.arange(P * stride) % table_rows).astype(np.int32)
    return [np.zeros(P * slab, np.uint8), np.full(P * 256, wl.SENTINEL, np.uint8),
            np.zeros((P, 8), np.int32), C, np.zeros((P, P), np.int32), index]


def _idx_both(bufs, P=4, S=8, slab=64, core_num=1, dtype=wl.INT8, R=4, stride=8, capacity=0,
              override=None):
    ptrs = [b.ctypes.data for b in bufs]
    for i, v in (override or {}).items():
        ptrs[i] = v
    cfg = a2av.a2av_config(0, P, slab, 256, S, 0, 0, 0, 0, 0)
    lib_st = a2av.a2av_check_indexed_args(cfg, capacity, *ptrs, P, core_num, dtype, R, stride)
    or_st = oracle.lib().a2av_oracle_run_indexed(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4],
                                                 ptrs[5], P, S, slab, 256, core_num, dtype,
                                                 capacity, R, stride)
    return lib_st, or_st


IDX_ROWS = [
    ("ok", {}),
    ("null index", {"override": {5: None}}),
    ("null recv", {"override": {4: None}}),
    ("dtype bf16", {"dtype": wl.BF16}),
    ("row_elems 0", {"R": 0}),
    ("stride 0", {"stride": 0}),
    ("core_num 2^31", {"core_num": 2**31}),
    ("S < B", {"core_num": 12}),
    ("capacity", {"core_num": 8, "capacity": 4}),
    ("slab not whole fp32", {"dtype": wl.FP32, "slab": 66}),
]


@pytest.mark.parametrize("row", IDX_ROWS, ids=[r[0] for r in IDX_ROWS])
def test_indexed_host_checks_match_oracle(row):
    name, kw = row
    slab = kw.get("slab", 64)
    b = _idx_bufs(slab=slab)
    lib_st, or_st = _idx_both(b, **kw)
    assert lib_st == or_st, (name, lib_st, or_st)


def test_indexed_host_checks_aliasing_matches_oracle():
    b = _idx_bufs()
    for j in range(5):
        lib_st, or_st = _idx_both(b, override={5: b[j].ctypes.data + 4})
        assert lib_st == or_st == a2av.ERR_INVALID_ARGS, j
    # The device decides bad entries: the host check passes them.
    b = _idx_bufs()
    b[5][3] = -1
    assert _idx_both(b) == (a2av.OK, a2av.ERR_INVALID_ARGS)


# ------------------------------------------------------------------ host counts

def _hc_cfg(P, in_slab, tgt_slab, limit=0):
    return a2av.a2av_config(0, P, in_slab, tgt_slab, 4, 0, limit, 0, 0, 0)


@pytest.mark.parametrize("seed", range(12))
def test_host_count_checks_match_oracle(seed):
    # a2av_check_host_counts against the oracle's count checks (negative,
    # then a row or column over its slab; the signal is equal here), and its
    # chunk plan against ceil(T / limit).
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 9))
    dtype = [wl.FP32, wl.INT8][seed % 2]
    e = wl.ELEM_SIZE[dtype]
    C = rng.integers(0, 50, size=(P, P)).astype(np.int32)
    in_slab = int(C.sum(axis=1).max()) * e + int(rng.integers(0, 3)) * e
    tgt_slab = int(C.sum(axis=0).max()) * e + int(rng.integers(0, 3)) * e
    kind = seed % 4
    if kind == 1:
        C[rng.integers(P), rng.integers(P)] = -int(rng.integers(1, 5))
    elif kind == 2:
        C[rng.integers(P), rng.integers(P)] += 60            # some row or column over
    in_slab, tgt_slab = max(in_slab, e), max(tgt_slab, e)
    limit = int(rng.choice([0, 64, 100 * e]))
    st, payload, launches = a2av.a2av_check_host_counts(_hc_cfg(P, in_slab, tgt_slab, limit), C,
                                                        dtype)
    inp = np.zeros(P * in_slab, np.uint8)
    tgt = np.zeros(P * tgt_slab, np.uint8)
    sig = np.zeros((P, 1), np.int32)
    rc = np.zeros((P, P), np.int32)
    st_o = oracle.run(inp, tgt, sig, C, rc, P=P, S=1, in_slab=in_slab, tgt_slab=tgt_slab,
                      core_num=1, dtype=dtype)
    assert st == st_o, (st, st_o)
    if st == a2av.OK:
        T = int(C.astype(np.int64).sum()) * e
        lim = limit or (1 << 30)
        assert payload == T and launches == max(1, -(-T // lim))


def test_host_count_checks_arguments():
    C = np.ones((4, 4), np.int32)
    assert a2av.a2av_check_host_counts(_hc_cfg(4, 64, 64), C, wl.BF16)[0] == \
        a2av.ERR_UNSUPPORTED_DTYPE
    assert a2av.a2av_check_host_counts(_hc_cfg(4, 64, 64), None, wl.FP32)[0] == a2av.ERR_NULLPTR
    assert a2av.a2av_check_host_counts(_hc_cfg(65, 64, 64), C, wl.FP32)[0] == \
        a2av.ERR_INVALID_ARGS
    # P = 64 with 1 GiB slabs: the geometry bound needs 64 launches; a small
    # payload needs one.
    C64 = np.ones((64, 64), np.int32)
    st, payload, launches = a2av.a2av_check_host_counts(_hc_cfg(64, 1 << 30, 1 << 30), C64,
                                                        wl.INT8)
    assert (st, payload, launches) == (a2av.OK, 4096, 1)


def test_gather_chunk_plan_takes_the_smaller_bound():
    # The row gather's plan covers min(P * tgt_slab, P * index_stride * row
    # bytes).  P = 8, input slabs of 2^16 bytes, target slabs of 2^20 bytes,
    # rows of 4 bytes.  At a chunk limit of 8 bytes the target bound needs
    # exactly 2^20 launches (accepted, whatever the gather lists); at 7 bytes
    # it needs more (refused) unless the gather lists bound the payload more
    # tightly.
    P = 8
    args = lambda cfg, stride: (ctypes.byref(cfg), 0, 1 << 40, 1 << 41, 1 << 42, 1 << 43,
                                1 << 44, 1 << 45, P, 1, wl.INT8, 4, stride)
    ok = a2av.a2av_config(0, P, 1 << 16, 1 << 20, 1, 0, 8, 0, 0, 0)
    over = a2av.a2av_config(0, P, 1 << 16, 1 << 20, 1, 0, 7, 0, 0, 0)
    lib = a2av.lib()
    assert lib.a2av_check_indexed_args(*args(ok, 1 << 18)) == a2av.OK
    assert lib.a2av_check_indexed_args(*args(ok, 1 << 30)) == a2av.OK
    assert lib.a2av_check_indexed_args(*args(over, 1 << 30)) == a2av.ERR_INVALID_ARGS
    assert lib.a2av_check_indexed_args(*args(over, 1 << 18)) == a2av.ERR_INVALID_ARGS
    # 2^17 rows of 4 bytes per source: 2^22 bytes / 7 < 2^20 launches.
    assert lib.a2av_check_indexed_args(*args(over, 1 << 17)) == a2av.OK


@pytest.mark.parametrize("kind", ["blocked", "bias", "indexed"])
@pytest.mark.parametrize("seed", range(16))
def test_host_count_checks_of_every_exchange_match_oracle(kind, seed):
    # a2av_check_host_counts_ex (the host part of the blocked, bias and
    # indexed *_host_counts entry points) against the oracle's status for the
    # same counts: negative, then not whole sub-blocks / bias rows / gathered
    # rows, then a source over in_slab (over index_stride rows for the row
    # gather) or a column over tgt_slab.  Signal equal and gather entries in
    # range, so the oracle's first failure, if any, is a count check; its
    # chunk plan against ceil(T / limit).
    rng = np.random.default_rng(1000 + seed)
    P = int(rng.integers(1, 7))
    if kind == "bias":
        dtype = [wl.BF16, wl.FP16][seed % 2]
        nblk, hidden = int(rng.choice([1, 2, 3])), int(rng.choice([1, 4, 8]))
        unit = nblk * hidden
    else:
        dtype = [wl.FP32, wl.INT8][seed % 2]
        nblk = int(rng.choice([1, 2, 4])) if kind == "blocked" else 1
        hidden = 0
        unit = nblk if kind == "blocked" else int(rng.choice([1, 3, 5]))
    e = wl.ELEM_SIZE[dtype]
    C = (rng.integers(0, 6, size=(P, P)) * unit).astype(np.int32)
    what = seed % 4
    if what == 1:
        C[rng.integers(P), rng.integers(P)] = -unit
    elif what == 2 and unit > 1:
        C[rng.integers(P), rng.integers(P)] += 1             # not whole
    elif what == 3:
        C[rng.integers(P), rng.integers(P)] += 8 * unit      # some row or column over
    rows = C.astype(np.int64).sum(axis=1) // unit
    stride = int(max(rows.max(initial=0), 1)) if kind == "indexed" else 0
    slack = int(rng.integers(0, 2)) * unit * e
    in_slab = max(int(C.sum(axis=1).max(initial=0)) * e, unit * e) + slack
    tgt_slab = max(int(C.sum(axis=0).max(initial=0)) * e, e) + slack
    if what == 3:
        stride = max(1, stride - 8)
        in_slab, tgt_slab = max(unit * e, in_slab - 8 * unit * e), max(e, tgt_slab - 8 * unit * e)
    limit = int(rng.choice([0, 64, 96]))
    cfg = _hc_cfg(P, in_slab, tgt_slab, limit)
    st, payload, launches = a2av.a2av_check_host_counts_ex(cfg, C, dtype, unit, stride)

    inp = np.zeros(P * in_slab, np.uint8)
    tgt = np.zeros(P * tgt_slab, np.uint8)
    sig = np.zeros((P, 4), np.int32)
    rc = np.zeros((P, P), np.int32)
    geo = dict(P=P, S=4, in_slab=in_slab, tgt_slab=tgt_slab, core_num=1, dtype=dtype)
    if kind == "blocked":
        st_o = oracle.run_blocked(inp, tgt, sig, C, rc, nblk=nblk, **geo)
    elif kind == "bias":
        b = np.zeros(P * nblk * hidden, np.float32 if dtype == wl.BF16 else np.uint16)
        st_o = oracle.run_bias(inp, tgt, sig, C, rc, b, nblk=nblk, hidden=hidden, **geo)
    else:
        index = np.zeros(P * stride, np.int32)               # row 0 of every table
        st_o = oracle.run_indexed(inp, tgt, sig, C, rc, index, row_elems=unit,
                                  index_stride=stride, **geo)
    assert st == st_o, (kind, what, st, st_o)
    if st == a2av.OK:
        T = int(C.astype(np.int64).sum()) * e
        assert payload == T and launches == max(1, -(-T // (limit or (1 << 30))))


def test_host_count_checks_ex_arguments():
    C = np.full((4, 4), 6, np.int32)
    cfg = _hc_cfg(4, 1024, 1024)
    assert a2av.a2av_check_host_counts_ex(cfg, C, 7, 1, 0)[0] == a2av.ERR_UNSUPPORTED_DTYPE
    assert a2av.a2av_check_host_counts_ex(cfg, None, wl.FP32, 1, 0)[0] == a2av.ERR_NULLPTR
    assert a2av.a2av_check_host_counts_ex(cfg, C, wl.FP32, 0, 0)[0] == a2av.ERR_INVALID_ARGS
    assert a2av.a2av_check_host_counts_ex(cfg, C, wl.FP32, 1, -1)[0] == a2av.ERR_INVALID_ARGS
    assert a2av.a2av_check_host_counts_ex(cfg, C, wl.FP16, 3, 0) == (a2av.OK, 192, 1)
    assert a2av.a2av_check_host_counts_ex(cfg, C, wl.INT8, 4, 0)[0] == a2av.ERR_INVALID_ARGS
    # Row gather: 4 sources x 4 destinations x 2 rows of 3 elements = 8 rows
    # per source: a list of 8 holds them, 7 does not.
    assert a2av.a2av_check_host_counts_ex(cfg, C, wl.INT8, 3, 8)[0] == a2av.OK
    assert a2av.a2av_check_host_counts_ex(cfg, C, wl.INT8, 3, 7)[0] == a2av.ERR_OVER_CAPACITY
    # The plain checker is the unit-1 case.
    assert a2av.a2av_check_host_counts(cfg, C, wl.FP32) == \
        a2av.a2av_check_host_counts_ex(cfg, C, wl.FP32, 1, 0)
