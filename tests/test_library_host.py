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


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "a2av.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(a2av_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(a2av.EXPORTS)
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
