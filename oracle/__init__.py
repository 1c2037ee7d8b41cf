"""CPU oracle for the variable-count all-to-all exchange (all_to_all_v).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
imports nothing from the product path: the two share no code.

Two independent implementations live here:

* ``liba2av_oracle.so`` (``a2av_oracle.c``): plain C loops, one ``memcpy`` per
  (source, destination) segment, its own argument checks, its own prefix sums.
* :mod:`oracle.brute`: a pure-Python brute force for tiny P that builds each
  destination slab by concatenating byte strings.

Semantics follow the five-operand ``all_to_all_v(input, target, signal,
send_counts, recv_counts, core_num)`` of the PyPTO "LowerL2TensorCollectives
Pass" page (section "Behavior"); segment addressing follows the ncclx
``ctranAllToAllvIbImpl`` pseudocode on the "vccl alltoallv dev log" page
(section 5).  What pins each function is stated in ``a2av_oracle.c``; the
signal's +1-per-exchange value, a reading of the barrier the pages describe,
is pinned against the event model in ``tests/barrier_model.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "a2av_oracle.c")
_LIB = os.path.join(_HERE, "liba2av_oracle.so")

OK = 0
ERR_NULLPTR = 1
ERR_INVALID_ARGS = 2
ERR_UNSUPPORTED_DTYPE = 3
ERR_OVER_CAPACITY = 4
ERR_LAUNCH_CAPACITY = 5

FP32 = 0
INT8 = 1
FP16 = 2
BF16 = 3
ELEM_SIZE = {FP32: 4, INT8: 1, FP16: 2, BF16: 2}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liba2av_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
             "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = load(_LIB)
    return _lib


def use_library(path: str) -> None:
    """Route every call of this module to the oracle library at ``path``
    (the tests' mutation pins run the pins against deliberately broken
    copies of ``a2av_oracle.c``, one process per copy)."""
    global _lib
    _lib = load(path)


def load(path: str) -> ctypes.CDLL:
    """Load an oracle library built from ``a2av_oracle.c`` and declare its
    functions' argument and return types."""
    L = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.a2av_oracle_blocks.argtypes = [i64, i64]
    L.a2av_oracle_blocks.restype = i64
    run_args = [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, i64]
    L.a2av_oracle_run.argtypes = run_args
    L.a2av_oracle_run.restype = ctypes.c_int
    L.a2av_oracle_check.argtypes = run_args
    L.a2av_oracle_check.restype = ctypes.c_int
    L.a2av_oracle_run_blocked.argtypes = run_args + [i32]
    L.a2av_oracle_run_blocked.restype = ctypes.c_int
    L.a2av_oracle_run_bias.argtypes = run_args + [i32, vp, i32]
    L.a2av_oracle_run_bias.restype = ctypes.c_int
    L.a2av_oracle_run_indexed.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i64, i64,
                                          i32, i64, i32, i64]
    L.a2av_oracle_run_indexed.restype = ctypes.c_int
    u16, u32 = ctypes.c_uint16, ctypes.c_uint32
    L.a2av_oracle_f32_to_bf16.argtypes = [u32]
    L.a2av_oracle_f32_to_bf16.restype = u16
    L.a2av_oracle_bf16_to_f32.argtypes = [u16]
    L.a2av_oracle_bf16_to_f32.restype = u32
    L.a2av_oracle_f32_to_f16.argtypes = [u32]
    L.a2av_oracle_f32_to_f16.restype = u16
    L.a2av_oracle_f16_to_f32.argtypes = [u16]
    L.a2av_oracle_f16_to_f32.restype = u32
    L.a2av_oracle_displacements.argtypes = [vp, i32, i32, vp, vp]
    L.a2av_oracle_displacements.restype = None
    L.a2av_oracle_move.argtypes = [vp, vp, vp, i32, i32, i64, i64]
    L.a2av_oracle_move.restype = None
    return L


def blocks(P: int, L: int) -> int:
    """CalAllToAllVBlocks(P, L) as the oracle computes it (-1 on bad input)."""
    return int(lib().a2av_oracle_blocks(P, L))


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def run(input_bytes: np.ndarray, target_bytes: np.ndarray, signal: np.ndarray,
        send_counts: np.ndarray, recv_counts: np.ndarray, *, P: int, S: int,
        in_slab: int, tgt_slab: int, core_num: int, dtype: int,
        capacity: int = 0) -> int:
    """Run the exchange in place on host numpy buffers; returns a status.

    ``input_bytes`` / ``target_bytes`` are flat uint8 arrays of ``P*in_slab`` /
    ``P*tgt_slab`` bytes; ``signal`` is int32 ``[P, S]``; counts are int32
    ``[P, P]``.  On error nothing is written.
    """
    for a, n in ((input_bytes, P * in_slab), (target_bytes, P * tgt_slab)):
        assert a.dtype == np.uint8 and a.size == n
    assert signal.dtype == np.int32 and signal.size == P * S
    assert send_counts.dtype == np.int32 and send_counts.size == P * P
    assert recv_counts.dtype == np.int32 and recv_counts.size == P * P
    return int(lib().a2av_oracle_run(
        _ptr(input_bytes), _ptr(target_bytes), _ptr(signal), _ptr(send_counts),
        _ptr(recv_counts), P, S, in_slab, tgt_slab, core_num, dtype, capacity))


def run_blocked(input_bytes: np.ndarray, target_bytes: np.ndarray, signal: np.ndarray,
                send_counts: np.ndarray, recv_counts: np.ndarray, *, P: int, S: int,
                in_slab: int, tgt_slab: int, core_num: int, dtype: int, nblk: int,
                capacity: int = 0) -> int:
    """The blocked exchange (each segment is nblk sub-blocks read from the
    source's block-rows); nblk = 1 is :func:`run`.  Same buffers as run."""
    for a, n in ((input_bytes, P * in_slab), (target_bytes, P * tgt_slab)):
        assert a.dtype == np.uint8 and a.size == n
    assert signal.dtype == np.int32 and signal.size == P * S
    assert send_counts.dtype == np.int32 and send_counts.size == P * P
    assert recv_counts.dtype == np.int32 and recv_counts.size == P * P
    return int(lib().a2av_oracle_run_blocked(
        _ptr(input_bytes), _ptr(target_bytes), _ptr(signal), _ptr(send_counts),
        _ptr(recv_counts), P, S, in_slab, tgt_slab, core_num, dtype, capacity, nblk))


def run_bias(input_bytes: np.ndarray, target_bytes: np.ndarray, signal: np.ndarray,
             send_counts: np.ndarray, recv_counts: np.ndarray, bias: np.ndarray | None, *,
             P: int, S: int, in_slab: int, tgt_slab: int, core_num: int, dtype: int, nblk: int,
             hidden: int, capacity: int = 0) -> int:
    """The exchange with the bias Add fused in front (16-bit payloads): the
    blocked exchange of (input + bias broadcast over rows), each sum formed in
    binary32 and rounded to nearest even.  ``bias`` is float32 [P, nblk, hidden]
    for BF16 payloads, uint16 (binary16 bits) for FP16."""
    for a, n in ((input_bytes, P * in_slab), (target_bytes, P * tgt_slab)):
        assert a.dtype == np.uint8 and a.size == n
    assert signal.dtype == np.int32 and signal.size == P * S
    return int(lib().a2av_oracle_run_bias(
        _ptr(input_bytes), _ptr(target_bytes), _ptr(signal), _ptr(send_counts),
        _ptr(recv_counts), P, S, in_slab, tgt_slab, core_num, dtype, capacity, nblk,
        _ptr(bias), hidden))


def run_indexed(input_bytes: np.ndarray, target_bytes: np.ndarray, signal: np.ndarray,
                send_counts: np.ndarray, recv_counts: np.ndarray, index: np.ndarray | None, *,
                P: int, S: int, in_slab: int, tgt_slab: int, core_num: int, dtype: int,
                row_elems: int, index_stride: int, capacity: int = 0) -> int:
    """The indexed exchange: source s sends the rows of its input table named by
    index[s] (int32 [P, index_stride]), in destination order."""
    for a, n in ((input_bytes, P * in_slab), (target_bytes, P * tgt_slab)):
        assert a.dtype == np.uint8 and a.size == n
    assert signal.dtype == np.int32 and signal.size == P * S
    if index is not None:
        assert index.dtype == np.int32 and index.size == P * index_stride
    return int(lib().a2av_oracle_run_indexed(
        _ptr(input_bytes), _ptr(target_bytes), _ptr(signal), _ptr(send_counts),
        _ptr(recv_counts), _ptr(index), P, S, in_slab, tgt_slab, core_num, dtype, capacity,
        row_elems, index_stride))


# The 16-bit conversions take and return bit patterns (binary32 bits as a
# uint32, 16-bit values as a uint16), so NaN payloads are not changed on the
# way through Python floats.  The array forms apply them element by element.

def f32_to_bf16(bits: int) -> int:
    return int(lib().a2av_oracle_f32_to_bf16(bits))


def bf16_to_f32(h: int) -> int:
    return int(lib().a2av_oracle_bf16_to_f32(h))


def f32_to_f16(bits: int) -> int:
    return int(lib().a2av_oracle_f32_to_f16(bits))


def f16_to_f32(h: int) -> int:
    return int(lib().a2av_oracle_f16_to_f32(h))


def _map(fn, a: np.ndarray, out_dtype) -> np.ndarray:
    return np.array([fn(int(v)) for v in np.asarray(a).ravel()], out_dtype)


def f32_to_bf16_array(bits: np.ndarray) -> np.ndarray:
    """uint32 binary32 patterns -> uint16 bfloat16 patterns."""
    return _map(lib().a2av_oracle_f32_to_bf16, bits, np.uint16)


def bf16_to_f32_array(h: np.ndarray) -> np.ndarray:
    return _map(lib().a2av_oracle_bf16_to_f32, h, np.uint32)


def f32_to_f16_array(bits: np.ndarray) -> np.ndarray:
    """uint32 binary32 patterns -> uint16 binary16 patterns."""
    return _map(lib().a2av_oracle_f32_to_f16, bits, np.uint16)


def f16_to_f32_array(h: np.ndarray) -> np.ndarray:
    return _map(lib().a2av_oracle_f16_to_f32, h, np.uint32)


def check(input_ptr, target_ptr, signal_ptr, send_ptr, recv_ptr, *, P, S, in_slab,
          tgt_slab, core_num, dtype, capacity=0, send_counts=None, signal=None) -> int:
    """Argument checks only, on raw addresses (counts/signal read when given)."""
    return int(lib().a2av_oracle_check(
        input_ptr, target_ptr, signal_ptr, send_ptr, recv_ptr, P, S, in_slab, tgt_slab,
        core_num, dtype, capacity))


def displacements(send_counts: np.ndarray, dtype: int) -> tuple[np.ndarray, np.ndarray]:
    """(sdispl[s][d], rdispl[d][s]) in bytes, int64 [P, P] each."""
    C = np.ascontiguousarray(send_counts, dtype=np.int32)
    P = C.shape[0]
    sd = np.zeros((P, P), np.int64)
    rd = np.zeros((P, P), np.int64)
    lib().a2av_oracle_displacements(_ptr(C), P, dtype, _ptr(sd), _ptr(rd))
    return sd, rd


def move(input_bytes: np.ndarray, target_bytes: np.ndarray, send_counts: np.ndarray, *,
         P: int, dtype: int, in_slab: int, tgt_slab: int) -> None:
    """The segment-copy step alone (no checks); counts must be valid."""
    C = np.ascontiguousarray(send_counts, dtype=np.int32)
    lib().a2av_oracle_move(_ptr(input_bytes), _ptr(target_bytes), _ptr(C), P, dtype,
                           in_slab, tgt_slab)
