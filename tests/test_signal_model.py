"""The oracle's signal update pinned against the event model of the block
barrier (tests/barrier_model.py): over random P, signal strides, block counts
and entry values (INT32_MAX, INT32_MIN, -1 and 0 among them), and over
sequences of exchanges whose block count changes from one to the next, the
oracle must accept exactly the exchanges the model completes, refuse the
others with INVALID_ARGS, and leave the signal as the model's counters."""
import numpy as np
import pytest

import oracle
from all_movement_amd import workloads as wl
from tests.barrier_model import BarrierModel

EDGE_BASES = [2**31 - 1, -2**31, -1, 0, 1, 2**31 - 2]


def _oracle_exchange(sig, P, core_num, rng, payload=True):
    """One oracle exchange on the signal array (in place); returns its status."""
    S = sig.shape[1]
    C = rng.integers(0, 3, (P, P)).astype(np.int32) if payload else np.zeros((P, P), np.int32)
    in_slab = tgt_slab = 4 * P
    inp = rng.integers(0, 256, P * in_slab).astype(np.uint8)
    tgt = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    rc = np.zeros((P, P), np.int32)
    return oracle.run(inp, tgt, sig, C, rc, P=P, S=S, in_slab=in_slab, tgt_slab=tgt_slab,
                      core_num=core_num, dtype=oracle.INT8)


def _compare_sequence(P, S, sig0, core_nums, seed):
    rng = np.random.default_rng(seed)
    model = BarrierModel(sig0)
    sig = sig0.copy()
    for L in core_nums:
        B = oracle.blocks(P, L)
        accepted = model.exchange(B, rng)
        st = _oracle_exchange(sig, P, L, rng, payload=bool(rng.integers(2)))
        assert st == (oracle.OK if accepted else oracle.ERR_INVALID_ARGS), (P, S, L, B)
        np.testing.assert_array_equal(sig, model.signal())


@pytest.mark.parametrize("base", EDGE_BASES)
def test_signal_edge_entry_values(base):
    # Five exchanges from an edge value: the counters cross the int32 wrap
    # where the value starts next to it; columns past B keep their value.
    P, S = 3, 7
    sig0 = np.full((P, S), base, np.int32)
    sig0[:, 5:] = 77
    _compare_sequence(P, S, sig0, [4, 4, 3, 5, 4], seed=base & 0xFFFF)


def test_signal_random_geometries():
    rng = np.random.default_rng(11)
    for case in range(60):
        P = int(rng.integers(1, 9))
        S = int(rng.integers(1, 19))
        base = int(rng.choice(EDGE_BASES + [int(rng.integers(-2**31, 2**31))]))
        sig0 = np.full((P, S), base, np.int32)
        # Entries outside the first B0 columns start elsewhere, so a later
        # exchange admitting more blocks must be refused.
        B0 = int(rng.integers(1, S + 1))
        sig0[:, B0:] = rng.integers(-2**31, 2**31, (P, S - B0), dtype=np.int64).astype(np.int32)
        core_nums = [int(rng.integers(1, 3 * S + 2)) for _ in range(int(rng.integers(1, 6)))]
        _compare_sequence(P, S, sig0, core_nums, seed=1000 + case)


def test_signal_unequal_entry_is_refused_and_untouched():
    P, S = 4, 4
    sig0 = np.zeros((P, S), np.int32)
    sig0[2, 1] = 5
    _compare_sequence(P, S, sig0, [4, 1, 2], seed=7)     # B = 4 and 2 refused, B = 1 runs


def test_signal_block_count_changes_between_exchanges():
    # B = 8, then 1, then 8 again (refused: columns 1..7 lag), then 1 ...
    P, S = 8, 8
    sig0 = np.full((P, S), 2**31 - 3, np.int32)
    _compare_sequence(P, S, sig0, [10, 1, 10, 1, 1, 8], seed=3)


def test_model_refuses_more_blocks_than_columns():
    model = BarrierModel(np.zeros((2, 3), np.int32))
    assert not model.exchange(4, np.random.default_rng(0))
    assert (model.signal() == 0).all()
