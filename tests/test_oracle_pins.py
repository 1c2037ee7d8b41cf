"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every pin here is independent of the oracle's own code: printed cases from the
pages (tests/golden), closed forms (transpose, exclusive cumsum), library
routines (numpy block transpose), brute force (oracle.brute, a separate
pure-Python construction), invariants (round trip, byte conservation) and
special cases (P=1 identity, all-zero counts).
"""
import ctypes
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute, locate
from all_movement_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(w_counts, P, dtype, in_slab, tgt_slab, core_num=1, S=None, seed=3, signal=None):
    C = np.ascontiguousarray(w_counts, np.int32)
    if S is None:
        S = max(1, oracle.blocks(P, core_num))
    inp = wl.random_bytes_np(seed, 0, P * in_slab)
    tgt = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    sig = np.zeros((P, S), np.int32) if signal is None else signal.copy()
    rc = np.full((P, P), -7, np.int32)
    st = oracle.run(inp, tgt, sig, C, rc, P=P, S=S, in_slab=in_slab, tgt_slab=tgt_slab,
                    core_num=core_num, dtype=dtype)
    return st, inp, tgt, sig, rc


# ------------------------------------------------------------------- fold

def test_fold_printed_cases():
    g = json.load(open(os.path.join(GOLDEN, "fold_cases.json")))
    for c in g["printed_cases"] + g["rule_cases"]:
        assert oracle.blocks(c["P"], c["L"]) == c["B"]
    # The printed case also fixes that S = 8 is accepted for L=10, P=8.
    c = g["printed_cases"][0]
    P, S = c["P"], c["S_accepted"]
    C = np.zeros((P, P), np.int32)
    st, *_ = _run(C, P, wl.FP32, 64, 64, core_num=c["L"], S=S)
    assert st == oracle.OK
    st, *_ = _run(C, P, wl.FP32, 64, 64, core_num=c["L"], S=S - 1)
    assert st == oracle.ERR_INVALID_ARGS


def test_fold_brute_force():
    # Enumerate the multiples of P up to L and take the largest (or L when L < P).
    for P in range(1, 65):
        for L in range(1, 400):
            mult = [m for m in range(P, L + 1, P)]
            want = L if L < P else max(mult)
            assert oracle.blocks(P, L) == want, (P, L)
    assert oracle.blocks(8, 2**31 - 1) == (2**31 - 1) // 8 * 8
    assert oracle.blocks(0, 5) == -1 and oracle.blocks(4, 0) == -1


def test_fold_workloads():
    got = [oracle.blocks(wl.workload(k, scale=64).P, wl.workload(k, scale=64).core_num)
           for k in range(1, 6)]
    assert got == [1, 8, 64, 256, 256]


# ------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 17, 32, 64])
def test_recv_counts_is_transpose(P):
    rng = np.random.default_rng(P)
    C = rng.integers(0, 50, size=(P, P)).astype(np.int32)
    st, _, _, _, rc = _run(C, P, wl.INT8, 64 * P, 64 * P)
    assert st == oracle.OK
    np.testing.assert_array_equal(rc, C.T)


@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_displacements_exclusive_cumsum(dtype):
    rng = np.random.default_rng(11)
    P = 13
    C = rng.integers(0, 1000, size=(P, P)).astype(np.int32)
    e = wl.ELEM_SIZE[dtype]
    sd, rd = oracle.displacements(C, dtype)
    Cb = C.astype(np.int64) * e
    want_sd = np.concatenate([np.zeros((P, 1), np.int64), np.cumsum(Cb, axis=1)[:, :-1]], axis=1)
    want_rd = np.concatenate([np.zeros((P, 1), np.int64), np.cumsum(Cb.T, axis=1)[:, :-1]], axis=1)
    np.testing.assert_array_equal(sd, want_sd)
    np.testing.assert_array_equal(rd, want_rd)


# ------------------------------------------------------------------- brute force

def _brute_compare(C, dtype, in_slab, tgt_slab, seed):
    P = C.shape[0]
    e = wl.ELEM_SIZE[dtype]
    st, inp, tgt, sig, rc = _run(C, P, dtype, in_slab, tgt_slab, seed=seed)
    assert st == oracle.OK
    in_slabs = [bytes(inp[s * in_slab:(s + 1) * in_slab]) for s in range(P)]
    old = [bytes([wl.SENTINEL]) * tgt_slab for _ in range(P)]
    want = brute.exchange(in_slabs, old, C.tolist(), e)
    got = [bytes(tgt[d * tgt_slab:(d + 1) * tgt_slab]) for d in range(P)]
    assert got == want, C.tolist()
    assert rc.tolist() == brute.transpose(C.tolist())


@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_brute_force_all_2x2_in_0_1_2(dtype):
    e = wl.ELEM_SIZE[dtype]
    for vals in itertools.product(range(3), repeat=4):
        C = np.array(vals, np.int32).reshape(2, 2)
        _brute_compare(C, dtype, in_slab=5 * e, tgt_slab=6 * e, seed=sum(vals))


@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_brute_force_all_3x3_in_0_1(dtype):
    e = wl.ELEM_SIZE[dtype]
    for vals in itertools.product(range(2), repeat=9):
        C = np.array(vals, np.int32).reshape(3, 3)
        _brute_compare(C, dtype, in_slab=4 * e, tgt_slab=5 * e, seed=int("".join(map(str, vals)), 2))


@pytest.mark.parametrize("P", [4, 7])
def test_brute_force_random_odd_int8(P):
    rng = np.random.default_rng(100 + P)
    for _ in range(20):
        C = rng.integers(0, 37, size=(P, P)).astype(np.int32)
        _brute_compare(C, wl.INT8, in_slab=37 * P + 3, tgt_slab=37 * P + 5,
                       seed=int(rng.integers(1 << 30)))


# ------------------------------------------------------------------- special cases

@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_P1_is_identity(dtype):
    e = wl.ELEM_SIZE[dtype]
    for n in [0, 1, 5, 16, 33]:
        C = np.array([[n]], np.int32)
        st, inp, tgt, sig, rc = _run(C, 1, dtype, 40 * e, 48 * e, core_num=3)
        assert st == oracle.OK
        np.testing.assert_array_equal(tgt[: n * e], inp[: n * e])
        assert (tgt[n * e:] == wl.SENTINEL).all()
        assert rc[0, 0] == n
        assert sig.tolist() == [[1, 1, 1]]


@pytest.mark.parametrize("P,n", [(2, 3), (4, 16), (8, 5), (3, 7)])
def test_equal_counts_is_block_transpose(P, n):
    C = np.full((P, P), n, np.int32)
    slab = P * n * 4
    st, inp, tgt, _, _ = _run(C, P, wl.FP32, slab, slab)
    assert st == oracle.OK
    want = inp.reshape(P, P, n * 4).transpose(1, 0, 2).reshape(-1)
    np.testing.assert_array_equal(tgt, want)


def test_bmm_rs_a2a_page_example_layout():
    g = json.load(open(os.path.join(GOLDEN, "bmm_rs_a2a_example.json")))
    ep, tp, E, Cc, H = g["EP"], g["TP"], g["E"], g["C"], g["H"]
    Eop, Hot = E // ep, H // tp
    assert [Eop, ep * Cc] == g["x_shape_yshard0"][:2]
    assert g["y_shape_yshard0"] == [E, Cc, Hot]
    # Per source rank p: temp3 packed by destination, block for dst j is
    # (E/ep, C, H/tp) of values encoding (p, j, e, c, h).
    P = ep
    n = Eop * Cc * Hot
    vals = np.zeros((P, P, Eop, Cc, Hot), np.int64)
    for p, j, e, c, h in itertools.product(range(P), range(P), range(Eop), range(Cc), range(Hot)):
        vals[p, j, e, c, h] = (((p * P + j) * Eop + e) * Cc + c) * Hot + h
    inp = vals.astype(np.int32).view(np.uint8).reshape(-1).copy()
    slab = P * n * 4
    tgt = np.zeros(P * slab, np.uint8)
    sig = np.zeros((P, 1), np.int32)
    rc = np.zeros((P, P), np.int32)
    C = np.full((P, P), n, np.int32)
    assert oracle.run(inp, tgt, sig, C, rc, P=P, S=1, in_slab=slab, tgt_slab=slab,
                      core_num=1, dtype=wl.FP32) == oracle.OK
    y = tgt.view(np.int32).reshape(P, E, Cc, Hot)   # y on each destination rank: (E, C, H/tp)
    for d, p, e in itertools.product(range(P), range(P), range(Eop)):
        np.testing.assert_array_equal(y[d, p * Eop + e], vals[p, d, e].astype(np.int32))


@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_round_trip_with_transposed_counts(dtype):
    rng = np.random.default_rng(5)
    P = 6
    e = wl.ELEM_SIZE[dtype]
    C = rng.integers(0, 40, size=(P, P)).astype(np.int32)
    slab = 40 * P * e + 16
    st, inp, tgt, _, rc = _run(C, P, dtype, slab, slab)
    assert st == oracle.OK
    back = np.zeros(P * slab, np.uint8)
    sig = np.zeros((P, 1), np.int32)
    rc2 = np.zeros((P, P), np.int32)
    assert oracle.run(tgt, back, sig, np.ascontiguousarray(rc), rc2, P=P, S=1, in_slab=slab,
                      tgt_slab=slab, core_num=1, dtype=dtype) == oracle.OK
    for s in range(P):
        n = int(C[s].sum()) * e
        np.testing.assert_array_equal(back[s * slab:s * slab + n], inp[s * slab:s * slab + n])
    np.testing.assert_array_equal(rc2, C)


def test_byte_conservation():
    rng = np.random.default_rng(9)
    P = 9
    C = rng.integers(1, 30, size=(P, P)).astype(np.int32)
    slab = 30 * P * 4
    st, inp, tgt, _, _ = _run(C, P, wl.FP32, slab, slab)
    assert st == oracle.OK
    written = (tgt.reshape(P, slab) != wl.SENTINEL)
    # Every destination's received prefix is exactly its column sum; past it
    # the sentinel survives (random bytes can equal the sentinel, so compare
    # the prefix length from the right end only where it differs).
    for d in range(P):
        n = int(C[:, d].sum()) * 4
        assert not written[d, n:].any()
        assert written[d, :n].sum() >= n - (inp == wl.SENTINEL).sum()
    assert C.sum() * 4 == sum(int(C[:, d].sum()) * 4 for d in range(P))


def test_all_zero_counts():
    P = 5
    C = np.zeros((P, P), np.int32)
    st, inp, tgt, sig, rc = _run(C, P, wl.INT8, 32, 32, core_num=12, S=16)
    assert st == oracle.OK
    assert (tgt == wl.SENTINEL).all()
    assert (rc == 0).all()
    B = oracle.blocks(P, 12)
    assert B == 10
    assert (sig[:, :B] == 1).all() and (sig[:, B:] == 0).all()


def test_exact_capacity_and_one_over():
    P = 3
    C = np.array([[4, 0, 4], [0, 8, 0], [0, 0, 0]], np.int32)   # rows 8,8,0; cols 4,8,4
    st, inp, tgt, _, _ = _run(C, P, wl.FP32, in_slab=32, tgt_slab=32)
    assert st == oracle.OK
    C2 = C.copy()
    C2[2, 1] = 1                                                # column 1 -> 9 elems = 36 B
    st, _, tgt2, sig2, rc2 = _run(C2, P, wl.FP32, in_slab=32, tgt_slab=32)
    assert st == oracle.ERR_OVER_CAPACITY
    assert (tgt2 == wl.SENTINEL).all() and (sig2 == 0).all() and (rc2 == -7).all()


def test_signal_wraps_and_spares_columns_past_B():
    P = 4
    S = 8
    sig = np.full((P, S), 2**31 - 1, np.int32)
    sig[:, 6:] = 123
    C = np.ones((P, P), np.int32)
    st, _, _, sig_out, _ = _run(C, P, wl.INT8, 16, 16, core_num=6, S=S, signal=sig)
    B = oracle.blocks(P, 6)
    assert B == 4
    assert st == oracle.OK
    assert (sig_out[:, :B] == -2**31).all()
    assert (sig_out[:, B:6] == 2**31 - 1).all() and (sig_out[:, 6:] == 123).all()


# ------------------------------------------------------------------- diagnostics

def _buffers(P, S, in_slab, tgt_slab):
    return (np.zeros(P * in_slab, np.uint8), np.full(P * tgt_slab, wl.SENTINEL, np.uint8),
            np.zeros((P, S), np.int32), np.ones((P, P), np.int32), np.zeros((P, P), np.int32))


def _chk(bufs, P, S, in_slab, tgt_slab, core_num=1, dtype=wl.INT8, capacity=0, override=None):
    ptrs = [b.ctypes.data for b in bufs]
    if override:
        for i, v in override.items():
            ptrs[i] = v
    return oracle.check(*ptrs, P=P, S=S, in_slab=in_slab, tgt_slab=tgt_slab, core_num=core_num,
                        dtype=dtype, capacity=capacity)


def test_diagnostics_each_row():
    P, S = 4, 4
    b = _buffers(P, S, 16, 16)
    assert _chk(b, P, S, 16, 16) == oracle.OK
    for i in range(5):
        assert _chk(b, P, S, 16, 16, override={i: None}) == oracle.ERR_NULLPTR
    assert _chk(b, P, S, 16, 16, dtype=2) == oracle.ERR_UNSUPPORTED_DTYPE
    assert _chk(b, P, S, 16, 16, dtype=-1) == oracle.ERR_UNSUPPORTED_DTYPE
    b65 = _buffers(65, 1, 1, 1)
    assert _chk(b65, 65, 1, 1, 1) == oracle.ERR_INVALID_ARGS
    assert _chk(b, P, S, 16, 16, core_num=0) == oracle.ERR_INVALID_ARGS
    assert _chk(b, P, S, 16, 16, core_num=2**31) == oracle.ERR_INVALID_ARGS
    assert _chk(b, P, S, 16, 16, core_num=2**31 - 1) == oracle.ERR_INVALID_ARGS  # B huge > S
    assert _chk(b, P, S, 16, 16, core_num=5) == oracle.OK                         # B = 4 = S
    assert _chk(b, P, S, 16, 16, core_num=8) == oracle.ERR_INVALID_ARGS           # B = 8 > S
    # S >= B exactly ("Launch width": the signal holds a column per admitted
    # block): S = B passes, S = B - 1 does not.
    b7, b8 = list(_buffers(P, 7, 16, 16)), _buffers(P, 8, 16, 16)
    b7[2] = np.zeros(P * 8, np.int32)[:P * 7].reshape(P, 7)   # zeros past the last row too
    assert _chk(b7, P, 7, 16, 16, core_num=8) == oracle.ERR_INVALID_ARGS          # S = B - 1
    assert _chk(b8, P, 8, 16, 16, core_num=8) == oracle.OK                        # S = B
    bS = _buffers(P, 8, 16, 16)
    assert _chk(bS, P, 8, 16, 16, core_num=8, capacity=4) == oracle.ERR_LAUNCH_CAPACITY
    assert _chk(bS, P, 8, 16, 16, core_num=8, capacity=8) == oracle.OK
    assert _chk(bS, P, 8, 16, 16, core_num=1, capacity=0) == oracle.OK
    # Aliasing: target overlapping input, recv_counts overlapping send_counts.
    assert _chk(b, P, S, 16, 16, override={1: b[0].ctypes.data + 8}) == oracle.ERR_INVALID_ARGS
    assert _chk(b, P, S, 16, 16, override={4: b[3].ctypes.data + 4}) == oracle.ERR_INVALID_ARGS
    assert _chk(b, P, S, 16, 16, override={2: b[1].ctypes.data}) == oracle.ERR_INVALID_ARGS
    # Slab not a whole number of fp32 elements.
    b6 = _buffers(P, S, 18, 16)
    assert _chk(b6, P, S, 18, 16, dtype=wl.FP32) == oracle.ERR_INVALID_ARGS
    assert _chk(b6, P, S, 18, 16, dtype=wl.INT8) == oracle.OK
    # Negative count.
    bn = _buffers(P, S, 16, 16)
    bn[3][1, 2] = -1
    assert _chk(bn, P, S, 16, 16) == oracle.ERR_INVALID_ARGS
    # Over capacity: a row (column) of 4 ones is 16 bytes of fp32, 4 of int8.
    bo = _buffers(P, S, 12, 64)
    assert _chk(bo, P, S, 12, 64, dtype=wl.FP32) == oracle.ERR_OVER_CAPACITY
    assert _chk(bo, P, S, 12, 64, dtype=wl.INT8) == oracle.OK
    bo2 = _buffers(P, S, 64, 12)
    assert _chk(bo2, P, S, 64, 12, dtype=wl.FP32) == oracle.ERR_OVER_CAPACITY
    assert _chk(bo2, P, S, 64, 12, dtype=wl.INT8) == oracle.OK
    # Unequal signal inside [P, B]; outside B it does not matter.
    bs = _buffers(P, 8, 16, 16)
    bs[2][3, 3] = 1
    assert _chk(bs, P, 8, 16, 16, core_num=4) == oracle.ERR_INVALID_ARGS
    bs[2][3, 3] = 0
    bs[2][3, 5] = 9
    assert _chk(bs, P, 8, 16, 16, core_num=4) == oracle.OK


def test_adjacent_operands_are_distinct():
    # "Current limitations" asks for distinct windows: operands that touch
    # without sharing a byte are distinct, one shared byte is not.  The five
    # operands carved back to back from one allocation.
    P, S, slab = 4, 4, 16
    sizes = [P * slab, P * slab, P * S * 4, P * P * 4, P * P * 4]
    pool = np.zeros(sum(sizes) + 8, np.uint8)
    base = (pool.ctypes.data + 3) & ~3
    ptrs, at = [], base
    for n in sizes:
        ptrs.append(at)
        at += n
    counts = np.ones((P, P), np.int32)
    ctypes.memmove(ptrs[3], counts.ctypes.data, counts.nbytes)
    chk = lambda q: oracle.check(*q, P=P, S=S, in_slab=slab, tgt_slab=slab,  # noqa: E731
                                 core_num=1, dtype=wl.INT8, capacity=0)
    assert chk(ptrs) == oracle.OK
    for i in range(1, 5):                    # operand i moved one byte into operand i - 1
        q = list(ptrs)
        q[i] -= 1
        assert chk(q) == oracle.ERR_INVALID_ARGS, i


def test_diagnostics_precedence():
    P, S = 4, 4
    b = _buffers(P, S, 16, 16)
    b[3][0, 0] = -1                                     # negative count ...
    assert _chk(b, P, S, 16, 16, dtype=5) == oracle.ERR_UNSUPPORTED_DTYPE   # ... loses to dtype
    assert _chk(b, P, S, 16, 16, core_num=0) == oracle.ERR_INVALID_ARGS
    b[3][:] = 100                                       # over capacity and ...
    b[3][0, 0] = -1                                     # ... negative: negative wins
    assert _chk(b, P, S, 16, 16) == oracle.ERR_INVALID_ARGS
    b[3][0, 0] = 100
    b[2][0, 0] = 5                                      # over capacity and unequal signal
    assert _chk(b, P, S, 16, 16) == oracle.ERR_OVER_CAPACITY


def test_error_writes_nothing():
    P = 4
    C = np.full((P, P), 3, np.int32)
    C[1, 1] = -2
    st, _, tgt, sig, rc = _run(C, P, wl.FP32, 64, 64)
    assert st == oracle.ERR_INVALID_ARGS
    assert (tgt == wl.SENTINEL).all() and (sig == 0).all() and (rc == -7).all()


# ------------------------------------------------------------------- sampled view

def test_locate_agrees_with_brute():
    rng = np.random.default_rng(21)
    P = 5
    C = rng.integers(0, 9, size=(P, P)).astype(np.int32)
    in_slab, tgt_slab = 9 * P + 2, 9 * P + 4
    st, inp, tgt, _, _ = _run(C, P, wl.INT8, in_slab, tgt_slab)
    assert st == oracle.OK
    for d in range(P):
        for off in range(tgt_slab):
            src = locate.source_of(C, d, off, 1, in_slab)
            want = wl.SENTINEL if src is None else inp[src]
            assert tgt[d * tgt_slab + off] == want


# ------------------------------------------------------------------- generators

def test_splitmix64_published_vector():
    # splitmix64 from state 0: the first outputs of the published reference.
    w = wl.random_words_np(0, 0, 3)
    assert [int(x) for x in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_fill_random_torch_matches_numpy():
    import torch
    for n in [0, 1, 7, 8, 9, 1000, 4099]:
        t = torch.empty(n, dtype=torch.uint8)
        wl.fill_random_(t, 1234, chunk_words=64)
        np.testing.assert_array_equal(t.numpy(), wl.random_bytes_np(1234, 0, n))
    np.testing.assert_array_equal(wl.random_bytes_np(9, 5, 20), wl.random_bytes_np(9, 0, 25)[5:])


@pytest.mark.parametrize("dtype", [wl.BF16, wl.FP16])
def test_finite16_torch_matches_numpy(dtype):
    import torch
    n = 5000
    t = torch.empty(2 * n, dtype=torch.uint8)
    wl.fill_random_(t, 55)
    wl.finite16_(t, dtype, chunk=777)
    want = wl.finite16_from_words(wl.random_bytes_np(55, 0, 2 * n).view(np.uint16), dtype)
    np.testing.assert_array_equal(t.numpy().view(np.uint16), want)
    # Every mapped word is a finite, non-zero float of the type.
    f = want.view(np.float16).astype(np.float32) if dtype == wl.FP16 else \
        (want.astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(f).all() and (f != 0).all()


def test_bias_workload_shape():
    w = wl.bias_workload(wl.BF16)
    assert w.payload_bytes == 4 * 2**30 and w.elem == 2
    A, H = w.extra["nblk"], w.extra["hidden"]
    assert (w.counts % (A * H) == 0).all()
    assert w.extra["E_over_ep"] * w.extra["ep"] * w.extra["C"] * H == w.counts[0].sum()
    assert wl.bias_np(w, A, H).shape == (w.P, A, H) and wl.bias_np(w, A, H).dtype == np.float32
    w16 = wl.bias_workload(wl.FP16, scale=64)
    assert wl.bias_np(w16, A, H).dtype == np.uint16
    assert w.name.startswith("c5b_") and w16.name.startswith("c5h_")


def test_workload_shapes():
    w3 = wl.workload(3)
    assert w3.payload_bytes == 448 * 2**20
    assert (w3.counts.sum(axis=1) * 1 == w3.in_slab).all()          # exactly full rows
    assert w3.counts.sum(axis=0).max() <= w3.tgt_slab
    assert (w3.counts % 7168 == 0).all()
    share = w3.counts.sum(axis=0) / w3.counts.sum()
    assert share[0] > share[1] > share[7]                             # Zipf popularity
    w5 = wl.workload(5)
    assert w5.payload_bytes == 8 * 2**30
    w4 = wl.workload(4)
    assert (w4.counts == 0).sum() >= 205 and w4.counts.max() <= 2**19
    w2 = wl.workload(2)
    assert (w2.counts == 0).sum() >= 6


# ------------------------------------------------------------------- blocked exchange

def _run_blocked(C, P, dtype, in_slab, tgt_slab, nblk, core_num=1, seed=4):
    C = np.ascontiguousarray(C, np.int32)
    S = max(1, oracle.blocks(P, core_num))
    inp = wl.random_bytes_np(seed, 0, P * in_slab)
    tgt = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    sig = np.zeros((P, S), np.int32)
    rc = np.full((P, P), -7, np.int32)
    st = oracle.run_blocked(inp, tgt, sig, C, rc, P=P, S=S, in_slab=in_slab, tgt_slab=tgt_slab,
                            core_num=core_num, dtype=dtype, nblk=nblk)
    return st, inp, tgt, sig, rc


@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
def test_blocked_with_one_block_is_the_plain_exchange(dtype):
    rng = np.random.default_rng(31)
    P = 6
    e = wl.ELEM_SIZE[dtype]
    C = rng.integers(0, 50, size=(P, P)).astype(np.int32)
    slab = 50 * P * e + 24
    a = _run(C, P, dtype, slab, slab, core_num=4)
    b = _run_blocked(C, P, dtype, slab, slab, 1, core_num=4, seed=3)
    assert a[0] == b[0] == oracle.OK
    for x, y in zip(a[1:], b[1:]):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("P,A,Q", [(2, 3, 5), (4, 2, 8), (3, 4, 1), (8, 8, 3)])
def test_blocked_equal_counts_is_numpy_transpose(P, A, Q):
    # Source slab s viewed as (A, P, Q): expert block a, destination rows d.
    C = np.full((P, P), A * Q, np.int32)
    slab = P * A * Q * 4
    st, inp, tgt, _, _ = _run_blocked(C, P, wl.FP32, slab, slab, A)
    assert st == oracle.OK
    src = inp.view(np.int32).reshape(P, A, P, Q)
    want = src.transpose(2, 0, 1, 3).reshape(-1)
    np.testing.assert_array_equal(tgt.view(np.int32), want)


def test_blocked_cann_example_layout():
    g = json.load(open(os.path.join(GOLDEN, "bmm_rs_a2a_example.json")))
    ep, tp, E, Cc, H = g["EP"], g["TP"], g["E"], g["C"], g["H"]
    Eop, Hot = E // ep, H // tp
    P = ep
    # temp3 on source p in its own layout (E/ep, ep*C, H/tp), values encode (p, e, row, h).
    vals = np.zeros((P, Eop, ep * Cc, Hot), np.int64)
    for p_, e_, r_, h_ in itertools.product(range(P), range(Eop), range(ep * Cc), range(Hot)):
        vals[p_, e_, r_, h_] = ((p_ * Eop + e_) * ep * Cc + r_) * Hot + h_
    inp = vals.astype(np.int32).view(np.uint8).reshape(-1).copy()
    n = Eop * Cc * Hot
    slab = P * n * 4
    tgt = np.zeros(P * slab, np.uint8)
    sig = np.zeros((P, 1), np.int32)
    rc = np.zeros((P, P), np.int32)
    C = np.full((P, P), n, np.int32)
    assert oracle.run_blocked(inp, tgt, sig, C, rc, P=P, S=1, in_slab=slab, tgt_slab=slab,
                              core_num=1, dtype=wl.FP32, nblk=Eop) == oracle.OK
    y = tgt.view(np.int32).reshape(P, E, Cc, Hot)          # y on rank j: (E, C, H/tp)
    for j, p_, e_ in itertools.product(range(P), range(P), range(Eop)):
        want = vals[p_, e_, j * Cc:(j + 1) * Cc, :].astype(np.int32)
        np.testing.assert_array_equal(y[j, p_ * Eop + e_], want)


@pytest.mark.parametrize("dtype", [wl.FP32, wl.INT8])
@pytest.mark.parametrize("nblk", [2, 3])
def test_blocked_brute_force(dtype, nblk):
    rng = np.random.default_rng(nblk * 10 + dtype)
    e = wl.ELEM_SIZE[dtype]
    for P in (2, 3, 4):
        for _ in range(15):
            C = (rng.integers(0, 6, size=(P, P)) * nblk).astype(np.int32)
            in_slab = 6 * nblk * P * e + 3 * e
            tgt_slab = 6 * nblk * P * e + 5 * e
            st, inp, tgt, _, rc = _run_blocked(C, P, dtype, in_slab, tgt_slab, nblk,
                                               seed=int(rng.integers(1 << 30)))
            assert st == oracle.OK
            in_slabs = [bytes(inp[s * in_slab:(s + 1) * in_slab]) for s in range(P)]
            old = [bytes([wl.SENTINEL]) * tgt_slab for _ in range(P)]
            want = brute.exchange_blocked(in_slabs, old, C.tolist(), e, nblk)
            got = [bytes(tgt[d * tgt_slab:(d + 1) * tgt_slab]) for d in range(P)]
            assert got == want, (P, C.tolist())
            np.testing.assert_array_equal(rc, C.T)


def test_blocked_diagnostics():
    P = 4
    C = np.full((P, P), 6, np.int32)
    st, _, tgt, sig, rc = _run_blocked(C, P, wl.INT8, 64, 64, 4)     # 6 % 4 != 0
    assert st == oracle.ERR_INVALID_ARGS
    assert (tgt == wl.SENTINEL).all() and (sig == 0).all() and (rc == -7).all()
    st, *_ = _run_blocked(C, P, wl.INT8, 64, 64, 0)                   # nblk < 1
    assert st == oracle.ERR_INVALID_ARGS
    st, *_ = _run_blocked(C, P, wl.INT8, 64, 64, 3)                   # divides: fine
    assert st == oracle.OK
    C2 = C.copy()
    C2[0, 0] = -3                                                     # negative wins
    st, *_ = _run_blocked(C2, P, wl.INT8, 64, 64, 4)
    assert st == oracle.ERR_INVALID_ARGS
    C3 = np.full((P, P), 7, np.int32)                                 # 7 % 2 and over capacity
    st, *_ = _run_blocked(C3, P, wl.INT8, 16, 16, 2)
    assert st == oracle.ERR_INVALID_ARGS                              # divisibility first
    C4 = np.full((P, P), 8, np.int32)
    st, *_ = _run_blocked(C4, P, wl.INT8, 16, 16, 2)
    assert st == oracle.ERR_OVER_CAPACITY


# ------------------------------------------------------------------- fused bias Add

def _f32_test_patterns(seed):
    """binary32 bit patterns for the narrowing pins: random patterns of every
    exponent, exact ties, f32 subnormals, the 16-bit formats' overflow edges,
    the infinities and NaNs (quiet, signalling, all-ones fraction, both signs)."""
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, 2**32, 60000, dtype=np.uint64).astype(np.uint32)
    # every exponent field with random sign and fraction
    expo = (np.arange(256, dtype=np.uint32) << 23)[:, None] | \
        rng.integers(0, 2**23, (256, 40), dtype=np.uint32) | \
        (rng.integers(0, 2, (256, 40), dtype=np.uint32) << 31)
    ties_bf16 = np.concatenate([(np.arange(1, 300, dtype=np.uint32) << 16) | 0x8000,
                                (np.arange(1, 300, dtype=np.uint32) << 16) | 0x18000])
    ties_f16 = np.concatenate([
        ((np.arange(1, 300, dtype=np.float64) + 0.5) * 2.0 ** -24).astype(np.float32).view(np.uint32),
        (np.arange(1024, 1400, dtype=np.float64) + 0.5).astype(np.float32).view(np.uint32)])
    vals = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.0, 65519.99, 65520.0, 65535.0,
                     70000.0, 131008.0, -65520.0, -70000.0, 1e10, 3.0e38, 3.4028235e38,
                     6.1e-5, 5.96e-8, 2.98e-8, 2.9802322e-8, 1e-40, -1e-40],
                    np.float32).view(np.uint32)
    special = np.array([0x7F800000, 0xFF800000,                 # +-Inf
                        0x7FC00000, 0xFFC00000,                 # quiet NaNs
                        0x7F800001, 0xFF800001, 0x7FA00000,     # signalling NaNs
                        0x7FFFFFFF, 0xFFFFFFFF, 0x7FBFFFFF,     # all-ones fractions
                        0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00400000,  # subnormals
                        0x7F7FFFFF, 0xFF7FFFFF,                 # largest finite binary32
                        0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001,     # bf16 overflow edge
                        0x7F7E8000, 0xFF7F8000], np.uint32)
    return np.concatenate([rand, expo.ravel(), ties_bf16, ties_f16, vals, special])


def _assert_same_or_both_nan(got, want, is_nan):
    nan_g, nan_w = is_nan(got), is_nan(want)
    np.testing.assert_array_equal(nan_g, nan_w)
    np.testing.assert_array_equal(got[~nan_w], want[~nan_w])


def _bf16_is_nan(h):
    h = np.asarray(h, np.uint32)
    return ((h >> 7) & 0xFF == 0xFF) & (h & 0x7F != 0)


def _f16_is_nan(h):
    h = np.asarray(h, np.uint32)
    return ((h >> 10) & 0x1F == 0x1F) & (h & 0x3FF != 0)


def _f32_is_nan(u):
    u = np.asarray(u, np.uint32)
    return ((u >> 23) & 0xFF == 0xFF) & (u & 0x7FFFFF != 0)


def test_bf16_narrowing_matches_torch():
    # torch's CPU float32 -> bfloat16 rounds to nearest even, overflows to
    # infinity and returns a NaN for a NaN: the same results as IEEE 754's
    # rules applied to the bfloat16 layout (NaN-ness compared for NaNs).
    import torch
    bits = _f32_test_patterns(5)
    want = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    got = oracle.f32_to_bf16_array(bits)
    _assert_same_or_both_nan(got, want, _bf16_is_nan)
    # The named edges, stated: the largest finite bfloat16 is 0x7F7F; half an
    # ulp above it is a tie that rounds to the even neighbour, infinity.
    assert oracle.f32_to_bf16(0x7F7F7FFF) == 0x7F7F
    assert oracle.f32_to_bf16(0x7F7F8000) == 0x7F80
    assert oracle.f32_to_bf16(0xFF7F8000) == 0xFF80
    assert oracle.f32_to_bf16(0x7F800000) == 0x7F80 and oracle.f32_to_bf16(0xFF800000) == 0xFF80
    for nan in (0x7FFFFFFF, 0xFFFFFFFF, 0x7F800001, 0xFF800001):
        h = oracle.f32_to_bf16(nan)
        assert _bf16_is_nan(h) and (h >> 15) == (nan >> 31) and h & 0x40, hex(h)


def test_bf16_widening_exhaustive_against_torch():
    import torch
    halves = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(halves.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_to_f32_array(halves)
    _assert_same_or_both_nan(got, want.view(np.uint32), _f32_is_nan)


def test_f16_narrowing_matches_numpy():
    # numpy's float32 -> float16 follows IEEE 754: round to nearest even,
    # overflow to infinity, NaN to NaN (NaN-ness compared for NaNs).
    bits = _f32_test_patterns(6)
    with np.errstate(over="ignore", invalid="ignore"):
        want = bits.view(np.float32).astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16_array(bits)
    _assert_same_or_both_nan(got, want, _f16_is_nan)
    f = lambda v: oracle.f32_to_f16(int(np.array([v], np.float32).view(np.uint32)[0]))
    assert f(65504.0) == 0x7BFF and f(65519.0) == 0x7BFF    # largest finite binary16
    assert f(65520.0) == 0x7C00 and f(70000.0) == 0x7C00    # the tie and beyond: overflow
    assert f(131008.0) == 0x7C00 and f(-70000.0) == 0xFC00
    assert oracle.f32_to_f16(0x7F800000) == 0x7C00 and oracle.f32_to_f16(0xFF800000) == 0xFC00
    for nan in (0x7FFFFFFF, 0xFFFFFFFF, 0x7F800001, 0xFF800001):
        h = oracle.f32_to_f16(nan)
        assert _f16_is_nan(h) and (h >> 15) == (nan >> 31) and h & 0x200, hex(h)
    assert oracle.f32_to_f16(0x00000001) == 0 and oracle.f32_to_f16(0x80000001) == 0x8000


def test_f16_widening_exhaustive_against_numpy():
    halves = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = halves.view(np.float16).astype(np.float32).view(np.uint32)
    got = oracle.f16_to_f32_array(halves)
    _assert_same_or_both_nan(got, want, _f32_is_nan)
    # Non-NaN results are exact, and NaN keeps its sign and payload.
    assert oracle.f16_to_f32(0x7C00) == 0x7F800000 and oracle.f16_to_f32(0xFC00) == 0xFF800000
    assert oracle.f16_to_f32(0x7DFF) == 0x7F800000 | (0x1FF << 13)
    assert oracle.f16_to_f32(0xFFFF) == 0xFF800000 | (0x3FF << 13)


def _bias_case(P, nblk, hidden, rows, dtype, seed=3, bias=None, pad=32):
    rng = np.random.default_rng(seed)
    C = (rng.integers(0, rows + 1, size=(P, P)) * nblk * hidden).astype(np.int32)
    e = 2
    in_slab = int(C.sum(axis=1).max(initial=0)) * e + pad
    tgt_slab = int(C.sum(axis=0).max(initial=0)) * e + pad
    words = wl.random_bytes_np(seed + 100, 0, P * in_slab).view(np.uint16)
    inp = wl.finite16_from_words(words, dtype).view(np.uint8).copy()
    if bias is None:
        bias = wl.bias_values(seed + 200, P, nblk, hidden, dtype)
    return C, in_slab, tgt_slab, inp, np.ascontiguousarray(bias)


def _run_bias(C, P, in_slab, tgt_slab, inp, bias, dtype, nblk, hidden, core_num=1):
    S = max(1, oracle.blocks(P, core_num))
    tgt = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    sig = np.zeros((P, S), np.int32)
    rc = np.full((P, P), -7, np.int32)
    st = oracle.run_bias(inp, tgt, sig, np.ascontiguousarray(C, np.int32), rc, bias, P=P, S=S,
                         in_slab=in_slab, tgt_slab=tgt_slab, core_num=core_num, dtype=dtype,
                         nblk=nblk, hidden=hidden)
    return st, tgt, sig, rc


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_bias_of_negative_zero_is_the_blocked_exchange(dtype):
    # x + (-0) == x for every finite x, so the result is the blocked exchange
    # of the same bytes (an int8 exchange with counts doubled).
    P, nblk, hidden = 4, 3, 8
    negz = np.full((P, nblk, hidden), -0.0, np.float32) if dtype == oracle.BF16 else \
        np.full((P, nblk, hidden), 0x8000, np.uint16)
    C, in_slab, tgt_slab, inp, bias = _bias_case(P, nblk, hidden, 5, dtype, bias=negz)
    st, tgt, sig, rc = _run_bias(C, P, in_slab, tgt_slab, inp, bias, dtype, nblk, hidden)
    assert st == oracle.OK
    tgt2 = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    sig2 = np.zeros((P, 1), np.int32)
    rc2 = np.full((P, P), -7, np.int32)
    st2 = oracle.run_blocked(inp, tgt2, sig2, (C * 2).astype(np.int32), rc2, P=P, S=1,
                             in_slab=in_slab, tgt_slab=tgt_slab, core_num=1, dtype=oracle.INT8,
                             nblk=nblk)
    assert st2 == oracle.OK
    np.testing.assert_array_equal(tgt, tgt2)
    np.testing.assert_array_equal(rc, C.T)


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_bias_cann_flow_against_torch(dtype):
    # Equal counts: temp2 per source is (A, P*Cr, Hd); temp3 = temp2 + bias[s, a, None, :]
    # in fp32, rounded to the payload type by torch; y = permute to (P, P, A, Cr*Hd).
    import torch
    P, A, Cr, Hd = 4, 2, 3, 16
    C = np.full((P, P), A * Cr * Hd, np.int32)
    slab = P * A * Cr * Hd * 2
    words = wl.random_bytes_np(77, 0, P * slab).view(np.uint16)
    x16 = wl.finite16_from_words(words, dtype)
    bias = wl.bias_values(78, P, A, Hd, dtype)
    st, tgt, _, _ = _run_bias(C, P, slab, slab, x16.view(np.uint8).copy(), bias, dtype, A, Hd)
    assert st == oracle.OK
    tdt = torch.bfloat16 if dtype == oracle.BF16 else torch.float16
    x = torch.from_numpy(x16.view(np.int16)).view(tdt).float().view(P, A, P * Cr, Hd)
    if dtype == oracle.BF16:
        b = torch.from_numpy(bias)
    else:
        b = torch.from_numpy(bias.view(np.int16)).view(torch.float16).float()
    temp3 = (x + b.view(P, A, 1, Hd)).to(tdt)                    # (P, A, P*Cr, Hd)
    y = temp3.view(P, A, P, Cr * Hd).permute(2, 0, 1, 3).contiguous()
    want = y.view(torch.int16).numpy().reshape(-1).view(np.uint8)
    np.testing.assert_array_equal(tgt, want)


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_bias_every_ieee_class_against_torch(dtype):
    # [CANN]'s flow (fp32 add, round to the payload type, permute) computed by
    # torch on payloads and biases that reach every IEEE class: overflowing
    # sums (65504 + 65504 in FP16, the top binade of BF16 plus a large FP32
    # bias) become infinities, inf + (-inf) and any NaN operand give a NaN,
    # subnormals add exactly.  Non-NaN elements bit for bit; NaN elements
    # NaN on both sides.
    import torch
    P, A, Cr, Hd = 4, 2, 3, 64
    C = np.full((P, P), A * Cr * Hd, np.int32)
    slab = P * A * Cr * Hd * 2
    words = wl.random_bytes_np(91, 0, P * slab).view(np.uint16)
    x16 = wl.edge16_from_words(words, dtype)
    bias = wl.edge_bias_values(92, P, A, Hd, dtype)
    st, tgt, _, _ = _run_bias(C, P, slab, slab, x16.view(np.uint8).copy(), bias, dtype, A, Hd)
    assert st == oracle.OK
    tdt = torch.bfloat16 if dtype == oracle.BF16 else torch.float16
    x = torch.from_numpy(x16.view(np.int16)).view(tdt).float().view(P, A, P * Cr, Hd)
    if dtype == oracle.BF16:
        b = torch.from_numpy(bias)
    else:
        b = torch.from_numpy(bias.view(np.int16)).view(torch.float16).float()
    temp3 = (x + b.view(P, A, 1, Hd)).to(tdt)
    y = temp3.view(P, A, P, Cr * Hd).permute(2, 0, 1, 3).contiguous()
    want = y.view(torch.int16).numpy().reshape(-1).view(np.uint16)
    got = tgt.view(np.uint16)
    is_nan = _bf16_is_nan if dtype == oracle.BF16 else _f16_is_nan
    _assert_same_or_both_nan(got, want, is_nan)
    # The classes were all met: infinities from finite operands (overflow),
    # NaNs, subnormal results.
    xb = x.numpy()
    bb = np.broadcast_to(b.view(P, A, 1, Hd).numpy(), xb.shape)
    t3 = temp3.float().numpy()
    assert (np.isinf(t3) & np.isfinite(xb) & np.isfinite(bb)).any()
    assert np.isnan(t3).any()
    tiny = 2.0 ** -126 if dtype == oracle.BF16 else 2.0 ** -14
    assert ((t3 != 0) & (np.abs(t3) < tiny)).any()


def test_bias_diagnostics():
    P, nblk, hidden = 2, 2, 8
    C, in_slab, tgt_slab, inp, bias = _bias_case(P, nblk, hidden, 3, oracle.BF16, seed=9)
    st, *_ = _run_bias(C, P, in_slab, tgt_slab, inp, None, oracle.BF16, nblk, hidden)
    assert st == oracle.ERR_NULLPTR
    st, *_ = _run_bias(C, P, in_slab, tgt_slab, inp, bias, oracle.FP32, nblk, hidden)
    assert st == oracle.ERR_UNSUPPORTED_DTYPE
    st, *_ = _run_bias(C, P, in_slab, tgt_slab, inp, bias, oracle.BF16, nblk, 0)
    assert st == oracle.ERR_INVALID_ARGS
    C2 = C.copy()
    C2[0, 1] += nblk                                   # not whole rows of every sub-block
    st, tgt, sig, rc = _run_bias(C2, P, in_slab + 64, tgt_slab + 64,
                                 np.zeros(P * (in_slab + 64), np.uint8), bias, oracle.BF16,
                                 nblk, hidden)
    assert st == oracle.ERR_INVALID_ARGS
    assert (tgt == wl.SENTINEL).all() and (sig == 0).all() and (rc == -7).all()
    # The bias may not overlap another operand.
    st = oracle.run_bias(inp, np.zeros(P * tgt_slab, np.uint8), np.zeros((P, 1), np.int32),
                         C, np.zeros((P, P), np.int32), inp, P=P, S=1, in_slab=in_slab,
                         tgt_slab=tgt_slab, core_num=1, dtype=oracle.BF16, nblk=nblk,
                         hidden=hidden)
    assert st == oracle.ERR_INVALID_ARGS


# ------------------------------------------------------------ indexed exchange

def _run_indexed(inp, C, index, *, P, in_slab, tgt_slab, dtype, row_elems, stride,
                 core_num=1, signal=None):
    S = max(1, oracle.blocks(P, core_num))
    tgt = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    sig = np.zeros((P, S), np.int32) if signal is None else signal.copy()
    rc = np.full((P, P), -7, np.int32)
    st = oracle.run_indexed(inp, tgt, sig, np.ascontiguousarray(C, np.int32), rc,
                            None if index is None else np.ascontiguousarray(index, np.int32),
                            P=P, S=S, in_slab=in_slab, tgt_slab=tgt_slab, core_num=core_num,
                            dtype=dtype, row_elems=row_elems, index_stride=stride)
    return st, tgt, sig, rc


@pytest.mark.parametrize("dtype", [oracle.FP32, oracle.INT8])
def test_indexed_identity_index_is_the_plain_exchange(dtype):
    # index[s][k] = k on a packed input: the gather is the identity.
    rng = np.random.default_rng(31)
    P, R = 5, 3
    e = 4 if dtype == oracle.FP32 else 1
    C = (rng.integers(0, 7, size=(P, P)) * R).astype(np.int32)
    in_slab = int(C.sum(axis=1).max()) * e + 8 * e
    tgt_slab = int(C.sum(axis=0).max()) * e + 4 * e
    inp = wl.random_bytes_np(5, 0, P * in_slab)
    stride = int(C.sum(axis=1).max()) // R + 2
    index = np.tile(np.arange(stride, dtype=np.int32), (P, 1))
    st, tgt, sig, rc = _run_indexed(inp, C, index, P=P, in_slab=in_slab, tgt_slab=tgt_slab,
                                    dtype=dtype, row_elems=R, stride=stride, core_num=7)
    assert st == oracle.OK
    tgt2 = np.full(P * tgt_slab, wl.SENTINEL, np.uint8)
    sig2 = np.zeros_like(sig)
    rc2 = np.zeros((P, P), np.int32)
    assert oracle.run(inp, tgt2, sig2, C, rc2, P=P, S=sig.shape[1], in_slab=in_slab,
                      tgt_slab=tgt_slab, core_num=7, dtype=dtype) == oracle.OK
    np.testing.assert_array_equal(tgt, tgt2)
    np.testing.assert_array_equal(sig, sig2)
    np.testing.assert_array_equal(rc, C.T)


@pytest.mark.parametrize("P,R,dtype", [(1, 4, oracle.FP32), (2, 1, oracle.INT8),
                                       (4, 3, oracle.INT8), (7, 2, oracle.FP32)])
def test_indexed_numpy_gather_then_brute_force(P, R, dtype):
    # numpy fancy indexing builds each source's packed rows; the pure-Python
    # brute force then places them.  Repeats and arbitrary order in index.
    rng = np.random.default_rng(P * 10 + R)
    e = 4 if dtype == oracle.FP32 else 1
    rb = R * e
    table_rows = 11
    in_slab = table_rows * rb + 3 * e          # a partial row at the end is never named
    C = (rng.integers(0, 5, size=(P, P)) * R).astype(np.int32)
    rows = C.sum(axis=1) // R
    stride = int(rows.max()) + 3
    index = rng.integers(0, table_rows, size=(P, stride)).astype(np.int32)
    index[:, -1] = -99                         # entries past a source's rows are never read
    tgt_slab = int(C.sum(axis=0).max()) * e + 2 * e
    inp = wl.random_bytes_np(P + R, 0, P * in_slab)
    st, tgt, _, _ = _run_indexed(inp, C, index, P=P, in_slab=in_slab, tgt_slab=tgt_slab,
                                 dtype=dtype, row_elems=R, stride=stride)
    assert st == oracle.OK
    packed = []
    for s in range(P):
        table = inp[s * in_slab:s * in_slab + table_rows * rb].reshape(table_rows, rb)
        packed.append(table[index[s, :rows[s]]].tobytes())
    old = [bytes([wl.SENTINEL]) * tgt_slab] * P
    want = brute.exchange(packed, old, C.tolist(), e)
    assert tgt.tobytes() == b"".join(want)


def test_indexed_tiny_brute_force_every_count_matrix():
    import itertools
    P, R = 2, 2
    rb = R
    for flat in itertools.product([0, 2, 4], repeat=4):
        C = np.array(flat, np.int32).reshape(P, P)
        rows = C.sum(axis=1) // R
        stride = max(1, int(rows.max()))
        index = np.array([[(3 * s + k) % 3 for k in range(stride)] for s in range(P)], np.int32)
        in_slab = 3 * rb
        tgt_slab = 8 + 1
        inp = wl.random_bytes_np(sum(flat) + 1, 0, P * in_slab)
        st, tgt, sig, rc = _run_indexed(inp, C, index, P=P, in_slab=in_slab, tgt_slab=tgt_slab,
                                        dtype=oracle.INT8, row_elems=R, stride=stride)
        assert st == oracle.OK
        packed = [b"".join(inp[s * in_slab + index[s, k] * rb:s * in_slab + index[s, k] * rb + rb]
                           .tobytes() for k in range(rows[s])) for s in range(P)]
        want = brute.exchange(packed, [bytes([wl.SENTINEL]) * tgt_slab] * P, C.tolist(), 1)
        assert tgt.tobytes() == b"".join(want), flat
        np.testing.assert_array_equal(rc, C.T)
        assert (sig == 1).all()


def test_indexed_moe_dispatch_equals_the_packed_exchange():
    # The MoE dispatch from token tables and the routing's gather list gives
    # exactly what the plain exchange gives on c3's packed input, in which a
    # token routed to two ranks is stored twice.
    w3 = wl.workload(3, scale=64)
    wi = wl.indexed_workload(scale=64)
    np.testing.assert_array_equal(wi.counts, w3.counts)
    tgt3 = np.full(w3.tgt_bytes, wl.SENTINEL, np.uint8)
    sig3 = np.zeros((w3.P, w3.S), np.int32)
    rc3 = np.zeros((w3.P, w3.P), np.int32)
    assert oracle.run(wl.input_bytes_np(w3), tgt3, sig3, w3.counts, rc3, P=w3.P, S=w3.S,
                      in_slab=w3.in_slab, tgt_slab=w3.tgt_slab, core_num=w3.core_num,
                      dtype=w3.dtype) == oracle.OK
    st, tgt, sig, rc = _run_indexed(wl.input_bytes_np(wi), wi.counts, wi.extra["index"], P=wi.P,
                                    in_slab=wi.in_slab, tgt_slab=wi.tgt_slab, dtype=wi.dtype,
                                    row_elems=wi.extra["row_elems"],
                                    stride=wi.extra["index_stride"], core_num=wi.core_num)
    assert st == oracle.OK
    np.testing.assert_array_equal(tgt, tgt3)
    np.testing.assert_array_equal(sig, sig3)
    assert wi.in_slab * 2 == w3.in_slab                # half the input: no duplicated tokens


def test_indexed_diagnostics():
    P, R = 3, 2
    rng = np.random.default_rng(4)
    C = (rng.integers(1, 4, size=(P, P)) * R).astype(np.int32)
    rows = C.sum(axis=1) // R
    stride = int(rows.max())
    table_rows = 6
    in_slab, tgt_slab = table_rows * R * 4, int(C.sum(axis=0).max()) * 4
    inp = wl.random_bytes_np(1, 0, P * in_slab)
    index = rng.integers(0, table_rows, size=(P, stride)).astype(np.int32)
    kw = dict(P=P, in_slab=in_slab, tgt_slab=tgt_slab, dtype=oracle.FP32, row_elems=R,
              stride=stride)

    def status(C=C, index=index, **over):
        args = dict(kw)
        args.update(over)
        st, tgt, sig, rc = _run_indexed(inp[:P * args["in_slab"]].copy(), C, index, **args)
        if st != oracle.OK:
            assert (tgt == wl.SENTINEL).all() and (rc == -7).all() and (sig == 0).all()
        return st

    assert status() == oracle.OK
    assert status(index=None) == oracle.ERR_NULLPTR
    assert status(dtype=oracle.BF16) == oracle.ERR_UNSUPPORTED_DTYPE
    assert status(row_elems=0) == oracle.ERR_INVALID_ARGS
    assert status(stride=0, index=np.zeros((P, 1), np.int32)[:, :0].copy()) == oracle.ERR_INVALID_ARGS
    C2 = C.copy()
    C2[1, 2] += 1                                     # not whole rows
    assert status(C=C2) == oracle.ERR_INVALID_ARGS
    C3 = C.copy()
    C3[0, 0] = -2
    assert status(C=C3) == oracle.ERR_INVALID_ARGS
    C4 = C.copy()
    C4[0, 0] += 2 * R * (stride - rows[0] + 1)        # more rows than the index holds
    assert status(C=C4, tgt_slab=tgt_slab * 4) == oracle.ERR_OVER_CAPACITY
    assert status(tgt_slab=tgt_slab - 4) == oracle.ERR_OVER_CAPACITY
    for bad in (-1, table_rows):
        ix = index.copy()
        ix[2, rows[2] - 1] = bad
        assert status(index=ix) == oracle.ERR_INVALID_ARGS
    # Over capacity is reported before a bad index.
    ix = index.copy()
    ix[0, 0] = -1
    assert status(index=ix, tgt_slab=tgt_slab - 4) == oracle.ERR_OVER_CAPACITY
    # A partial row at the table's end cannot be named.
    assert status(in_slab=in_slab - 4, index=np.minimum(index, table_rows - 1)) in (
        oracle.OK, oracle.ERR_INVALID_ARGS)
    ix = index.copy()
    ix[1, 0] = table_rows - 1
    assert status(in_slab=in_slab - 4, index=ix) == oracle.ERR_INVALID_ARGS
    # The index may not overlap another operand.
    S = 1
    tgt = np.zeros(P * tgt_slab, np.uint8)
    st = oracle.run_indexed(inp, tgt, np.zeros((P, S), np.int32), C, np.zeros((P, P), np.int32),
                            tgt[:P * stride * 4].view(np.int32), P=P, S=S, in_slab=in_slab,
                            tgt_slab=tgt_slab, core_num=1, dtype=oracle.FP32, row_elems=R,
                            index_stride=stride)
    assert st == oracle.ERR_INVALID_ARGS
