"""GPU parity of the exchange with the bias Add fused in front (a2av_run_bias):
the tail of the CANN BatchMatMulReduceScatterAllToAll op, temp3 = temp2 + bias
then the AllToAll, for BF16 payloads with an FP32 bias and FP16 payloads with
an FP16 bias.  Bit-exact against the oracle's run_bias (each sum formed in
binary32 and rounded to nearest even)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from all_movement_amd import a2av  # noqa: E402
from all_movement_amd import workloads as wl  # noqa: E402
from tests.gpu_harness import DEV, Case, exchange_for, say  # noqa: E402

DTYPES = [wl.BF16, wl.FP16]


@pytest.fixture(autouse=True)
def _gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bias_case(P, nblk, hidden, rows, dtype, core_num=1, seed=1, pad=48, zero_frac=0.15):
    """Counts of whole rows of every sub-block (rows * nblk * hidden elements)."""
    rng = np.random.default_rng(seed)
    C = (rng.integers(0, rows + 1, size=(P, P)) * nblk * hidden).astype(np.int32)
    C[rng.random((P, P)) < zero_frac] = 0
    w = wl.custom(P, dtype, C, core_num=core_num, seed=seed + 11)
    w.in_slab += pad
    w.tgt_slab += pad + 16
    return w


def bias_of(w, nblk, hidden):
    return wl.bias_np(w, nblk, hidden), wl.bias_tensor(w, nblk, hidden, DEV)


def check_bias(w, nblk, hidden, runs=1, core_num=None, bias_np=None, **kw):
    c = Case(w, input_np=wl.input16_np(w))
    if bias_np is None:
        bn, bt = bias_of(w, nblk, hidden)
    else:
        bn = bias_np
        bt = torch.from_numpy(bn.view(np.float16) if w.dtype == wl.FP16 else bn).to(DEV)
    ex = exchange_for(w, **kw)
    try:
        for _ in range(runs):
            st = c.run_gpu(ex, core_num, nblk=nblk, bias=bt, hidden=hidden)
        exp = None
        for _ in range(runs):
            exp = c.run_oracle(core_num, nblk=nblk, bias=bn, hidden=hidden)
            c.signal_np0 = exp[2].copy()
        c.assert_matches(st, exp)
    finally:
        ex.close()
    return c


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [8, 24, 2048, 7168, 8200])
@pytest.mark.parametrize("P", [1, 3, 8, 32])
def test_bias_sweep(P, hidden, dtype):
    # Rows of at most 8192 elements give each thread a fixed column (7168 and
    # 24 leave some threads idle); 8200 takes the path whose column wraps
    # around the row from word to word.
    rows = max(1, {1: 40, 3: 30, 8: 12, 32: 3}[P] * 2048 // max(hidden, 2048)
               if hidden >= 2048 else {1: 900, 3: 400, 8: 120, 32: 20}[P])
    for nblk in [1, 3]:
        for L in sorted({1, 2 * P + 1, 256}):
            say("P", P, "hidden", hidden, "dtype", dtype, "nblk", nblk, "L", L)
            w = bias_case(P, nblk, hidden, rows, dtype, core_num=L, seed=P * 7 + nblk)
            check_bias(w, nblk, hidden)


@pytest.mark.parametrize("dtype", DTYPES)
def test_bias_two_runs_and_small_chunks(dtype):
    w = bias_case(4, 2, 40, 60, dtype, core_num=8, seed=5)
    say("two runs, chunk limit 4096 and 8208")
    check_bias(w, 2, 40, runs=2, chunk_limit_bytes=4096)
    check_bias(w, 2, 40, runs=1, chunk_limit_bytes=8208)


def test_bias_host_rejections():
    P, nblk, hidden = 4, 2, 16
    w = bias_case(P, nblk, hidden, 10, wl.BF16, core_num=4, seed=8)
    bn, bt = bias_of(w, nblk, hidden)
    c = Case(w, input_np=wl.input16_np(w))
    ex = exchange_for(w)
    try:
        def run(**kw):
            args = dict(nblk=nblk, bias=bt, hidden=hidden)
            args.update(kw)
            return c.run_gpu(ex, **args)
        with pytest.raises(ValueError, match="UNSUPPORTED_DTYPE"):   # plain exchange: fp32/int8 only
            ex.run(c.input, c.target, c.signal, c.send, c.recv, 4, wl.BF16)
        saved = c.w.dtype
        try:
            c.w.dtype = wl.FP32
            with pytest.raises(ValueError, match="UNSUPPORTED_DTYPE"):
                run(bias=torch.zeros(P * nblk * hidden, dtype=torch.float32, device=DEV))
        finally:
            c.w.dtype = saved
        st = a2av.a2av_run_bias(ex.h, c.input.data_ptr(), c.target.data_ptr(), c.signal.data_ptr(),
                                c.send.data_ptr(), c.recv.data_ptr(), None, P, 4, wl.BF16, nblk,
                                hidden, None)
        assert st == a2av.ERR_NULLPTR
        for nb, hd in [(nblk, 0), (0, hidden)]:
            st = a2av.a2av_run_bias(ex.h, c.input.data_ptr(), c.target.data_ptr(),
                                    c.signal.data_ptr(), c.send.data_ptr(), c.recv.data_ptr(),
                                    bt.data_ptr(), P, 4, wl.BF16, nb, hd, None)
            assert st == a2av.ERR_INVALID_ARGS
        # The bias may not overlap another operand (here: the target).
        st = a2av.a2av_run_bias(ex.h, c.input.data_ptr(), c.target.data_ptr(), c.signal.data_ptr(),
                                c.send.data_ptr(), c.recv.data_ptr(), c.target.data_ptr(), P, 4,
                                wl.BF16, nblk, hidden, None)
        assert st == a2av.ERR_INVALID_ARGS
        # Limits of the GPU path: rows of a multiple of 8 elements, 16-byte
        # aligned operands.  (The oracle has none of these limits.)
        with pytest.raises(ValueError, match="INVALID_ARGS"):
            run(bias=torch.zeros(P * nblk * 12, dtype=torch.float32, device=DEV), hidden=12)
        torch.cuda.synchronize()
        assert (c.target.cpu().numpy() == wl.SENTINEL).all()
        assert (c.signal.cpu().numpy() == 0).all()
    finally:
        ex.close()
    for off in [(2, 0), (0, 8)]:
        c2 = Case(w, input_np=wl.input16_np(w), in_offset=off[0], tgt_offset=off[1])
        ex2 = exchange_for(w)
        try:
            with pytest.raises(ValueError, match="INVALID_ARGS"):
                c2.run_gpu(ex2, nblk=nblk, bias=bt, hidden=hidden)
        finally:
            ex2.close()
    bt2 = torch.empty(P * nblk * hidden + 2, dtype=torch.float32, device=DEV)[2:]  # 8 B past 16
    bt2.copy_(bt.view(-1))
    c3 = Case(w, input_np=wl.input16_np(w))
    ex3 = exchange_for(w)
    try:
        with pytest.raises(ValueError, match="INVALID_ARGS"):
            c3.run_gpu(ex3, nblk=nblk, bias=bt2, hidden=hidden)
    finally:
        ex3.close()
    w5 = bias_case(P, nblk, hidden, 10, wl.BF16, core_num=4, seed=8)
    c5 = Case(w5, input_np=wl.input16_np(w5))
    ex5 = exchange_for(w5, chunk_limit_bytes=1000)                  # not a multiple of 16
    try:
        with pytest.raises(ValueError, match="INVALID_ARGS"):
            c5.run_gpu(ex5, nblk=nblk, bias=bt, hidden=hidden)
    finally:
        ex5.close()


@pytest.mark.parametrize("dtype", DTYPES)
def test_bias_device_rejections_match_oracle(dtype):
    P, nblk, hidden = 4, 2, 16
    base = bias_case(P, nblk, hidden, 10, dtype, core_num=4, seed=12, zero_frac=0.0)
    # A count that nblk divides but that is not whole rows of every sub-block.
    C = base.counts.copy()
    C[1, 2] += nblk
    w = wl.custom(P, dtype, C, core_num=4, seed=13)
    w.in_slab += 64
    w.tgt_slab += 64
    c = check_bias(w, nblk, hidden)
    assert (c.target.cpu().numpy() == wl.SENTINEL).all()
    # Over capacity: a column sum beyond the target slab.
    w2 = wl.custom(P, dtype, base.counts, core_num=4, seed=14,
                   tgt_slab=int(base.counts.sum(axis=0).max()) * 2 - 16)
    w2.tgt_slab -= w2.tgt_slab % 16
    check_bias(w2, nblk, hidden)


def _is_nan16(h: np.ndarray, dtype: int) -> np.ndarray:
    h = h.astype(np.uint32)
    if dtype == wl.BF16:
        return ((h >> 7) & 0xFF == 0xFF) & (h & 0x7F != 0)
    return ((h >> 10) & 0x1F == 0x1F) & (h & 0x3FF != 0)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("P,hidden", [(3, 24), (8, 2048), (2, 8200)])
def test_bias_every_ieee_class(P, hidden, dtype):
    # Payloads and biases that reach every IEEE class: sums that overflow to
    # infinity (65504 + 65504 in FP16; the top BF16 binade plus a large FP32
    # bias), infinities of both signs, inf + (-inf), NaN operands (quiet,
    # signalling, all-ones fractions), subnormals and zeros.  Against the
    # oracle: every element bit for bit where the oracle's result is not a
    # NaN, a NaN where it is (IEEE 754 leaves the NaN's payload open); the
    # sentinel tails, the signal and recv_counts exactly.
    nblk = 2
    rows = 6 if hidden >= 2048 else 40
    w = bias_case(P, nblk, hidden, rows, dtype, core_num=2 * P, seed=31 + P)
    x = wl.edge16_from_words(wl.random_bytes_np(w.payload_seed, 0, w.in_bytes).view(np.uint16),
                             dtype)
    bn = wl.edge_bias_values(w.payload_seed + 7, P, nblk, hidden, dtype)
    bt = torch.from_numpy(bn.view(np.float16) if dtype == wl.FP16 else bn).to(DEV)
    c = Case(w, input_np=x.view(np.uint8))
    ex = exchange_for(w)
    try:
        say("P", P, "hidden", hidden, "dtype", dtype, "payload", w.payload_bytes)
        st = c.run_gpu(ex, nblk=nblk, bias=bt, hidden=hidden)
    finally:
        ex.close()
    st_o, tgt_o, sig_o, rc_o = c.run_oracle(nblk=nblk, bias=bn, hidden=hidden)
    assert st == st_o == a2av.OK
    got = c.target.cpu().numpy().view(np.uint16)
    want = tgt_o.view(np.uint16)
    nan_w = _is_nan16(want, dtype)
    np.testing.assert_array_equal(_is_nan16(got, dtype), nan_w)
    bad = np.nonzero(got[~nan_w] != want[~nan_w])[0]
    assert bad.size == 0, (bad.size, [hex(v) for v in got[~nan_w][bad[:4]]],
                           [hex(v) for v in want[~nan_w][bad[:4]]])
    np.testing.assert_array_equal(c.signal.cpu().numpy(), sig_o)
    np.testing.assert_array_equal(c.recv.cpu().numpy(), rc_o)
    assert nan_w.any() and (want == (0x7C00 if dtype == wl.FP16 else 0x7F80)).any()


def _row_expected(x_row: np.ndarray, b_row: np.ndarray, dtype: int) -> np.ndarray:
    """One row plus its bias by the oracle: a one-rank, one-row exchange."""
    H = b_row.size
    out = np.zeros(2 * H, np.uint8)
    st = oracle.run_bias(np.ascontiguousarray(x_row), out, np.zeros((1, 1), np.int32),
                         np.array([[H]], np.int32), np.zeros((1, 1), np.int32),
                         np.ascontiguousarray(b_row.reshape(1, 1, H)), P=1, S=1,
                         in_slab=2 * H, tgt_slab=2 * H, core_num=1, dtype=dtype, nblk=1,
                         hidden=H)
    assert st == oracle.OK
    return out


@pytest.mark.parametrize("dtype", DTYPES)
def test_bias_workload_scaled_full_oracle(dtype):
    # The full-size workload's shape at 1/16: (E/ep=8, ep*C=8*128, H/tp=2048).
    w = wl.bias_workload(dtype, scale=16)
    A, H = w.extra["nblk"], w.extra["hidden"]
    say(w.name, "scale 1/16", w.payload_bytes)
    check_bias(w, A, H)


@pytest.mark.parametrize("dtype", DTYPES)
def test_bias_workload_full_size(dtype):
    # 4 GiB of BF16 payload with the FP32 bias, or of FP16 payload with the
    # FP16 bias, in the launch configuration the benchmark times.  Checked
    # three ways: sampled rows against the oracle one row at a time; every
    # element against torch's own fp32 add and round-to-nearest-even cast to
    # the payload type; counts and flags.
    w = wl.bias_workload(dtype)
    P, A, H, Cn = w.P, w.extra["nblk"], w.extra["hidden"], w.extra["C"]
    say(w.name, w.payload_bytes)
    inp = wl.input16_tensor(w, DEV)
    tgt = torch.full((w.tgt_bytes,), wl.SENTINEL, dtype=torch.uint8, device=DEV)
    sig = torch.zeros((P, w.S), dtype=torch.int32, device=DEV)
    sc = torch.from_numpy(w.counts).to(DEV)
    rc = torch.zeros((P, P), dtype=torch.int32, device=DEV)
    bn, bt = bias_of(w, A, H)
    ex = exchange_for(w)
    try:
        ex.run(inp, tgt, sig, sc, rc, w.core_num, w.dtype, nblk=A, bias=bt, hidden=H)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK
    finally:
        ex.close()
    np.testing.assert_array_equal(rc.cpu().numpy(), w.counts.T)
    assert (sig.cpu().numpy() == 1).all()
    rng = np.random.default_rng(2024)
    row = 2 * H
    for _ in range(48):
        d, s, a, r = (int(rng.integers(0, P)), int(rng.integers(0, P)), int(rng.integers(0, A)),
                      int(rng.integers(0, Cn)))
        src = s * w.in_slab + ((a * P + d) * Cn + r) * row
        dst = d * w.tgt_slab + ((s * A + a) * Cn + r) * row
        x_row = wl.finite16_from_words(
            wl.random_bytes_np(w.payload_seed, src, row).view(np.uint16), w.dtype).view(np.uint8)
        np.testing.assert_array_equal(inp[src:src + row].cpu().numpy(), x_row)
        want = _row_expected(x_row, bn[s, a], w.dtype)
        got = tgt[dst:dst + row].cpu().numpy()
        assert np.array_equal(got, want), (d, s, a, r)
    tdt = torch.bfloat16 if dtype == wl.BF16 else torch.float16
    x = inp.view(tdt).view(P, A, P, Cn, H)
    y = tgt.view(tdt).view(P, P, A, Cn, H)
    bf = bt.float().view(P, A, 1, H)
    for d in range(P):
        want = (x[:, :, d].float() + bf).to(tdt)
        assert torch.equal(y[d].view(torch.int16), want.view(torch.int16)), d


def test_bias_negative_zero_is_the_permute_fp16_full_size():
    # x + (-0) == x: with a -0 bias the FP16 run is the blocked exchange, which
    # for equal counts is the permute (P, A, P, Q) -> (P, P, A, Q).
    w = wl.bias_workload(wl.FP16)
    P, A, H = w.P, w.extra["nblk"], w.extra["hidden"]
    Q = int(w.counts[0, 0]) // A
    inp = wl.input16_tensor(w, DEV)
    tgt = torch.full((w.tgt_bytes,), wl.SENTINEL, dtype=torch.uint8, device=DEV)
    sig = torch.zeros((P, w.S), dtype=torch.int32, device=DEV)
    sc = torch.from_numpy(w.counts).to(DEV)
    rc = torch.zeros((P, P), dtype=torch.int32, device=DEV)
    negz = torch.full((P, A, H), -0.0, dtype=torch.float16, device=DEV)
    ex = exchange_for(w)
    try:
        ex.run(inp, tgt, sig, sc, rc, w.core_num, w.dtype, nblk=A, bias=negz, hidden=H)
        torch.cuda.synchronize()
        assert ex.query_error() == a2av.OK
    finally:
        ex.close()
    src = inp.view(torch.int16).view(P, A, P, Q)
    dst = tgt.view(torch.int16).view(P, P, A, Q)
    for d in range(P):
        assert torch.equal(dst[d], src[:, :, d, :]), d
    assert (sig.cpu().numpy() == 1).all()
