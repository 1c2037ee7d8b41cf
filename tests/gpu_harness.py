"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
(via the Python binding) and the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from all_movement_amd import a2av
from all_movement_amd import workloads as wl

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


class Case:
    """Device and host copies of one exchange's operands."""

    def __init__(self, w: wl.Workload, *, input_np: np.ndarray | None = None,
                 host_input: bool = True, signal_np: np.ndarray | None = None,
                 in_offset: int = 0, tgt_offset: int = 0):
        self.w = w
        P = w.P
        if input_np is None and host_input:
            input_np = wl.input_bytes_np(w)
        if input_np is not None:
            # Optional byte offsets place the operands at unaligned addresses.
            buf = torch.empty(w.in_bytes + in_offset, dtype=torch.uint8, device=DEV)
            self.input = buf[in_offset:]
            self.input.copy_(upload(input_np))
            self.input_np = input_np
        else:
            self.input = wl.input_tensor(w, DEV)
            self.input_np = None
        tbuf = torch.empty(w.tgt_bytes + tgt_offset, dtype=torch.uint8, device=DEV)
        self.target = tbuf[tgt_offset:]
        self.target.fill_(wl.SENTINEL)
        sig = wl.signal_np(w) if signal_np is None else signal_np
        self.signal_np0 = sig.copy()
        self.signal = upload(sig)
        self.send = upload(w.counts)
        self.recv = torch.full((P, P), -7, dtype=torch.int32, device=DEV)

    def run_gpu(self, ex: a2av.Exchange, core_num: int | None = None, sync: bool = True,
                nblk: int = 1, bias=None, hidden: int = 0, index=None, row_elems: int = 0,
                host_counts: np.ndarray | None = None) -> int:
        w = self.w
        ex.run(self.input, self.target, self.signal, self.send, self.recv,
               w.core_num if core_num is None else core_num, w.dtype, nblk=nblk, bias=bias,
               hidden=hidden, index=index, row_elems=row_elems, host_counts=host_counts)
        if sync:
            torch.cuda.synchronize()
            return ex.query_error()
        return a2av.OK

    def run_oracle(self, core_num: int | None = None, capacity: int = 0, nblk: int = 1,
                   bias: np.ndarray | None = None, hidden: int = 0,
                   index: np.ndarray | None = None, row_elems: int = 0):
        w = self.w
        inp = self.input_np if self.input_np is not None else self.input.cpu().numpy()
        tgt = np.full(w.tgt_bytes, wl.SENTINEL, np.uint8)
        sig = self.signal_np0.copy()
        rc = np.full((w.P, w.P), -7, np.int32)
        kw = dict(P=w.P, S=w.S, in_slab=w.in_slab, tgt_slab=w.tgt_slab,
                  core_num=w.core_num if core_num is None else core_num, dtype=w.dtype,
                  capacity=capacity)
        C = np.ascontiguousarray(w.counts, np.int32)
        if index is not None:
            st = oracle.run_indexed(inp, tgt, sig, C, rc, np.ascontiguousarray(index, np.int32),
                                    row_elems=row_elems, index_stride=index.shape[1], **kw)
        elif bias is not None:
            st = oracle.run_bias(inp, tgt, sig, C, rc, np.ascontiguousarray(bias), nblk=nblk,
                                 hidden=hidden, **kw)
        elif nblk == 1:
            st = oracle.run(inp, tgt, sig, C, rc, **kw)
        else:
            st = oracle.run_blocked(inp, tgt, sig, C, rc, nblk=nblk, **kw)
        return st, tgt, sig, rc

    def assert_matches(self, st_gpu, expect):
        st, tgt, sig, rc = expect
        assert st_gpu == st, (a2av.a2av_status_string(st_gpu), a2av.a2av_status_string(st))
        got = self.target.cpu().numpy()
        if not np.array_equal(got, tgt):
            bad = np.nonzero(got != tgt)[0]
            raise AssertionError(f"{bad.size} target bytes differ; first at {bad[:8].tolist()} "
                                 f"(slab {bad[0] // self.w.tgt_slab}, offset "
                                 f"{bad[0] % self.w.tgt_slab})")
        np.testing.assert_array_equal(self.signal.cpu().numpy(), sig)
        np.testing.assert_array_equal(self.recv.cpu().numpy(), rc)


def exchange_for(w: wl.Workload, **kw) -> a2av.Exchange:
    return a2av.Exchange(w.P, w.in_slab, w.tgt_slab, w.S, device=0, **kw)


def check_case(w: wl.Workload, core_num: int | None = None, runs: int = 1, nblk: int = 1, **kw):
    """Run the GPU path ``runs`` times and the oracle as often; compare everything."""
    c = Case(w)
    ex = exchange_for(w, **kw)
    try:
        for _ in range(runs):
            st = c.run_gpu(ex, core_num, nblk=nblk)
        exp = None
        for _ in range(runs):
            exp = c.run_oracle(core_num, nblk=nblk)
            if runs > 1:
                c.signal_np0 = exp[2].copy()
        c.assert_matches(st, exp)
    finally:
        ex.close()
    return c
