"""Python binding of the all_to_all_v C ABI (include/a2av.h).

Argument marshalling only: every step of the exchange runs in the HIP
library ``liba2av.so`` built in this directory.  The functions below carry
the C names; :class:`Exchange` wraps them for torch tensors (torch provides
device memory and streams, nothing else).  The binding never converts or
copies a tensor: it passes ``data_ptr()`` after checking device, dtype, size
and contiguity, so a tensor that would need a copy is refused rather than
silently duplicated.

If the library is missing, loading raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liba2av.so")

OK = 0
ERR_NULLPTR = 1
ERR_INVALID_ARGS = 2
ERR_UNSUPPORTED_DTYPE = 3
ERR_OVER_CAPACITY = 4
ERR_LAUNCH_CAPACITY = 5
ERR_HIP = 6
ERR_TIMEOUT = 7

FP32 = 0
INT8 = 1
FP16 = 2
BF16 = 3
ELEM_SIZE = {FP32: 4, INT8: 1, FP16: 2, BF16: 2}
FLAG_PROFILE = 1
FLAG_NO_BLOCK_WAIT = 2

EXPORTS = ["a2av_create", "a2av_run", "a2av_run_blocked", "a2av_run_bias", "a2av_run_indexed",
           "a2av_run_noalloc", "a2av_run_host_counts", "a2av_check_host_counts",
           "a2av_run_blocked_host_counts", "a2av_run_bias_host_counts",
           "a2av_run_indexed_host_counts", "a2av_check_host_counts_ex",
           "a2av_check_bias_args", "a2av_check_indexed_args", "a2av_destroy",
           "a2av_blocks", "a2av_check_args", "a2av_query_error", "a2av_launch_info_get", "a2av_profile_read",
           "a2av_profile_sample", "a2av_status_string", "a2av_last_hip_error"]


# Probes (include/a2av_probe.h): measurement of the copy kernel's
# instructions alone and of the cooperative launch's own cost, not part of
# the exchange.
PROBE_READ = 0
PROBE_WRITE = 1
PROBE_COPY = 2
PROBE_EXPORTS = ["a2av_probe_stream", "a2av_probe_launch"]


class a2av_config(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("P", ctypes.c_int32),
                ("in_slab_bytes", ctypes.c_int64), ("tgt_slab_bytes", ctypes.c_int64),
                ("S", ctypes.c_int32), ("wg_per_block", ctypes.c_int32),
                ("chunk_limit_bytes", ctypes.c_int64), ("capacity_override", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("spin_limit", ctypes.c_int32)]


class a2av_launch_info(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_int64), ("wg_per_block", ctypes.c_int32),
                ("workgroups", ctypes.c_int32), ("threads_per_wg", ctypes.c_int32),
                ("chunk_launches", ctypes.c_int32), ("chunk_limit_bytes", ctypes.c_int64),
                ("capacity", ctypes.c_int64), ("cooperative", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load liba2av.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(or python all_movement_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    cfgp = ctypes.POINTER(a2av_config)
    L.a2av_create.argtypes = [ctypes.POINTER(vp), cfgp]
    L.a2av_create.restype = ctypes.c_int
    L.a2av_run.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, vp]
    L.a2av_run.restype = ctypes.c_int
    L.a2av_run_blocked.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp]
    L.a2av_run_blocked.restype = ctypes.c_int
    L.a2av_run_bias.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, vp]
    L.a2av_run_bias.restype = ctypes.c_int
    L.a2av_run_indexed.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i64, vp]
    L.a2av_run_indexed.restype = ctypes.c_int
    L.a2av_run_host_counts.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, vp]
    L.a2av_run_host_counts.restype = ctypes.c_int
    L.a2av_check_host_counts.argtypes = [cfgp, vp, i32, ctypes.POINTER(i64), ctypes.POINTER(i32)]
    L.a2av_check_host_counts.restype = ctypes.c_int
    L.a2av_run_blocked_host_counts.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp]
    L.a2av_run_blocked_host_counts.restype = ctypes.c_int
    L.a2av_run_bias_host_counts.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                            i32, vp]
    L.a2av_run_bias_host_counts.restype = ctypes.c_int
    L.a2av_run_indexed_host_counts.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                               i64, vp]
    L.a2av_run_indexed_host_counts.restype = ctypes.c_int
    L.a2av_check_host_counts_ex.argtypes = [cfgp, vp, i32, i64, i64, ctypes.POINTER(i64),
                                            ctypes.POINTER(i32)]
    L.a2av_check_host_counts_ex.restype = ctypes.c_int
    L.a2av_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i32, i64, i32, vp]
    L.a2av_run_noalloc.restype = ctypes.c_int
    L.a2av_probe_stream.argtypes = [i32, vp, vp, i64, i32, vp]
    L.a2av_probe_stream.restype = ctypes.c_int
    L.a2av_probe_launch.argtypes = [i32, vp, i64, i32, vp]
    L.a2av_probe_launch.restype = ctypes.c_int
    L.a2av_destroy.argtypes = [vp]
    L.a2av_destroy.restype = ctypes.c_int
    L.a2av_blocks.argtypes = [i64, i64]
    L.a2av_blocks.restype = i64
    L.a2av_check_args.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, i32, i64, i32]
    L.a2av_check_args.restype = ctypes.c_int
    L.a2av_check_bias_args.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32]
    L.a2av_check_bias_args.restype = ctypes.c_int
    L.a2av_check_indexed_args.argtypes = [cfgp, i64, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                          i64]
    L.a2av_check_indexed_args.restype = ctypes.c_int
    L.a2av_query_error.argtypes = [vp]
    L.a2av_query_error.restype = ctypes.c_int
    L.a2av_launch_info_get.argtypes = [vp, i64, ctypes.POINTER(a2av_launch_info)]
    L.a2av_launch_info_get.restype = ctypes.c_int
    L.a2av_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32),
                                    ctypes.POINTER(i32)]
    L.a2av_profile_read.restype = ctypes.c_int
    L.a2av_profile_sample.argtypes = [vp, i32]
    L.a2av_profile_sample.restype = ctypes.c_int
    L.a2av_status_string.argtypes = [ctypes.c_int]
    L.a2av_status_string.restype = ctypes.c_char_p
    L.a2av_last_hip_error.argtypes = [vp]
    L.a2av_last_hip_error.restype = ctypes.c_char_p
    _lib = L
    return L


# ---------------------------------------------------------------- C names

def a2av_create(cfg: a2av_config) -> tuple[int, int | None]:
    h = ctypes.c_void_p()
    st = lib().a2av_create(ctypes.byref(h), ctypes.byref(cfg))
    return st, h.value


def a2av_run(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype,
             stream) -> int:
    return lib().a2av_run(h, input, target, signal, send_counts, recv_counts, P, core_num,
                          dtype, stream)


def a2av_run_blocked(h, input, target, signal, send_counts, recv_counts, P, core_num, dtype,
                     nblk, stream) -> int:
    return lib().a2av_run_blocked(h, input, target, signal, send_counts, recv_counts, P,
                                  core_num, dtype, nblk, stream)


def a2av_run_bias(h, input, target, signal, send_counts, recv_counts, bias, P, core_num, dtype,
                  nblk, hidden, stream) -> int:
    return lib().a2av_run_bias(h, input, target, signal, send_counts, recv_counts, bias, P,
                               core_num, dtype, nblk, hidden, stream)


def a2av_run_indexed(h, input, target, signal, send_counts, recv_counts, index, P, core_num,
                     dtype, row_elems, index_stride, stream) -> int:
    return lib().a2av_run_indexed(h, input, target, signal, send_counts, recv_counts, index, P,
                                  core_num, dtype, row_elems, index_stride, stream)


def a2av_run_host_counts(h, input, target, signal, send_counts, recv_counts, host_send_counts,
                         P, core_num, dtype, stream) -> int:
    return lib().a2av_run_host_counts(h, input, target, signal, send_counts, recv_counts,
                                      host_send_counts, P, core_num, dtype, stream)


def a2av_run_blocked_host_counts(h, input, target, signal, send_counts, recv_counts,
                                 host_send_counts, P, core_num, dtype, nblk, stream) -> int:
    return lib().a2av_run_blocked_host_counts(h, input, target, signal, send_counts, recv_counts,
                                              host_send_counts, P, core_num, dtype, nblk, stream)


def a2av_run_bias_host_counts(h, input, target, signal, send_counts, recv_counts, bias,
                              host_send_counts, P, core_num, dtype, nblk, hidden, stream) -> int:
    return lib().a2av_run_bias_host_counts(h, input, target, signal, send_counts, recv_counts,
                                           bias, host_send_counts, P, core_num, dtype, nblk,
                                           hidden, stream)


def a2av_run_indexed_host_counts(h, input, target, signal, send_counts, recv_counts, index,
                                 host_send_counts, P, core_num, dtype, row_elems, index_stride,
                                 stream) -> int:
    return lib().a2av_run_indexed_host_counts(h, input, target, signal, send_counts, recv_counts,
                                              index, host_send_counts, P, core_num, dtype,
                                              row_elems, index_stride, stream)


def _host_ptr(host_send_counts):
    import numpy as np
    if isinstance(host_send_counts, np.ndarray):
        if host_send_counts.dtype != np.int32 or not host_send_counts.flags.c_contiguous:
            raise ValueError("host_send_counts must be a contiguous int32 array")
        return host_send_counts.ctypes.data
    return host_send_counts


def a2av_check_host_counts(cfg: a2av_config, host_send_counts, dtype) -> tuple[int, int, int]:
    """(status, payload bytes, chunk launches); host_send_counts is an int32
    numpy array [P, P] (or a raw host address)."""
    payload, launches = ctypes.c_int64(), ctypes.c_int32()
    st = lib().a2av_check_host_counts(ctypes.byref(cfg), _host_ptr(host_send_counts), dtype,
                                      ctypes.byref(payload), ctypes.byref(launches))
    return st, payload.value, launches.value


def a2av_check_host_counts_ex(cfg: a2av_config, host_send_counts, dtype, unit: int,
                              index_stride: int) -> tuple[int, int, int]:
    """a2av_check_host_counts for every exchange: (status, payload bytes,
    chunk launches) with counts in multiples of ``unit`` and, when
    ``index_stride`` > 0, the indexed exchange's row limit."""
    payload, launches = ctypes.c_int64(), ctypes.c_int32()
    st = lib().a2av_check_host_counts_ex(ctypes.byref(cfg), _host_ptr(host_send_counts), dtype,
                                         unit, index_stride, ctypes.byref(payload),
                                         ctypes.byref(launches))
    return st, payload.value, launches.value


def a2av_run_noalloc(input, target, signal, send_counts, recv_counts, status, P, in_slab_bytes,
                     tgt_slab_bytes, S, core_num, dtype, stream) -> int:
    return lib().a2av_run_noalloc(input, target, signal, send_counts, recv_counts, status, P,
                                  in_slab_bytes, tgt_slab_bytes, S, core_num, dtype, stream)


def a2av_probe_stream(kind, src, dst, nbytes, workgroups, stream) -> int:
    return lib().a2av_probe_stream(kind, src, dst, nbytes, workgroups, stream)


def a2av_probe_launch(cooperative, dst, nbytes, workgroups, stream) -> int:
    return lib().a2av_probe_launch(cooperative, dst, nbytes, workgroups, stream)


def a2av_destroy(h) -> int:
    return lib().a2av_destroy(h)


def a2av_blocks(P: int, L: int) -> int:
    return int(lib().a2av_blocks(P, L))


def a2av_check_args(cfg: a2av_config, capacity, input, target, signal, send_counts,
                    recv_counts, P, core_num, dtype) -> int:
    return lib().a2av_check_args(ctypes.byref(cfg), capacity, input, target, signal,
                                 send_counts, recv_counts, P, core_num, dtype)


def a2av_check_bias_args(cfg: a2av_config, capacity, input, target, signal, send_counts,
                         recv_counts, bias, P, core_num, dtype, nblk, hidden) -> int:
    return lib().a2av_check_bias_args(ctypes.byref(cfg), capacity, input, target, signal,
                                      send_counts, recv_counts, bias, P, core_num, dtype, nblk,
                                      hidden)


def a2av_check_indexed_args(cfg: a2av_config, capacity, input, target, signal, send_counts,
                            recv_counts, index, P, core_num, dtype, row_elems,
                            index_stride) -> int:
    return lib().a2av_check_indexed_args(ctypes.byref(cfg), capacity, input, target, signal,
                                         send_counts, recv_counts, index, P, core_num, dtype,
                                         row_elems, index_stride)


def a2av_query_error(h) -> int:
    return lib().a2av_query_error(h)


def a2av_launch_info_get(h, core_num: int) -> tuple[int, a2av_launch_info]:
    info = a2av_launch_info()
    st = lib().a2av_launch_info_get(h, core_num, ctypes.byref(info))
    return st, info


def a2av_profile_read(h) -> tuple[int, float, float, int, int]:
    k1, k2 = ctypes.c_double(), ctypes.c_double()
    n, runs = ctypes.c_int32(), ctypes.c_int32()
    st = lib().a2av_profile_read(h, ctypes.byref(k1), ctypes.byref(k2), ctypes.byref(n),
                                 ctypes.byref(runs))
    return st, k1.value, k2.value, n.value, runs.value


def a2av_profile_sample(h, every: int) -> int:
    return lib().a2av_profile_sample(h, every)


def a2av_status_string(status: int) -> str:
    return lib().a2av_status_string(status).decode()


def a2av_last_hip_error(h) -> str:
    return lib().a2av_last_hip_error(h).decode()


# ---------------------------------------------------------------- torch wrapper

class A2avError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {a2av_status_string(status)}")


def _raise(status: int, what: str, h=None):
    if status == OK:
        return
    msg = what
    if status == ERR_HIP and h is not None:
        msg += f" ({a2av_last_hip_error(h)})"
    if status in (ERR_NULLPTR, ERR_INVALID_ARGS, ERR_UNSUPPORTED_DTYPE, ERR_OVER_CAPACITY,
                  ERR_LAUNCH_CAPACITY):
        raise ValueError(f"{msg}: {a2av_status_string(status)}")
    raise A2avError(status, msg)


class Exchange:
    """A handle for one geometry: P virtual ranks, slab sizes and signal stride.

    ``run`` takes torch tensors: ``input`` (uint8 view of P*in_slab bytes, or
    any dtype of that many bytes), ``target`` likewise for P*tgt_slab bytes,
    ``signal`` int32 [P, S], ``send_counts`` / ``recv_counts`` int32 [P, P], all
    contiguous on the handle's device.
    """

    def __init__(self, P: int, in_slab_bytes: int, tgt_slab_bytes: int, S: int, *,
                 device: int | None = None, wg_per_block: int = 0, chunk_limit_bytes: int = 0,
                 capacity_override: int = 0, profile: bool = False, spin_limit: int = 0,
                 block_wait: bool = True):
        import torch
        if device is None:
            device = torch.cuda.current_device()
        self.device = int(device)
        self.cfg = a2av_config(self.device, P, in_slab_bytes, tgt_slab_bytes, S, wg_per_block,
                               chunk_limit_bytes, capacity_override,
                               (FLAG_PROFILE if profile else 0) |
                               (0 if block_wait else FLAG_NO_BLOCK_WAIT), spin_limit)
        st, h = a2av_create(self.cfg)
        _raise(st, "a2av_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            a2av_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, t, nbytes: int, name: str, dtype=None):
        import torch
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device.type != "cuda" or t.device.index != self.device:
            raise ValueError(f"{name} must live on cuda:{self.device}, not {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (the exchange never copies operands)")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if t.numel() * t.element_size() != nbytes:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, expected {nbytes}")
        return t.data_ptr()

    def run(self, input, target, signal, send_counts, recv_counts, core_num: int, dtype: int,
            stream=None, nblk: int = 1, bias=None, hidden: int = 0, index=None,
            row_elems: int = 0, check: bool = False, host_counts=None) -> None:
        """One exchange; ``nblk`` > 1 runs the blocked exchange (a2av_run_blocked);
        a ``bias`` tensor (float32 for BF16 payloads, float16 for FP16, [P, nblk,
        hidden] elements) runs the exchange with the bias Add fused in
        (a2av_run_bias); an ``index`` tensor (int32 [P, index_stride] gather
        lists of rows of ``row_elems`` elements) runs the indexed exchange
        (a2av_run_indexed); a ``host_counts`` array (numpy int32 [P, P], the
        same counts as ``send_counts``), alone or with any of these, runs the
        host-count form of the exchange (a2av_run_host_counts,
        a2av_run_blocked_host_counts, a2av_run_bias_host_counts,
        a2av_run_indexed_host_counts): count errors are raised before
        anything is enqueued, and the chunk plan follows the payload.

        The count and signal checks run on the device, so by default a
        failure is latched and reported by :meth:`query_error`.  With
        ``check=True`` the call waits for the run and raises on a device-side
        failure (ValueError for INVALID_ARGS / OVER_CAPACITY, A2avError for
        TIMEOUT), as if the checks had run before the call returned."""
        import torch
        if index is not None and bias is not None:
            raise ValueError("index and bias select different exchanges; give at most one")
        if index is not None and nblk != 1:
            raise ValueError("the indexed exchange takes no nblk")
        hc = None
        if host_counts is not None:
            import numpy as np
            hc = np.ascontiguousarray(host_counts, dtype=np.int32)
            if hc.shape != (self.cfg.P, self.cfg.P) or hc is not host_counts:
                raise ValueError("host_counts must be a contiguous int32 numpy array [P, P] "
                                 "(the exchange never copies operands)")
            hc = hc.ctypes.data
        c = self.cfg
        P = c.P
        ip = self._check(input, P * c.in_slab_bytes, "input")
        tp = self._check(target, P * c.tgt_slab_bytes, "target")
        sp = self._check(signal, P * c.S * 4, "signal", torch.int32)
        scp = self._check(send_counts, P * P * 4, "send_counts", torch.int32)
        rcp = self._check(recv_counts, P * P * 4, "recv_counts", torch.int32)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        if index is not None:
            if index.dim() != 2 or index.shape[0] != P:
                raise ValueError(f"index must be [P={P}, index_stride], got {tuple(index.shape)}")
            stride = index.shape[1]
            xp = self._check(index, P * stride * 4, "index", torch.int32)
            if hc is not None:
                st = a2av_run_indexed_host_counts(self.h, ip, tp, sp, scp, rcp, xp, hc, P,
                                                  core_num, dtype, row_elems, stride,
                                                  stream.cuda_stream)
            else:
                st = a2av_run_indexed(self.h, ip, tp, sp, scp, rcp, xp, P, core_num, dtype,
                                      row_elems, stride, stream.cuda_stream)
        elif bias is not None:
            be = {BF16: (torch.float32, 4), FP16: (torch.float16, 2)}.get(dtype)
            if be is None:  # the library reports the unsupported dtype
                bp = self._check(bias, bias.numel() * bias.element_size(), "bias")
            else:
                bp = self._check(bias, P * nblk * hidden * be[1], "bias", be[0])
            if hc is not None:
                st = a2av_run_bias_host_counts(self.h, ip, tp, sp, scp, rcp, bp, hc, P, core_num,
                                               dtype, nblk, hidden, stream.cuda_stream)
            else:
                st = a2av_run_bias(self.h, ip, tp, sp, scp, rcp, bp, P, core_num, dtype, nblk,
                                   hidden, stream.cuda_stream)
        elif hc is not None and nblk == 1:
            st = a2av_run_host_counts(self.h, ip, tp, sp, scp, rcp, hc, P, core_num, dtype,
                                      stream.cuda_stream)
        elif hc is not None:
            st = a2av_run_blocked_host_counts(self.h, ip, tp, sp, scp, rcp, hc, P, core_num,
                                              dtype, nblk, stream.cuda_stream)
        elif nblk == 1:
            st = a2av_run(self.h, ip, tp, sp, scp, rcp, P, core_num, dtype, stream.cuda_stream)
        else:
            st = a2av_run_blocked(self.h, ip, tp, sp, scp, rcp, P, core_num, dtype, nblk,
                                  stream.cuda_stream)
        _raise(st, "a2av_run", self.h)
        if check:
            _raise(self.query_error(), "a2av_run (device-side checks)", self.h)

    def query_error(self) -> int:
        return a2av_query_error(self.h)

    def launch_info(self, core_num: int) -> a2av_launch_info:
        st, info = a2av_launch_info_get(self.h, core_num)
        _raise(st, "a2av_launch_info_get")
        return info

    def profile_sample(self, every: int) -> None:
        """Record the profiling events on one run in ``every`` from now on."""
        _raise(a2av_profile_sample(self.h, every), "a2av_profile_sample", self.h)

    def profile(self) -> tuple[float, float, int, int]:
        """(K1 us, K2 us, K2 launches, runs) summed over the runs since the last call."""
        st, k1, k2, n, runs = a2av_profile_read(self.h)
        _raise(st, "a2av_profile_read", self.h)
        return k1, k2, n, runs
