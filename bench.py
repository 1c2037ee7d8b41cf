"""Benchmark of the all_to_all_v exchange on one MI355X.

One step = one a2av_run (K1 count kernel + the K2 copy launches) over one
seeded synthetic workload already resident in HBM.  Prints ONE JSON line with
the whole-run throughput (payload bytes read + written per second), the
roofline of the dominant kernel (K2, HBM-bound) from HIP events recorded by
the library on the run's stream during the timed region (on one timed step
in four: the events themselves cost a few microseconds each), and the CPU oracle
timed on a bounded sample of the same workload on the host.  Each workload
is also timed cache-cold: a 1 GiB buffer is written before every run, and
the medians of the single runs are reported under "cold".  The small
exchanges (c1, c2) are also timed as replays of one run captured into a HIP
graph ("graph").  Beside them: the rates of the copy kernel's own
instructions streaming 1 GiB ("ceiling"), and what a cooperative launch
costs on the stream against a regular one ("launch_cost").

    python bench.py [--steps K] [--warmup W] [--workload c5] [--also c3,c4]
"""
from __future__ import annotations

import argparse
import hashlib
import dataclasses
from dataclasses import dataclass
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "all_to_all_v achieved HBM GB/s (read+write) and % of MI355X peak, 1 GPU"
PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
# The workloads bench.py can time.  c1..c5 are the plain exchange.  c5u is
# c5's exchange taken on the source's own temp3 layout (E/ep, ep*C, H/tp):
# the blocked exchange with nblk = E/ep = 8.  c5b is that exchange in BF16
# with the bias Add fused in front (FP32 bias), c5h in FP16 (FP16 bias).  c3i is c3's MoE dispatch as the indexed
# exchange: token tables stored once, the routing as gather lists.
# cpu_scale: the size divisor of the oracle sample for the CPU baseline.
@dataclass(frozen=True)
class Spec:
    kind: str            # "plain", "blocked", "bias" or "indexed"
    k: int = 5           # workload index (plain and blocked)
    nblk: int = 1
    cpu_scale: int = 1
    cold_runs: int = 50  # runs of the cache-cold protocol (each after a 1 GiB flush)
    graph: bool = False  # also time replays of one run captured into a HIP graph
    half: bool = False   # bias workloads: FP16 payload and bias instead of BF16 + FP32
    host_counts: bool = False  # plain: run a2av_run_host_counts (chunk plan from the payload)
    core_num: int = 0    # > 0: this core_num instead of the workload's (a diagnostic line)
    block_wait: bool = True  # False: the handle takes A2AV_FLAG_NO_BLOCK_WAIT


WORKLOADS = {"c1": Spec("plain", 1, graph=True), "c2": Spec("plain", 2, graph=True), "c3": Spec("plain", 3, cpu_scale=4),
             "c4": Spec("plain", 4, cpu_scale=4, cold_runs=20),
             "c5": Spec("plain", 5, cpu_scale=8, cold_runs=5),
             "c5u": Spec("blocked", 5, nblk=8, cpu_scale=8, cold_runs=5),
             "c5b": Spec("bias", nblk=8, cpu_scale=16, cold_runs=5),
             "c5h": Spec("bias", nblk=8, cpu_scale=16, cold_runs=5, half=True),
             "c3i": Spec("indexed", cpu_scale=4),
             # c4 through a2av_run_host_counts: one launch for its ~0.8 GiB
             # instead of the two that cover its 2 GiB slab bound.
             "c4h": Spec("plain", 4, cpu_scale=4, cold_runs=20, host_counts=True),
             # Diagnostics, not the workloads' configurations: c3 and c4 with
             # core_num 1 (B = 1, one regular launch of the same workgroups),
             # beside their cooperative B = 64 / 256 runs, to show what the
             # cooperative launch itself costs a run.
             "c3b1": Spec("plain", 3, cpu_scale=4, core_num=1),
             "c4b1": Spec("plain", 4, cpu_scale=4, cold_runs=20, core_num=1),
             # c3 and c4 (with its host counts) on handles that skip the
             # blocks' wait: a regular final launch, the same flags.
             "c3nw": Spec("plain", 3, cpu_scale=4, block_wait=False),
             "c4hnw": Spec("plain", 4, cpu_scale=4, cold_runs=20, host_counts=True,
                           block_wait=False)}
FLUSH_BYTES = 1 << 30       # written before each cache-cold run: above the 256 MB MALL
# The library's profiling events cost a few microseconds each on the stream;
# the timed steps record them on one step in EVENTS_EVERY.
EVENTS_EVERY = 4
DTYPE_NAMES = {0: "fp32", 1: "u8", 2: "fp16", 3: "bf16"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "copy_kernel_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank lines left out, so
    that a change of wording does not void the counter figures taken on the
    same code."""
    h = hashlib.sha256()
    for f in ["kernels.hip", "kernels.h"]:
        for line in open(os.path.join(ROOT, "all_movement_amd", "csrc", f), encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per K2 launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def make_workload(spec: Spec, scale: int = 1):
    """The workload of a spec, at 1/scale of its size where the spec allows."""
    from all_movement_amd import workloads as wl
    if spec.kind == "indexed":
        return wl.indexed_workload(scale=scale)
    if spec.kind == "bias":
        return wl.bias_workload(wl.FP16 if spec.half else wl.BF16, scale=scale)
    w = wl.workload(spec.k, scale=scale)
    if spec.kind == "blocked":
        w.name += f"_temp3_layout_nblk{spec.nblk}"
    if spec.host_counts:
        w.name += "_host_counts"
    if spec.core_num:
        w.core_num = spec.core_num
        w.name += f"_core_num{spec.core_num}"
    if not spec.block_wait:
        w.name += "_no_block_wait"
    return w


def run_gpu(spec: Spec, steps: int, warmup: int, cold: bool = True):
    import numpy as np
    import torch
    from all_movement_amd import a2av
    from all_movement_amd import workloads as wl

    dev = torch.device("cuda:0")
    w = make_workload(spec)
    # Arguments of Exchange.run beyond the five operands, and the extra bytes
    # a run reads once (the bias, or the gather-list entries in use).
    extra = {"nblk": spec.nblk}
    if spec.host_counts:
        extra["host_counts"] = np.ascontiguousarray(w.counts, np.int32)
    extra_bytes = 0
    if spec.kind == "indexed":
        extra["row_elems"] = w.extra["row_elems"]
        extra["index"] = torch.from_numpy(w.extra["index"]).to(dev)
        extra_bytes = 4 * int(w.counts.astype(np.int64).sum()) // w.extra["row_elems"]
    elif spec.kind == "bias":
        extra["hidden"] = w.extra["hidden"]
        extra["bias"] = wl.bias_tensor(w, spec.nblk, extra["hidden"], dev)
        extra_bytes = extra["bias"].numel() * extra["bias"].element_size()
    log(f"[bench] {w.name}: payload {w.payload_bytes} B, generating inputs on the GPU")
    inp = wl.input16_tensor(w, dev) if spec.kind == "bias" else wl.input_tensor(w, dev)
    tgt = torch.full((w.tgt_bytes,), wl.SENTINEL, dtype=torch.uint8, device=dev)
    sig = torch.zeros((w.P, w.S), dtype=torch.int32, device=dev)
    sc = torch.from_numpy(w.counts).to(dev)
    rc = torch.zeros((w.P, w.P), dtype=torch.int32, device=dev)
    ex = a2av.Exchange(w.P, w.in_slab, w.tgt_slab, w.S, device=0, profile=True,
                       block_wait=spec.block_wait)
    info = ex.launch_info(w.core_num)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    for _ in range(warmup):
        ex.run(inp, tgt, sig, sc, rc, w.core_num, w.dtype, stream, **extra)
    torch.cuda.synchronize()
    if ex.query_error() != a2av.OK:
        raise RuntimeError("warmup run reported a device-side error")
    ex.profile()                           # drop the warmup tally
    ex.profile_sample(EVENTS_EVERY)        # timed steps 0, 4, 8, ... carry the events

    t0 = time.perf_counter()
    for _ in range(steps):
        ex.run(inp, tgt, sig, sc, rc, w.core_num, w.dtype, stream, **extra)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if ex.query_error() != a2av.OK:
        raise RuntimeError("timed run reported a device-side error")
    k1_us, k2_us, k2_launches, runs = ex.profile()

    # Cache-cold protocol: before each run, write a 1 GiB scratch buffer so
    # that no payload line survives in the L2s or the MALL, then time that
    # run alone -- by its events (K1 start to last K2 end) and by the host
    # clock around the run and a synchronize.  Medians are reported.
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev) if cold else None
    ex.profile_sample(1)
    dev_s, wall_s = [], []
    for i in range(spec.cold_runs if cold else 0):
        flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        ex.run(inp, tgt, sig, sc, rc, w.core_num, w.dtype, stream, **extra)
        torch.cuda.synchronize()
        wall_s.append(time.perf_counter() - c0)
        c1_us, c2_us, _, n = ex.profile()
        dev_s.append((c1_us + c2_us) * 1e-6 / max(n, 1))
    if ex.query_error() != a2av.OK:
        raise RuntimeError("cache-cold run reported a device-side error")
    del flush

    # Small exchanges are bound by the host's enqueue; a caller that replays a
    # captured run pays only the graph launch.  One run is captured and
    # replayed back to back (each replay is one more run).
    graph = None
    if spec.graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ex.run(inp, tgt, sig, sc, rc, w.core_num, w.dtype, **extra)
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        g_sec = (time.perf_counter() - g0) / steps
        if ex.query_error() != a2av.OK:
            raise RuntimeError("graph replay reported a device-side error")
        del g
        graph = {"runs": steps, "us_per_run": round(g_sec * 1e6, 2)}
    ex.close()
    sec = t1 - t0
    # Each payload byte read once and written once (plus the bias or the
    # gather lists, read once).
    moved = 2 * w.payload_bytes + extra_bytes
    res = {
        "w": w, "info": info, "sec": sec, "steps": steps, "moved": moved,
        "gbps": moved * steps / sec / 1e9, "ms_per_step": sec / steps * 1e3,
        "k1_us": k1_us / max(runs, 1), "k2_us_per_run": k2_us / max(runs, 1),
        "k2_launches_per_run": k2_launches / max(runs, 1), "profiled_steps": runs,
    }
    # The dominant kernel is K2; its launches share the payload.
    res["k2_us_per_launch"] = res["k2_us_per_run"] / res["k2_launches_per_run"]
    res["k2_gbps"] = moved / (res["k2_us_per_run"] * 1e-6) / 1e9
    dev_s.sort()
    wall_s.sort()
    if graph is not None:
        graph["gbps"] = round(moved / (graph["us_per_run"] * 1e-6) / 1e9, 2)
    res["graph"] = graph
    res["cold"] = None if not dev_s else {
        "runs": spec.cold_runs, "flush_bytes": FLUSH_BYTES,
        "gbps_device_median": round(moved / dev_s[len(dev_s) // 2] / 1e9, 1),
        "gbps_wall_median": round(moved / wall_s[len(wall_s) // 2] / 1e9, 1),
        "us_device_median": round(dev_s[len(dev_s) // 2] * 1e6, 2),
        "us_wall_median": round(wall_s[len(wall_s) // 2] * 1e6, 2),
    }
    del inp, tgt
    torch.cuda.empty_cache()
    return res


def copy_probe(nbytes: int, steps: int) -> None:
    """A plain device-to-device copy of a known size (torch's copy kernel):
    reads and writes exactly nbytes per launch, the reference that scales the
    HBM byte counters of the exchange's kernels."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": steps}), flush=True)


def stream_ceiling(nbytes: int = 1 << 30, reps: int = 10, warmup: int = 3):
    """The rates the copy kernel's own memory instructions reach when they
    only read, only write, or copy (the library's streaming probes, same
    launch shape and tile claims), over `nbytes`, timed with HIP events on
    the stream the probes are launched on."""
    import torch
    from all_movement_amd import a2av
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    out = {"bytes": nbytes}
    for name, kind, moved in [("read_only", a2av.PROBE_READ, nbytes),
                              ("write_only", a2av.PROBE_WRITE, nbytes),
                              ("copy", a2av.PROBE_COPY, 2 * nbytes)]:
        def launch():
            st = a2av.a2av_probe_stream(kind, src.data_ptr(), dst.data_ptr(), nbytes, 0,
                                        stream.cuda_stream)
            if st != a2av.OK:
                raise RuntimeError(f"a2av_probe_stream: {a2av.a2av_status_string(st)}")
        for _ in range(warmup):
            launch()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = {"gbps": round(moved / us / 1e3, 1), "us_per_launch": round(us, 2)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def launch_cost(nbytes: int = 64 << 20, reps: int = 40, warmup: int = 5):
    """What a cooperative launch costs on the stream, apart from any exchange
    (the library's launch probe): pairs of launches, one workgroup per CU, a
    store kernel writing `nbytes` with the copy kernel's store instruction and
    then the same kernel storing nothing, each launch regular or cooperative,
    back to back on one stream, timed with HIP events on that stream.  A
    cooperative launch's cost is the pair time with it less the pair time
    with both launches regular."""
    import torch
    from all_movement_amd import a2av
    dev = torch.device("cuda:0")
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {"bytes_first_launch": nbytes, "pairs": reps}
    for name, (c0, c1) in [("regular_regular", (0, 0)), ("coop_regular", (1, 0)),
                           ("regular_coop", (0, 1)), ("coop_coop", (1, 1))]:
        def pair():
            for coop, n in ((c0, nbytes), (c1, 0)):
                st = a2av.a2av_probe_launch(coop, dst.data_ptr(), n, 0, stream.cuda_stream)
                if st != a2av.OK:
                    raise RuntimeError(f"a2av_probe_launch: {a2av.a2av_status_string(st)}")
        for _ in range(warmup):
            pair()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pair()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    rr = out["regular_regular_us"]
    extra = [out["coop_regular_us"] - rr, out["regular_coop_us"] - rr,
             (out["coop_coop_us"] - rr) / 2]
    out["per_cooperative_launch_us"] = round(sum(extra) / len(extra), 2)
    del dst
    torch.cuda.empty_cache()
    return out


def cpu_baseline(spec: Spec, min_seconds: float = 10.0):
    """The oracle (as it stands) on a bounded sample of the workload on the host."""
    import numpy as np

    import oracle
    from all_movement_amd import workloads as wl

    # Sample: the same workload shape at 1/cpu_scale of its size (c5 at 1/8:
    # P=8 equal counts of 2^22 fp32, 1 GiB of payload), run whole.
    scale = spec.cpu_scale
    w = make_workload(spec, scale=scale)
    if spec.kind == "indexed":
        inp = wl.input_bytes_np(w)
        what = "checks + transpose + displacements + one memcpy per gathered row + signal"
    elif spec.kind == "bias":
        A, H = w.extra["nblk"], w.extra["hidden"]
        inp = wl.input16_np(w)
        bias = wl.bias_np(w, A, H)
        what = "checks + transpose + displacements + one fp32 add and bf16 rounding per element"
    elif spec.kind == "blocked":
        inp = wl.input_bytes_np(w)
        what = "checks + transpose + displacements + one memcpy per sub-block + signal"
    else:
        inp = wl.input_bytes_np(w)
        what = "checks + transpose + displacements + one memcpy per segment + signal"
    tgt = np.full(w.tgt_bytes, wl.SENTINEL, np.uint8)
    rc = np.zeros((w.P, w.P), np.int32)
    times = []
    t_end = time.perf_counter() + min_seconds
    while len(times) < 3 or time.perf_counter() < t_end:
        sig = np.zeros((w.P, w.S), np.int32)
        kw = dict(P=w.P, S=w.S, in_slab=w.in_slab, tgt_slab=w.tgt_slab, core_num=w.core_num,
                  dtype=w.dtype)
        t0 = time.perf_counter()
        if spec.kind == "indexed":
            st = oracle.run_indexed(inp, tgt, sig, w.counts, rc, w.extra["index"],
                                    row_elems=w.extra["row_elems"],
                                    index_stride=w.extra["index_stride"], **kw)
        elif spec.kind == "bias":
            st = oracle.run_bias(inp, tgt, sig, w.counts, rc, bias, nblk=A, hidden=H, **kw)
        elif spec.kind == "blocked":
            st = oracle.run_blocked(inp, tgt, sig, w.counts, rc, nblk=spec.nblk, **kw)
        else:
            st = oracle.run(inp, tgt, sig, w.counts, rc, **kw)
        times.append(time.perf_counter() - t0)
        assert st == oracle.OK
    times.sort()
    med = times[len(times) // 2]
    return {
        "value": round(2 * w.payload_bytes / med / 1e9, 3), "unit": "GB/s", "cores": 1,
        "kind": "oracle",
        "sample": f"{w.name} at 1/{scale} size ({w.payload_bytes} payload bytes), whole oracle "
                  f"({what}), single thread, median of {len(times)} runs over "
                  f"{sum(times):.1f} s",
        "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--also", default="c1,c2,c3,c4,c5u,c5b,c5h,c3i,c4h,c3b1,c4b1,c3nw,c4hnw",
                    help="other workloads reported beside it")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cache-cold runs (profiler runs that count only the timed runs)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only time the streaming probes (read-only, write-only, copy of 1 GiB "
                         "with the copy kernel's instructions) and print them")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming probes and the launch probe")
    ap.add_argument("--launch-cost-only", action="store_true",
                    help="only time the launch probe (regular against cooperative launches, "
                         "--steps pairs of each kind) and print it")
    ap.add_argument("--no-block-wait", action="store_true",
                    help="run every workload on a handle with A2AV_FLAG_NO_BLOCK_WAIT (a "
                         "regular final launch; for counter runs under a profiler)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain torch device copy of MIB MiB --steps times (the "
                         "known-size reference for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the exchange runs its P virtual ranks as slabs "
              "of one GPU's memory, and there is no multi-GPU exchange to time.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe << 20, args.steps)
        return
    if args.ceiling_only:
        print(json.dumps({"ceiling": stream_ceiling(reps=args.steps)}), flush=True)
        return
    if args.launch_cost_only:
        print(json.dumps({"launch_cost": launch_cost(reps=args.steps)}), flush=True)
        return
    spec = WORKLOADS[args.workload]
    if args.no_block_wait:
        spec = dataclasses.replace(spec, block_wait=False)
    main_res = run_gpu(spec, args.steps, args.warmup, cold=not args.no_cold)
    w, info = main_res["w"], main_res["info"]
    log(f"[bench] {w.name}: {main_res['gbps']:.1f} GB/s whole run, K2 "
        f"{main_res['k2_gbps']:.1f} GB/s, {main_res['ms_per_step']:.3f} ms/step")
    also = {}
    for name in [s for s in args.also.split(",") if s and s != args.workload]:
        also_spec = WORKLOADS[name]
        if args.no_block_wait:
            also_spec = dataclasses.replace(also_spec, block_wait=False)
        r = run_gpu(also_spec, args.steps, args.warmup, cold=not args.no_cold)
        log(f"[bench] {r['w'].name}: {r['gbps']:.1f} GB/s whole run, K2 {r['k2_gbps']:.1f} GB/s")
        also[r["w"].name] = {"value": round(r["gbps"], 1), "frac_of_peak": round(r["gbps"] / PEAK_GBPS, 4),
                             "k2_gbps": round(r["k2_gbps"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                             "blocks": r["info"].blocks, "workgroups": r["info"].workgroups,
                             "traffic_per_launch": measured_traffic(r["w"].name),
                             "cold": r["cold"], "graph": r["graph"]}

    traffic = measured_traffic(w.name)
    per_launch_bytes = main_res["moved"] / main_res["k2_launches_per_run"]
    roofline = {
        "bound": "hbm", "kernel": "copy_kernel (K2)",
        "achieved": round(per_launch_bytes / (main_res["k2_us_per_launch"] * 1e-6) / 1e9, 1),
        "peak": PEAK_GBPS, "unit": "GB/s",
        "frac": round(per_launch_bytes / (main_res["k2_us_per_launch"] * 1e-6) / 1e9 / PEAK_GBPS, 4),
        "traffic": traffic,
        "bytes_per_launch": int(per_launch_bytes),
        "launches_per_step": main_res["k2_launches_per_run"],
        "avg_launch_us": round(main_res["k2_us_per_launch"], 2),
        "k1_us": round(main_res["k1_us"], 2),
        "event_steps": f"{main_res['profiled_steps']} of {args.steps} timed steps carry the "
                       f"events (one in {EVENTS_EVERY})",
    }
    if not args.no_ceiling:
        ceiling = stream_ceiling()
        roofline["ceiling"] = ceiling["copy"]["gbps"]
        roofline["frac_of_ceiling"] = round(roofline["achieved"] / ceiling["copy"]["gbps"], 4)
    else:
        ceiling = None
    coop_cost = None if args.no_ceiling else launch_cost()
    out = {
        "metric": METRIC, "value": round(main_res["gbps"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAMES[w.dtype],
        "data": "synthetic (seeded SplitMix64 payload, seeded count matrices)",
        "config": {"workload": w.name, "P": w.P, "core_num": w.core_num,
                   "blocks": info.blocks, "workgroups": info.workgroups,
                   "chunk_launches": info.chunk_launches,
                   "payload_bytes": w.payload_bytes, "parallelism": "1 GPU, P virtual ranks"},
        "frac_of_peak": round(main_res["gbps"] / PEAK_GBPS, 4),
        "roofline": roofline,
        "cold": main_res["cold"],
        "graph": main_res["graph"],
        "ceiling": ceiling,
        "launch_cost": coop_cost,
        "also": also,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(spec)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
