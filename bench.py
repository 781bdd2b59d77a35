"""Benchmark: effective HBM bandwidth of RMSNorm bf16 at [4 x 4096 x 3072] on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--windows N]

One step is one launch of the RMSNorm path (load, square-accumulate, reduce,
scale, round, store) over the whole [4 x 4096 x 3072] bf16 batch.  Inputs are
seeded synthetic tensors (x ~ N(0,1), weight ~ U(0.5,1.5)), resident in HBM
before timing starts.  Consecutive steps cycle through enough copies of the
input and output buffers (>= 1 GiB in total) that the 256 MB memory-side
Infinity Cache cannot serve a step from the previous one.

Timing: after W warm-up launches, N windows (default 5) of exactly K launches
each are timed with HIP events recorded on the stream the kernels are
launched on.  Before each window the stream is held behind a short spin
kernel while the host enqueues the window's K launches, so a window measures
K back-to-back kernels and not the host's latency in issuing the first one;
each window is bracketed by device synchronisation.  value and ms_per_step
come from the median window, with the fastest and slowest beside them.  The
K launches are issued one by one on the stream; `--launch graph` captures
them into one HIP graph and replays it once per window instead (the library
only enqueues kernels, so the launches capture as they are).  The line
reports the headline in the other mode too ("graph_launch" /
"stream_launch").

value = algorithmic bytes per step (read x + write y + read weight once,
201,332,736 B) / seconds per step, in GB/s (10^9 B/s); it is compared with
MI355X's 8 TB/s HBM peak in the "roofline" object, and with copy kernels
moving the same buffers, timed the same way in the same run (ceiling/copy.hip:
plain and non-temporal 16-byte copies, non-temporal read-only and write-only
streams, and the runtime's device copy), under "copy_ceiling" and
"pct_of_copy_ceiling".  The same line reports the fused RMSNorm+RoPE
workload ([2 x 4096 x 2048], 32 heads x 64, fp32 cos/sin tables) under
"rope" (rotate-half pairs) and "rope_interleaved" (adjacent pairs), the
AdaLN-modulated RMSNorm ([2 x 4096 x 2048], per-sample scale/shift) under
"adaln", the other four shapes of the pages' RMSNorm micro-benchmark under
"pages_shapes" (with the page's H100 ms as context), the headline RMSNorm with
fp16 and fp32 I/O under "rms_f16" / "rms_f32" (and the RoPE / AdaLN workloads
in fp16 or fp32 under "rope_f16", "rope_f32", "adaln_f32"), RoPE (24 heads x
128, both pairings) and AdaLN at the headline's size under "rope_large",
"rope_interleaved_large" and "adaln_large", five shapes outside the pages'
set under "general" (hidden 3076, not a whole number of 16-byte vectors; 16
heads x 72 with rotate-half pairs; rows of 262144, beyond the register
budget; per-head rows of 128; AdaLN at hidden 1152), and the CPU oracle timed
on this host under "cpu_baseline".  The same CPU leg compares every timed
workload's output, element by element over the whole batch, with the
oracle's result ("parity").  Prints one JSON line.

--probe NAME (a short name below, or any workload of the pages' table, e.g.
rms_1x1024x2048) runs --launches launches of one workload with the same
rotating buffers and nothing else, for rocprofv3 kernel traces and counter
passes; --probe copy runs the runtime's device copy of the headline's bytes
(the counters' calibration), --probe copy_nt the non-temporal copy kernel.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "effective HBM GB/s (bytes read+written / time) and % of peak, RMSNorm bf16"
# H100 figure for the same shape and byte convention: 201,332,736 B in 0.157 ms
# (Hugging Face cuda-kernels skill page, "RMSNorm Micro-benchmarks"); context only.
H100_GBPS_4x4096x3072 = 201_332_736 / 0.157e-3 / 1e9
# The custom kernel's ms for every shape of that table (same page and
# section), quoted beside the MI355X figures for the same shapes; context only.
H100_MS = {"rms_1x1024x2048": 0.019, "rms_2x1024x2048": 0.024, "rms_4x1024x2048": 0.036,
           "rms_2x4096x3072_outliers": 0.087, "rms_4x4096x3072": 0.157}
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
KERNEL_SOURCES = (sorted(glob.glob(os.path.join(ROOT, "rmsnorm_video_dit_amd", "csrc", "*.hip")))
                  + sorted(glob.glob(os.path.join(ROOT, "rmsnorm_video_dit_amd", "csrc", "*.h"))))
DTYPE_CODE = {"bf16": 0, "f16": 1, "f32": 2}
# --probe names: workload and I/O dtype of each benchmark line
PROBES = {"rms": (datagen.HEADLINE, "bf16"), "rms_f16": (datagen.HEADLINE, "f16"),
          "rms_f32": (datagen.HEADLINE, "f32"), "rope": (datagen.ROPE, "bf16"),
          "ropei": (datagen.ROPE_INTERLEAVED, "bf16"), "adaln": (datagen.ADALN, "bf16"),
          "rope_f16": (datagen.ROPE, "f16"), "rope_f32": (datagen.ROPE, "f32"),
          "adaln_f32": (datagen.ADALN, "f32"),
          "rms_odd": ("rms_4x4096x3076", "bf16"), "rope_d72": ("rope_2x4096x1152_h16d72", "bf16"),
          "rms_long": ("rms_1x512x131072", "bf16"), "rms_split": ("rms_1x64x1048576", "bf16"),
          "rms_short": ("rms_2x4096x24_d128", "bf16"),
          "adaln_seg": ("adaln_8x4096x1152", "bf16"),
          "rope_large": ("rope_4x4096x3072_h24d128", "bf16"),
          "ropei_large": ("ropei_4x4096x3072_h24d128", "bf16"),
          "adaln_large": ("adaln_4x4096x3072", "bf16")}
ELEM_BYTES = {"bf16": 2, "f16": 2, "f32": 4}
ALL_CONFIGS = {**datagen.CONFIGS, **datagen.GENERAL_CONFIGS, **datagen.LARGE_CONFIGS}


def gbps(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9


def pct_of_peak(gb_s: float, peak_gbps: float) -> float:
    return 100.0 * gb_s / peak_gbps


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def source_hash() -> str:
    """Hash of the kernel sources' code (comments and blank space removed), so
    that stored counter figures stay valid across comment-only edits."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            code = _COMMENT.sub("", f.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def read_traffic_parts(kernel: str, workload: str):
    """(fetched, written) HBM bytes per launch from the committed counter
    summary, or None when there is none or the kernel sources changed since
    it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    cur = source_hash()
    for line in open(TRAFFIC_FILE):
        if line.startswith("#") or not line.strip():
            continue
        kv = dict(tok.split("=", 1) for tok in line.split())
        if kv.get("kernel") == kernel and kv.get("workload") == workload:
            if kv.get("src_sha") != cur:
                return None
            return float(kv["fetch_bytes"]), float(kv["write_bytes"])
    return None


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch (fetched + written), or None as above."""
    parts = read_traffic_parts(kernel, workload)
    return None if parts is None else parts[0] + parts[1]


def to_device(a, dev):
    """bf16 bit patterns (uint16) become a bfloat16 tensor; float16/float32
    arrays keep their type."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def to_host(t) -> np.ndarray:
    """A device output as the oracle compares it: bf16 as uint16 bit
    patterns, fp16 and fp32 as numpy arrays of that type."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Workload:
    """Rotating device buffers for one config, and the launch of one step."""

    def __init__(self, cfg: datagen.Config, dev, stream, max_sets=None, dtype: str = "bf16"):
        import torch
        import rmsnorm_video_dit_amd as ltx
        self.cfg, self.ltx, self.stream = cfg, ltx, stream
        self.dtype, self.code = dtype, DTYPE_CODE[dtype]
        self.nbytes = cfg.algorithmic_bytes(ELEM_BYTES[dtype])
        inp = datagen.make_inputs(cfg, dtype=dtype)
        self.host = inp
        per_set = 2 * cfg.rows * cfg.hidden * ELEM_BYTES[dtype]
        n = max(2, -(-ROTATE_BYTES // per_set))
        if max_sets:
            n = min(n, max_sets)
        self.nsets = n
        x0 = to_device(inp["x"], dev)
        self.x = [x0] + [x0.clone() for _ in range(n - 1)]
        self.y = [torch.empty_like(x0) for _ in range(n)]
        self.w = to_device(inp["w"], dev)
        if cfg.rope:
            self.cos = torch.from_numpy(inp["cos"]).to(dev)
            self.sin = torch.from_numpy(inp["sin"]).to(dev)
        if cfg.adaln:
            self.scale = to_device(inp["scale"], dev)
            self.shift = to_device(inp["shift"], dev)
        torch.cuda.synchronize()

    def step(self, i: int):
        c = self.cfg
        k = i % self.nsets
        if c.adaln:
            self.ltx.ltxnorm_rmsnorm_adaln_fwd_dt(self.y[k], self.x[k], self.w, self.scale,
                                                  self.shift, c.rows, c.hidden, c.seq, c.eps,
                                                  self.code, self.stream)
        elif c.rope:
            fn = (self.ltx.ltxnorm_rmsnorm_rope_interleaved_fwd_dt if c.interleaved
                  else self.ltx.ltxnorm_rmsnorm_rope_fwd_dt)
            fn(self.y[k], self.x[k], self.w, self.cos, self.sin, c.rows, c.hidden, c.heads,
               c.head_dim, c.seq, c.eps, self.code, self.stream)
        else:
            self.ltx.ltxnorm_rmsnorm_fwd_dt(self.y[k], self.x[k], self.w, c.rows, c.hidden, c.eps,
                                            self.code, self.stream)

    def output(self) -> np.ndarray:
        """The output of the last timed launches (every rotating set holds the
        same input, so any set's output is the timed kernel's result)."""
        return to_host(self.y[0])

    def time_steps(self, clock: "Clock", steps: int, warmup: int, graph: bool = False) -> list:
        """Warm up, then time `clock.windows` windows of exactly `steps`
        launches each (see Clock); returns seconds per step for every window.
        With `graph`, the `steps` launches are captured into one HIP graph
        first (they only enqueue kernels) and each window is one replay of it:
        every launch still runs in full, without the host-side cost of issuing
        it."""
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(steps):
                    self.step(warmup + i)
            torch.cuda.synchronize()

            def issue():
                with torch.cuda.stream(self.stream):
                    g.replay()
            res = clock.time(issue, steps)
            del g
            return res

        def issue():
            for i in range(steps):
                self.step(i)
        return clock.time(issue, steps)


class Clock:
    """Times windows of K launches on one stream with HIP events recorded on
    that stream.  Before each window the stream is held behind a spin kernel
    (torch's sleep kernel, about `hold_us` long) while the host records the
    start event and enqueues the K launches; the start event therefore fires
    when the first launch can begin at once, and the window measures K
    back-to-back kernels, not the host's time to issue the first of them.
    Each window is bracketed by device synchronisation on both sides."""

    def __init__(self, stream, windows: int = 5, hold_us: float = 2000.0):
        import torch
        self.stream, self.windows = stream, windows
        n = 2_000_000
        with torch.cuda.stream(stream):
            torch.cuda._sleep(1000)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.cuda._sleep(n)
            e1.record(stream)
        torch.cuda.synchronize()
        us = max(e0.elapsed_time(e1) * 1e3, 1.0)
        self.cycles_per_us = n / us
        self.hold_us = hold_us
        self.hold_cycles = max(1, int(hold_us * self.cycles_per_us))

    def time(self, issue, steps: int) -> list:
        """issue() enqueues exactly `steps` launches on the stream; returns
        seconds per launch for each of the windows."""
        import torch
        out = []
        for _ in range(self.windows):
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(self.stream):
                torch.cuda._sleep(self.hold_cycles)
            t0.record(self.stream)
            issue()
            t1.record(self.stream)
            torch.cuda.synchronize()
            out.append(t0.elapsed_time(t1) * 1e-3 / steps)
        return out


def stats(per_step: list) -> dict:
    """Median, min and max seconds per step over the windows."""
    s = sorted(per_step)
    return {"median": s[len(s) // 2] if len(s) % 2 else 0.5 * (s[len(s) // 2 - 1] + s[len(s) // 2]),
            "min": s[0], "max": s[-1]}


def timing_fields(per_step: list, nbytes: int) -> dict:
    """The per-workload timing fields: value from the median window, with the
    fastest and slowest windows beside it."""
    st = stats(per_step)
    return {"value": round(gbps(nbytes, st["median"]), 2), "unit": "GB/s",
            "ms_per_step": round(st["median"] * 1e3, 6),
            "gpu_ms_median": round(st["median"] * 1e3, 6),
            "gpu_ms_min": round(st["min"] * 1e3, 6), "gpu_ms_max": round(st["max"] * 1e3, 6),
            "frac": round(gbps(nbytes, st["median"]) / HBM_PEAK_GBPS, 4)}


def copy_ceilings(clock: Clock, wl: Workload, steps: int, warmup: int) -> dict:
    """The bandwidth ceiling on the same bytes: the committed copy kernels
    (ceiling/copy.hip) moving each rotating set's x into its y (plain and
    non-temporal 16-byte copies at 1, 2, 4 and 8 vectors per thread), a
    non-temporal read-only and write-only stream of the same buffers, and
    the runtime's device-to-device copy, each timed like the kernels."""
    import torch
    import ceiling
    nvec = wl.x[0].numel() * wl.x[0].element_size() // 16
    copy_bytes = 2 * 16 * nvec
    sink = torch.zeros(256, dtype=torch.int32, device=wl.x[0].device)
    h = wl.stream.cuda_stream
    out = {}

    def run(key, mode, per, nbytes):
        def step(i):
            k = i % wl.nsets
            ceiling.copy(wl.y[k].data_ptr(), wl.x[k].data_ptr(), nvec, mode, per, sink.data_ptr(), h)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()

        def issue():
            for i in range(steps):
                step(i)
        res = timing_fields(clock.time(issue, steps), nbytes)
        res["bytes_per_step"] = nbytes
        out[key] = res

    for per in (1, 2, 4, 8):
        run(f"nt_copy_x{per}", ceiling.NT_COPY, per, copy_bytes)
    for per in (2, 4):
        run(f"plain_copy_x{per}", ceiling.PLAIN, per, copy_bytes)
    run("nt_read_x4", ceiling.NT_READ, 4, copy_bytes // 2)
    run("nt_write_x4", ceiling.NT_WRITE, 4, copy_bytes // 2)

    def memcpy_step(i):
        k = i % wl.nsets
        wl.y[k].copy_(wl.x[k])
    with torch.cuda.stream(wl.stream):
        for i in range(warmup):
            memcpy_step(i)
    torch.cuda.synchronize()

    def memcpy_issue():
        with torch.cuda.stream(wl.stream):
            for i in range(steps):
                memcpy_step(i)
    out["runtime_d2d_copy"] = {**timing_fields(clock.time(memcpy_issue, steps), copy_bytes),
                               "bytes_per_step": copy_bytes}
    best_key = max((k for k in out if "copy" in k), key=lambda k: out[k]["value"])
    return {"best": best_key, "value": out[best_key]["value"], "unit": "GB/s", "kernels": out}


def describe(cfg: datagen.Config, dtype: str = "bf16") -> str:
    """The kernel and launch shape the library picks for a workload."""
    import rmsnorm_video_dit_amd as ltx
    op = (ltx.OP_ADALN if cfg.adaln else ltx.OP_ROPE_INTERLEAVED if cfg.interleaved
          else ltx.OP_ROPE if cfg.rope else ltx.OP_RMSNORM)
    return ltx.ltxnorm_describe_launch(op, cfg.rows, cfg.hidden, cfg.heads, cfg.head_dim,
                                       DTYPE_CODE[dtype])


def launch_floor_us(stream, launches: int = 1000) -> float:
    """Per-launch time of a back-to-back empty kernel on the same stream
    (torch's sleep kernel with zero cycles): the part of every step that no
    kernel design removes."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(20):
            torch.cuda._sleep(0)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(launches):
            torch.cuda._sleep(0)
        t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / launches


def cpu_threads() -> tuple:
    """(threads to use, CPUs this process may run on, CPUs of the host).  The
    pool takes every CPU the process may run on, capped by OMP_NUM_THREADS
    when the environment sets it (the CPU share a job on a shared host is
    given)."""
    host = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = host
    t = avail
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        t = min(t, int(env))
    return max(1, t), avail, host


def cpu_baseline(cfg: datagen.Config, inp: dict, checks: list, runs: int = 3,
                 run_s: float = 2.0) -> dict:
    """The CPU oracle (double arithmetic, one rounding) on this host: the full
    batch split into contiguous row blocks over a thread pool, and the full
    batch on one thread.  Each is timed `runs` times (a pooled run repeats
    whole passes for about `run_s` seconds) and the median per-pass time is
    reported.  The same
    leg then checks every timed kernel's output against the oracle (`checks`,
    see oracle_parity) and returns that report under "parity"."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    o = oracle.Oracle()
    threads, avail, host = cpu_threads()
    x, w = inp["x"], inp["w"]
    blocks = [b for b in np.array_split(np.arange(cfg.rows), threads) if len(b)]

    def work(b):
        y = o.rmsnorm(x[b[0]:b[-1] + 1], w, cfg.eps)
        o.round(y)
        return len(b)

    def med(v):
        v = sorted(v)
        return v[len(v) // 2]

    pool_s, passes = [], []
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, blocks))  # first touch of the pages and the library
        for _ in range(runs):
            # one run: whole passes over the batch until run_s has passed
            n, t0 = 0, time.perf_counter()
            while True:
                list(ex.map(work, blocks))
                n += 1
                el = time.perf_counter() - t0
                if el >= run_s:
                    break
            pool_s.append(el / n)
            passes.append(n)
    one_s = []
    whole = np.arange(cfg.rows)
    for _ in range(runs):
        t0 = time.perf_counter()
        work(whole)
        one_s.append(time.perf_counter() - t0)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    nbytes = cfg.algorithmic_bytes()
    return {"value": round(gbps(nbytes, med(pool_s)), 3), "unit": "GB/s",
            "cores": threads, "threads": threads, "host_cpus": host, "cpus_available": avail,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "kind": "oracle",
            "ms_median": round(med(pool_s) * 1e3, 2), "ms_runs": [round(s * 1e3, 2) for s in pool_s],
            "sample": f"the full {cfg.name} batch ({cfg.rows} rows x {cfg.hidden}, {nbytes} "
                      f"algorithmic bytes) in {len(blocks)} contiguous row blocks over {threads} "
                      f"threads; {runs} runs of {passes} passes, median per-pass time; double "
                      f"arithmetic + rounding to bf16",
            "single_thread": {"value": round(gbps(nbytes, med(one_s)), 3), "unit": "GB/s",
                              "ms_median": round(med(one_s) * 1e3, 2),
                              "sample": f"the full batch on one thread, median of {runs} runs"},
            "cpu_model": model,
            "parity": oracle_parity(checks)}


def oracle_parity(checks: list, workers: int = 4) -> dict:
    """Part of the CPU-baseline leg: element-by-element check of every timed
    kernel's output against the CPU oracle on the whole batch, with the pass rule of the parity tests
    (one output ulp; for rotated and modulated outputs a floor scaled by the
    magnitude of the two cancelling terms).  `checks` holds (key, config,
    io dtype, host inputs, device output copied to the host)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import parity
    o = oracle.Oracle()

    def one(item):
        key, cfg, dtype, inp, got = item
        x = inp["x"].reshape(-1, cfg.hidden)
        mag = None
        if cfg.adaln:
            y, mag = o.rmsnorm_adaln(x, inp["w"], inp["scale"], inp["shift"], cfg.seq, cfg.eps,
                                     with_mag=True)
        elif cfg.rope:
            y, mag = o.rmsnorm_rope(x, inp["w"], inp["cos"], inp["sin"], cfg.heads,
                                    cfg.head_dim, cfg.eps, with_mag=True,
                                    interleaved=cfg.interleaved)
        else:
            y = o.rmsnorm(x, inp["w"], cfg.eps)
        ref32, ref = o.round(y, dtype)
        del y
        rep = parity.compare(got.reshape(-1), ref.reshape(-1), mag, ref32)
        rep.update(workload=cfg.name, io_dtype=dtype)
        return key, rep

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(workers) as ex:
        reps = dict(ex.map(one, checks))
    return {"all_pass": all(r["pass"] for r in reps.values()),
            "rule": "|gpu - oracle| <= 1 ulp of the output type (bf16/fp16), or 2^-20 (|ref| + m) "
                    "for fp32; a 2^-16 m floor where RoPE / AdaLN terms of magnitude m cancel",
            "seconds": round(time.perf_counter() - t0, 1),
            "workloads": reps}


def probe(kind: str, launches: int):
    """A short run of one workload for rocprofv3 (kernel traces and counter
    passes), with the benchmark's rotating buffer sets."""
    import torch
    dev = torch.device("cuda:0")
    s = torch.cuda.Stream()
    if kind in ("copy", "copy_nt"):
        cfg = datagen.CONFIGS[datagen.HEADLINE]
        wl = Workload(cfg, dev, s)
        n = cfg.rows * cfg.hidden
        if kind == "copy":  # the runtime's copy kernel: the counters' calibration
            with torch.cuda.stream(s):
                for i in range(launches):
                    wl.y[i % wl.nsets].copy_(wl.x[i % wl.nsets])
        else:
            import ceiling
            for i in range(launches):
                k = i % wl.nsets
                ceiling.copy(wl.y[k].data_ptr(), wl.x[k].data_ptr(), 2 * n // 16, ceiling.NT_COPY,
                             2, None, s.cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"probe": kind, "bytes_read": 2 * n, "bytes_written": 2 * n,
                          "launches": launches}), flush=True)
        return
    name, dtype = PROBES.get(kind, (kind, "bf16"))
    cfg = ALL_CONFIGS[name]
    wl = Workload(cfg, dev, s, dtype=dtype)
    for i in range(launches):
        wl.step(i)
    torch.cuda.synchronize()
    print(json.dumps({"probe": kind, "workload": cfg.name, "dtype": dtype, "launches": launches,
                      "rotating_sets": wl.nsets, "algorithmic_bytes": wl.nbytes,
                      "kernel": describe(cfg, dtype)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--windows", type=int, default=5,
                    help="timed windows of --steps launches each; the median is reported")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-rope", action="store_true",
                    help="skip the RoPE, AdaLN, other-dtype and general line items (the "
                         "headline and the pages' other RMSNorm shapes only)")
    ap.add_argument("--no-pages", action="store_true",
                    help="skip the pages' other RMSNorm shapes (one of them runs the headline's "
                         "kernel instance, which would merge the two in a per-kernel trace)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the copy-ceiling kernels (they would appear in a kernel trace)")
    ap.add_argument("--probe", choices=sorted(PROBES) + sorted(datagen.CONFIGS) + ["copy", "copy_nt"])
    ap.add_argument("--launches", type=int, default=10)
    ap.add_argument("--launch", choices=["stream", "graph"], default="stream",
                    help="issue the timed launches one by one on the stream (default) or as one "
                         "captured HIP graph")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; rows are independent, so a multi-GPU "
              "deployment shards rows across GPUs with no communication, and the one-GPU "
              "figure is the per-GPU throughput. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.probe:
        probe(args.probe, args.launches)
        return

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible; the HIP kernels are the only path", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    name = torch.cuda.get_device_name(0)
    clock = Clock(stream, windows=max(1, args.windows))
    graph = args.launch == "graph"

    def timed(rw, mode_graph=graph):
        return timing_fields(rw.time_steps(clock, args.steps, args.warmup, mode_graph), rw.nbytes)

    cfg = datagen.CONFIGS[datagen.HEADLINE]
    wl = Workload(cfg, dev, stream)
    head = timed(wl)
    other = timed(wl, not graph)  # the other launch mode
    checks = [("headline", cfg, "bf16", wl.host, wl.output())]
    value = head["value"]
    sec = head["ms_per_step"] * 1e-3
    traffic = read_traffic("rmsnorm", cfg.name)
    ceil = None if args.no_ceiling else copy_ceilings(clock, wl, args.steps, args.warmup)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / H100_GBPS_4x4096x3072, 3),
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq": cfg.seq,
                   "hidden": cfg.hidden, "io_dtype": "bf16", "eps": cfg.eps,
                   "bytes_per_step": cfg.algorithmic_bytes(), "rotating_sets": wl.nsets,
                   "seed": datagen.BASE_SEED, "x_fnv": datagen.fnv1a64(wl.host["x"]),
                   "w_fnv": datagen.fnv1a64(wl.host["w"]),
                   "device": name},
        "dtype_note": "dtype is the arithmetic type (binary32 accumulation and scaling); the "
                      "tensors are bf16 (config.io_dtype)",
        "timing": {"windows": clock.windows, "launches_per_window": args.steps,
                   "gpu_ms_median": head["gpu_ms_median"], "gpu_ms_min": head["gpu_ms_min"],
                   "gpu_ms_max": head["gpu_ms_max"], "hold_us": clock.hold_us,
                   "method": "HIP events on the launch stream around each window of --steps "
                             "launches, the stream held behind a spin kernel while the host "
                             "enqueues them; value and ms_per_step from the median window"},
        "pct_of_peak": round(pct_of_peak(value, HBM_PEAK_GBPS), 2),
        "roofline": {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": head["frac"],
                     "traffic": None if traffic is None else round(traffic / sec / 1e9, 2),
                     "kernel": "rmsnorm_kernel",
                     "launch_shape": describe(cfg),
                     "kernel_us": round(sec * 1e6, 3)},
        "baseline_note": "vs_baseline divides by the H100 figure for this shape on the "
                         "pages (0.157 ms = 1282.4 GB/s); another GPU, context only",
    }
    if ceil is not None:
        line["copy_ceiling"] = ceil
        line["pct_of_copy_ceiling"] = round(100.0 * value / ceil["value"], 2)
    if traffic is not None:
        fetched, written = read_traffic_parts("rmsnorm", cfg.name)
        line["roofline"]["traffic_bytes_per_launch"] = int(traffic)
        line["roofline"]["fetch_bytes_per_launch"] = int(fetched)
        line["roofline"]["write_bytes_per_launch"] = int(written)
    line["launch"] = ("one HIP graph of the K launches, replayed once per window"
                      if graph else "K launches issued one by one on the stream")
    line["graph_launch" if not graph else "stream_launch"] = other
    floor = launch_floor_us(stream)
    line["launch_floor_us"] = round(floor, 3)
    line["launch_floor_note"] = ("per-launch time of an empty kernel launched back to back on the "
                                 "same stream; each step pays it, so small workloads cannot reach "
                                 "the HBM rate (context, not subtracted from value)")
    host = wl.host
    del wl
    torch.cuda.empty_cache()

    # the other shapes of the pages' micro-benchmark table, in both launch modes
    line["pages_shapes"] = {}
    for wname in () if args.no_pages else ("rms_1x1024x2048", "rms_2x1024x2048", "rms_4x1024x2048",
                                           "rms_2x4096x3072_outliers"):
        rc = datagen.CONFIGS[wname]
        rw = Workload(rc, dev, stream)
        r = timed(rw)
        g = timed(rw, not graph)
        line["pages_shapes"][wname] = {
            "kernel": describe(rc), **r,
            ("graph" if not graph else "stream") + "_ms_per_step": g["ms_per_step"],
            "bytes_per_step": rw.nbytes, "rotating_sets": rw.nsets,
            "h100_ms_on_the_pages": H100_MS[wname]}
        checks.append((wname, rc, "bf16", rw.host, rw.output()))
        del rw
        torch.cuda.empty_cache()
    if not args.no_pages:
        line["pages_shapes"]["note"] = ("the smaller shapes take a few microseconds per launch, most "
                                        "of it the launch itself (launch_floor_us); graph replay "
                                        "removes the host-side issue cost")

    if not args.no_rope:
        for key, wname, kernel, dtype in (
                ("rope", datagen.ROPE, "rmsnorm_rope", "bf16"),
                ("rope_interleaved", datagen.ROPE_INTERLEAVED, "rmsnorm_rope_interleaved", "bf16"),
                ("adaln", datagen.ADALN, "rmsnorm_adaln", "bf16"),
                ("rms_f16", datagen.HEADLINE, "rmsnorm_f16", "f16"),
                ("rms_f32", datagen.HEADLINE, "rmsnorm_f32", "f32"),
                ("rope_f16", datagen.ROPE, "rmsnorm_rope_f16", "f16"),
                ("rope_f32", datagen.ROPE, "rmsnorm_rope_f32", "f32"),
                ("adaln_f32", datagen.ADALN, "rmsnorm_adaln_f32", "f32"),
                ("rope_large", "rope_4x4096x3072_h24d128", "rmsnorm_rope_large", "bf16"),
                ("rope_interleaved_large", "ropei_4x4096x3072_h24d128", "rmsnorm_rope_il_large", "bf16"),
                ("adaln_large", "adaln_4x4096x3072", "rmsnorm_adaln_large", "bf16")):
            rc = ALL_CONFIGS[wname]
            rw = Workload(rc, dev, stream, dtype=dtype)
            r = timed(rw)
            rtraffic = read_traffic(kernel, rc.name)
            line[key] = {"workload": rc.name, "io_dtype": dtype, "kernel": describe(rc, dtype), **r,
                         "bytes_per_step": rw.nbytes, "rotating_sets": rw.nsets,
                         "traffic": None if rtraffic is None
                         else round(rtraffic / (r["ms_per_step"] * 1e-3) / 1e9, 2)}
            checks.append((key, rc, dtype, rw.host, rw.output()))
            del rw
            torch.cuda.empty_cache()
        # shapes served by the kernels for rows of any length
        line["general"] = {}
        for wname, kernel, path in (
                ("rms_4x4096x3076", "rmsnorm_odd", "general one-pass"),
                ("rope_2x4096x1152_h16d72", "rmsnorm_rope_d72", "head-packed vector kernel"),
                ("rms_1x512x131072", "rmsnorm_long", "two-pass"),
                ("rms_1x64x1048576", "rmsnorm_split", "split rows, chunks over many workgroups"),
                ("rms_2x4096x24_d128", "rmsnorm_short", "short rows, several per wavefront"),
                ("adaln_8x4096x1152", "rmsnorm_adaln_seg", "segmented rows, several per wavefront")):
            rc = datagen.GENERAL_CONFIGS[wname]
            rw = Workload(rc, dev, stream)
            r = timed(rw)
            rtraffic = read_traffic(kernel, rc.name)
            line["general"][wname] = {
                "path": path, "kernel": describe(rc), **r, "bytes_per_step": rw.nbytes,
                "rotating_sets": rw.nsets,
                "traffic": None if rtraffic is None
                else round(rtraffic / (r["ms_per_step"] * 1e-3) / 1e9, 2)}
            checks.append((wname, rc, "bf16", rw.host, rw.output()))
            del rw
            torch.cuda.empty_cache()

    if not args.no_cpu:
        cb = cpu_baseline(cfg, host, checks)
        line["parity"] = cb.pop("parity")
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
