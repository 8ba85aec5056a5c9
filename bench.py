#!/usr/bin/env python3
"""Benchmark of the grouped MXFP8 scale rearrangement on one MI355X.

A step is one rearrangement launch over one batch of synthetic scales (group
scan, lookup, strip load, in-tile interleave, zero padding, stores and tail
fill all happen inside that launch). The headline workload is the large
K-groups case: scales (28672, 8192), 8 groups along K. The other four named
rearrangement workloads (M groups (131072, 44), (16640, 160) and (1024, 16); K
groups (7168, 4096)) are timed the same way in the same run and reported in
the `configs` block of the same line. `--workload` selects any other named
workload as the headline (per-expert scales, the casts, pad, the inverse).

Timing protocol (the same for every workload):
  * Inputs are uploaded once and rotated over enough copies of input and
    output (1 GiB by default, four times the 256 MB Infinity Cache) that a
    launch never finds its input in a cache left warm by a recent launch:
    step i uses copy i mod copies, and between two uses of one copy the
    other copies move at least 1 GiB through the caches.
  * The K timed launches (steps W .. W+K-1) are captured in one HIP graph (the
    pages' own K-groups benchmark timed CUDA graphs of 1000 launches), which
    is replayed once beforehand (one-time costs). The warm-up then replays a
    graph of one rotation pass, max(W, copies) launches, steps
    W - max(W, copies) .. W-1, back to back for at least --warm-ms of GPU time
    (20 ms): every copy is used, and the copy each timed launch uses was last
    used a whole rotation earlier — the state of a long run's steady rotation,
    in which nothing of it is cached but its pages are mapped and the clocks
    have settled under load (a warm-up of W launches on other copies only, or
    with a cache flush before the timed launches, measured 3-15% slower per
    launch at K = 20 than at K = 2000).
  * After a synchronisation a spin kernel holds the GPU while the host
    enqueues the timed replays behind it; HIP events on the launch stream
    bracket the K launches only, so host enqueue time stays outside the
    interval. `ms_per_step`, `value` and `roofline.achieved` all come from that
    one event interval; `wall_ms` is the host time between the two
    synchronisations around it (spin kernel included).

Two secondary figures come from the same run, outside that interval: `warm`
(launches back to back on one input/output copy, cache-resident when it fits)
and `cold` (eager launches, each after an in-place update and a read of a
512 MiB buffer that evict the MALL and the L2s, each between its own pair of
events: median, p10 and p90 per launch, dispatch included).

Bytes per step follow the pages' convention: every input scale byte read once
plus the whole output allocation written once.

Prints one JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (read+write) and µs per scale rearrange, M- and K-groups"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "k_groups_large"
# the other named rearrangement workloads, timed in the same run and reported beside the headline
SECONDARY = ("m_groups_skinny", "k_groups", "m_groups_experts", "m_groups_tiny")
# The pages' own times for the same scale shapes and operation (GPU not named on the pages):
# M groups (131072, 44), 19.46 us for the fallback CUDA kernel ("[mxfp8 moe training] fallback
# cuda kernel for when input doesn't meet 2d TMA constraints", Benchmarks table); K groups
# 7168 x 131072 and 28672 x 262144 data, i.e. scales (7168, 4096) and (28672, 8192), 49.08 and
# 315.47 us for the CuTeDSL kernel ("Add CuTeDSL MXFP8 K-groups scale rearrange kernel",
# realistic-shapes table).
PAGES_US = {"m_groups_skinny": 19.46, "k_groups": 49.08, "k_groups_large": 315.47}
# kernel instantiation per staging mode: 0 = M flat strips, 1 = M row segments,
# 3 = M narrow row segments, 2 = K column windows of rows on 128-byte lines (7: the same with
# 512-column windows, taken on MI355X for the (7168, 4096) shape; 6: rows at any other
# alignment), 4 = per-expert row segments, 5 = the same with 512 threads (grids of more than
# 2048 units); the second argument is true for kernels whose stores also carry sc1 (M and K
# launches that move more than 256 MiB), the third for grids of more than one pass over the GPU,
# whose row blocks are dealt to the XCDs in turn; quantize_dim1_kernel<SMALL, PAIR>: PAIR for two
# feature blocks per workgroup (the per-expert cast of K a multiple of 128)
KERNEL_NAMES = {"m_groups_tiny": "rearrange_kernel<3, false, false>",
                "m_groups_skinny": "rearrange_kernel<0, false, false>",
                "m_groups_experts": "rearrange_kernel<3, false, false>", "k_groups": "rearrange_kernel<7, false, false>",
                "k_groups_large": "rearrange_kernel<2, true, true>",
                "experts_3d_small": "rearrange_kernel<4, false, false>",
                "experts_3d_e16": "rearrange_kernel<4, false, false>",
                "experts_3d_e64": "rearrange_kernel<5, false, true>",
                "quant_m_groups_small": "quantize_dim0_kernel", "quant_m_groups": "quantize_dim0_kernel<true, true>",
                "quant_m_groups_skinny": "quantize_dim0_kernel<true, true>",
                "quant_k_groups_small": "quantize_dim1_kernel", "quant_k_groups": "quantize_dim1_kernel<true, false>",
                "pad_m_groups_small": "pad_kernel<true, true, true, false>",
                "pad_m_groups": "pad_kernel<true, true, true, true>",
                "inverse_m_groups_skinny": "unrearrange_kernel<false, true, false>",
                "inverse_k_groups_large": "unrearrange_kernel<true, true, true>",
                "quant_3d_small": "quantize_dim1_kernel", "quant_3d_e16": "quantize_dim1_kernel<true, true>"}
CSRC = os.path.join(ROOT, "group_scale_factor_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source(name):
    """The source file of the kernel a workload runs."""
    if name.startswith("pad"):
        return os.path.join(CSRC, "mx_pad.hip")
    if name.startswith("inverse"):
        return os.path.join(CSRC, "mx_unrearrange.hip")
    return os.path.join(CSRC, "mx_quantize.hip" if name.startswith("quant") else "mx_rearrange.hip")


def code_text(text):
    """Source text with comments removed and whitespace collapsed: what the compiler sees of it."""
    import re

    text = re.sub(rb"/\*.*?\*/", b" ", text, flags=re.S)
    text = re.sub(rb"//[^\n]*", b" ", text)
    return b" ".join(text.split())


def kernel_source_digest(name, read=None):
    """Digest of the code of the kernel's source file followed by the headers it includes from the same
    folder (comments and whitespace ignored). `read(path)` returns a file's bytes (default: the tree)."""
    import re

    if read is None:
        def read(path):
            with open(path, "rb") as f:
                return f.read()
    path = kernel_source(name)
    text = read(path)
    h = hashlib.sha256(code_text(text))
    for inc in re.findall(rb'#include "([^"]+)"', text):
        local = os.path.join(os.path.dirname(path), inc.decode())
        try:
            h.update(code_text(read(local)))
        except (OSError, KeyError):
            pass
    return h.hexdigest()[:16]


def align_up(x, a):
    return (x + a - 1) // a * a


INVERSE = ("inv_M", "inv_K")


def in_bytes_of(w):
    """Algorithmic bytes read per launch (the inverse: the rows*cols scale bytes the blocked layout holds)."""
    if w.kind == "pad" or w.kind in INVERSE:
        return w.rows * w.cols
    if w.kind in ("quant", "quant_k"):
        return 2 * w.rows * w.K
    if w.kind == "quant_3d":
        return 2 * w.experts * w.K * w.N
    return w.experts * w.rows * w.cols if w.kind == "3d" else w.rows * w.cols


def blocked_bytes_of(sizes, w):
    """Size of the blocked buffer the inverse reads (the forward layout's allocation); `sizes` is the
    binding module, which holds the size helpers of the C headers."""
    size_fn = sizes.mx_rearrange_M_groups_out_bytes if w.kind == "inv_M" else sizes.mx_rearrange_K_groups_out_bytes
    return int(size_fn(w.rows, w.cols, w.num_groups))


def out_bytes_of(sizes, w):
    """Bytes written per launch: the whole output allocation(s)."""
    if w.kind in INVERSE:
        return w.rows * w.cols
    if w.kind == "pad":
        return int(sizes.mx_pad_M_groups_out_rows(w.rows, w.num_groups)) * w.cols
    if w.kind == "quant":
        return w.rows * w.K + int(sizes.mx_quantize_dim0_M_groups_scale_bytes(w.rows, w.K, w.num_groups))
    if w.kind == "quant_k":
        return w.rows * w.K + int(sizes.mx_quantize_dim1_K_groups_scale_bytes(w.rows, w.K, w.num_groups))
    if w.kind == "quant_3d":
        return w.experts * w.N * w.K + int(sizes.mx_quantize_dim1_3d_scale_bytes(w.experts, w.K, w.N))
    if w.kind == "3d":
        return int(sizes.mx_rearrange_3d_out_bytes(w.experts, w.rows, w.cols))
    size_fn = sizes.mx_rearrange_M_groups_out_bytes if w.kind == "M" else sizes.mx_rearrange_K_groups_out_bytes
    return int(size_fn(w.rows, w.cols, w.num_groups))


class Job:
    """Device buffers and launches for one workload, rotating over `copies` input/output copies."""

    def __init__(self, name, rotate_bytes=1 << 30, max_copies=4096):
        import numpy as np
        import torch

        import group_scale_factor_amd as gsf
        import workloads

        self.torch = torch
        self.w = w = workloads.make(name)
        self.kind = w.kind
        lib = gsf.library()
        self.out_bytes = out_bytes_of(gsf, w)
        self.in_bytes = in_bytes_of(w)
        self.bytes_per_step = self.in_bytes + self.out_bytes
        self.copies = max(1, min(max_copies, math.ceil(rotate_bytes / max(self.bytes_per_step, 1))))
        self.in_alloc = blocked_bytes_of(gsf, w) if w.kind in INVERSE else self.in_bytes
        in_pitch = align_up(self.in_alloc, 256)
        # quant: codes, then the blocked scales from the next 256-byte boundary
        self.q_pitch = (align_up(w.rows * w.K, 256) if w.kind in ("quant", "quant_k")
                        else align_up(w.experts * w.N * w.K, 256) if w.kind == "quant_3d" else 0)
        out_pitch = align_up(self.out_bytes + self.q_pitch, 256)
        dev = torch.device("cuda")
        host = {"quant": lambda: w.x.view(np.uint8), "quant_k": lambda: w.x.view(np.uint8),
                "pad": lambda: w.data, "inv_M": lambda: w.blocked(self.in_alloc),
                "quant_3d": lambda: np.ascontiguousarray(w.w).view(np.uint8),
                "inv_K": lambda: w.blocked(self.in_alloc)}.get(w.kind, lambda: w.scales)()
        src = torch.from_numpy(np.ascontiguousarray(host).reshape(-1)).to(dev)
        self.inp = torch.empty(in_pitch * self.copies, dtype=torch.uint8, device=dev)
        self.outbuf = torch.empty(out_pitch * self.copies, dtype=torch.uint8, device=dev)
        for k in range(self.copies):
            self.inp[k * in_pitch: k * in_pitch + self.in_alloc].copy_(src)
        self.offs = torch.from_numpy(w.offs).to(dev) if w.kind not in ("3d", "quant_3d") else None
        self.outs = [self.outbuf[k * out_pitch: k * out_pitch + self.out_bytes] for k in range(self.copies)]
        self.in_ptrs = [self.inp.data_ptr() + k * in_pitch for k in range(self.copies)]
        self.out_ptrs = [self.outbuf.data_ptr() + k * out_pitch for k in range(self.copies)]
        self.fn = {"M": lib.mx_block_rearrange_M_groups, "K": lib.mx_block_rearrange_K_groups,
                   "3d": lib.mx_block_rearrange_3d, "quant": lib.mx_quantize_dim0_M_groups,
                   "quant_k": lib.mx_quantize_dim1_K_groups, "pad": lib.mx_pad_M_groups,
                   "inv_M": lib.mx_block_unrearrange_M_groups, "inv_K": lib.mx_block_unrearrange_K_groups,
                   "quant_3d": lib.mx_quantize_dim1_3d}[w.kind]
        self.error = gsf.RearrangeError
        torch.cuda.synchronize()

    def step(self, i, stream=None):
        """One launch on `stream` (default: torch's current stream), input/output copy i mod copies."""
        k = i % self.copies
        if stream is None:
            stream = self.torch.cuda.current_stream().cuda_stream
        w = self.w
        if w.kind == "3d":   # experts packed: expert stride rows*cols, row stride cols
            rc = self.fn(self.in_ptrs[k], w.experts, w.rows, w.cols, w.rows * w.cols, w.cols, self.out_ptrs[k],
                         stream or None)
        elif w.kind == "pad":
            rc = self.fn(self.in_ptrs[k], w.rows, w.cols, w.cols, self.offs.data_ptr(), w.num_groups,
                         self.out_ptrs[k], stream or None)
        elif w.kind == "quant_3d":   # experts packed: expert stride K*N, row stride N (elements)
            rc = self.fn(self.in_ptrs[k], w.experts, w.K, w.N, w.K * w.N, w.N, self.out_ptrs[k],
                         self.out_ptrs[k] + self.q_pitch, stream or None)
        elif w.kind in INVERSE:   # row-major output with row stride cols
            rc = self.fn(self.in_ptrs[k], w.rows, w.cols, self.offs.data_ptr(), w.num_groups, self.out_ptrs[k],
                         w.cols, stream or None)
        elif w.kind in ("quant", "quant_k"):   # rows x K bf16 (quant_k: T tokens x N features)
            rc = self.fn(self.in_ptrs[k], w.rows, w.K, w.K, self.offs.data_ptr(), w.num_groups, self.out_ptrs[k],
                         self.out_ptrs[k] + self.q_pitch, stream or None)
        else:
            rc = self.fn(self.in_ptrs[k], w.rows, w.cols, w.cols, self.offs.data_ptr(), w.num_groups,
                         self.out_ptrs[k], stream or None)
        if rc != 0:
            raise self.error(rc)


def capture(job, first, count):
    """A HIP graph of `count` launches: steps first .. first+count-1."""
    torch = job.torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(first, first + count):
                job.step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


class Spinner:
    """Holds the GPU busy for a given time with torch's spin kernel, so that work the host enqueues
    behind it starts only once all of it is queued."""

    def __init__(self):
        import torch

        self.torch = torch
        if not hasattr(torch.cuda, "_sleep"):
            raise RuntimeError("torch.cuda._sleep is needed to hold the GPU while the timed launches are enqueued")
        cycles = 1 << 20
        torch.cuda._sleep(cycles)   # first launch loads the kernel
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(cycles)
        e1.record()
        torch.cuda.synchronize()
        self.us_per_cycle = max(e0.elapsed_time(e1) * 1e3 / cycles, 1e-6)

    def hold(self, us):
        self.torch.cuda._sleep(int(us / self.us_per_cycle))


def timed_launches(job, K, W, spinner, eager=False, warm_ms=20.0):
    """Runs the warm-up and the K timed launches of `job` by the protocol of the module docstring.

    Returns (event seconds for the K launches, host wall seconds between the synchronisations around
    them, host seconds the first enqueue of the timed launches took, warm-up launches run)."""
    import time as _time

    torch = job.torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # one rotation pass: every copy once, ending right before the first timed step (step W)
    first_warm = W - max(W, job.copies)
    warm_steps = range(first_warm, W)
    if eager:
        for i in warm_steps:
            job.step(i)
        torch.cuda.synchronize()
        t0 = _time.perf_counter()
        spinner.hold(1000.0)
        ev0.record()
        for i in range(W, W + K):
            job.step(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3, _time.perf_counter() - t0, None, len(warm_steps)
    # one graph holds all K timed launches: a replay boundary inside the timed region would add a gap
    # (about 8 us each under the tracer, between graphs of a few launches)
    g = capture(job, W, K)
    g_warm = capture(job, first_warm, len(warm_steps))
    # one replay of each first (one-time costs), timing the host's enqueue of the timed graph and the
    # GPU time of a rotation pass
    t = _time.perf_counter()
    g.replay()
    enqueue_s = _time.perf_counter() - t
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    g_warm.replay()
    w1.record()
    torch.cuda.synchronize()
    # rotation passes back to back for at least warm_ms of GPU time (clocks settled under load; the
    # first short timed region of a process measured 1-2% slower without it), the last one ending
    # right before step W
    reps = max(1, math.ceil(warm_ms / max(w0.elapsed_time(w1), 1e-3)))
    for _ in range(reps):
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = _time.perf_counter()
    # hold the GPU while the host enqueues the replay behind the spin kernel
    spinner.hold(max(300.0, 4e6 * enqueue_s))
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / 1e3, _time.perf_counter() - t0, enqueue_s, (reps + 1) * len(warm_steps)


def launch_floor_us(spinner, count=500):
    """Graph-replay cost of an empty launch on this GPU (torch's spin kernel told to spin 0 cycles),
    timed like the workload's launches."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(count):
                torch.cuda._sleep(0)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spinner.hold(1000.0)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


def capture_same(job, count):
    """A HIP graph of `count` launches that all use input/output copy 0 (cache-resident when it fits)."""
    torch = job.torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(count):
                job.step(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def warm_figure(job, K, spinner):
    """Secondary figure: launches back to back on one input/output copy, which stays in the MALL and
    the L2s when it fits. Not an HBM figure."""
    torch = job.torch
    n_warm = min(K, 200)
    g_warm = capture_same(job, n_warm)
    g_warm.replay()
    torch.cuda.synchronize()
    ew0, ew1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spinner.hold(1000.0)
    ew0.record()
    g_warm.replay()
    ew1.record()
    torch.cuda.synchronize()
    warm_us = ew0.elapsed_time(ew1) * 1e3 / n_warm
    return {"us_per_launch": round(warm_us, 3), "GBps": round(job.bytes_per_step / warm_us / 1e3, 2),
            "launches": n_warm, "note": "one input/output copy reused: cache-resident when it fits, not an HBM figure"}


# Bytes of the buffer updated in place and read before each cold launch: more than the 256 MB MALL
# plus the eight 4 MB L2s, so nothing of the launch's input or output is left in a cache.
FLUSH_BYTES = 512 << 20
# Cold launches per workload (fewer for workloads that move more than the MALL holds, whose launches
# are long)
COLD_LAUNCHES, COLD_LAUNCHES_LARGE = 200, 50


def cold_figure(job, n, flush):
    """Secondary figure: per-launch times with the caches flushed before every launch.

    Before each launch `flush` (FLUSH_BYTES) is updated in place and then read once more: the update
    evicts the MALL and the L2s, and the read leaves them holding clean lines, so that the launch pays
    for no write-back of the flush's own data (measured after the update alone, the (28672, 8192)
    K-groups kernel took 105.7 us instead of 88.0). Each launch is eager, between its own pair of HIP
    events, so a pair holds one launch's dispatch and run, and nothing else. Reports the median, p10
    and p90 over the n launches; a rocprofv3 kernel trace of the same run gives the kernel's own
    durations."""
    import numpy as np

    torch = job.torch
    words = flush.view(torch.int64)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        flush.add_(1)
        torch.amax(words)
        a.record()
        job.step(i)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    med, p10, p90 = (float(np.percentile(us, q)) for q in (50, 10, 90))
    return {"us_median": round(med, 3), "us_p10": round(p10, 3), "us_p90": round(p90, 3),
            "GBps_median": round(job.bytes_per_step / med / 1e3, 2),
            "frac_median": round(job.bytes_per_step / med / 1e3 / HBM_PEAK_GBPS, 4),
            "launches": n, "flush_bytes": FLUSH_BYTES,
            "note": "MALL and L2s flushed (512 MiB written, then read) before each launch; one event pair per "
                    "eager launch (dispatch included)"}


def copy_calibration(args):
    """K plain device-to-device copies of the workload's input size (reads N, writes N bytes each)."""
    import torch

    import workloads

    w = workloads.make(args.workload)
    n = in_bytes_of(w)
    copies = max(2, min(4096, math.ceil((args.rotate_mib << 20) / (2 * n))))
    src = torch.randint(0, 255, (copies, n), dtype=torch.uint8, device="cuda")
    dst = torch.empty((copies, n), dtype=torch.uint8, device="cuda")
    for i in range(args.warmup):
        dst[i % copies].copy_(src[i % copies])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        dst[i % copies].copy_(src[i % copies])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(json.dumps({"copy_calibration": True, "bytes_read": n, "bytes_written": n, "steps": args.steps,
                      "us_per_copy": round(wall / args.steps * 1e6, 3)}), flush=True)


# Threads for the all-core oracle figure: the host cores one GPU's job may use.
MAX_CPU_THREADS = 16


def host_cpu():
    """CPU model name and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def _oracle_job(w):
    """(call, bytes per call, sample text) of the oracle on a bounded sample of workload w.

    `call()` runs the oracle once; it allocates its own outputs, so several
    threads may call it at once (the C oracle runs without the GIL). Bytes
    follow the GPU convention: input read once plus every output byte written,
    the output sizes taken from one call.
    """
    import numpy as np

    import oracle

    if w.kind == "quant":
        rows = min(w.rows, 512)
        x = w.x[:rows]
        call = lambda: oracle.quantize_dim0_M_groups(x, [rows])
        q, blocked = call()
        return (call, 2 * x.size + q.size + blocked.size,
                "the first %d of the %d rows of the %s workload (K = %d, one group)" % (rows, w.rows, w.name, w.K))
    if w.kind == "quant_k":
        cols = min(w.K, 64)
        x = np.ascontiguousarray(w.x[:, :cols])
        call = lambda: oracle.quantize_dim1_K_groups(x, [w.rows])
        qT, blocked = call()
        return (call, 2 * x.size + qT.size + blocked.size,
                "the first %d of the %d features of the %s workload (T = %d tokens, one group)"
                % (cols, w.K, w.name, w.rows))
    if w.kind == "pad":
        call = lambda: oracle.pad_M_groups(w.data, w.offs)
        return (call, w.data.size + call().size,
                "the %s workload (%dx%d bytes, %d groups)" % (w.name, w.rows, w.cols, w.num_groups))
    if w.kind == "quant_3d":
        cols = min(w.N, 64)
        x = np.ascontiguousarray(w.w[:1, :, :cols])
        call = lambda: oracle.quantize_dim1_3d(x)
        q, blocked = call()
        return (call, 2 * x.size + q.size + blocked.size,
                "the first %d of the %d features of expert 0 of the %s workload (K = %d)"
                % (cols, w.N, w.name, w.K))
    if w.kind in INVERSE:
        kind = w.kind[-1]
        blocked = w.blocked(oracle.out_bytes(kind, w.rows, w.cols, w.num_groups))
        call = lambda: oracle.unrearrange(kind, blocked, w.rows, w.cols, w.offs)
        return (call, 2 * w.rows * w.cols,
                "the %s workload (blocked -> %dx%d scales, %d groups)" % (w.name, w.rows, w.cols, w.num_groups))
    if w.kind == "3d":
        call = lambda: oracle.rearrange_3d(w.scales)
        return (call, in_bytes_of(w) + call().size,
                "the %s workload (%s scales, %d experts)" % (w.name, "x".join(map(str, w.scales.shape)), w.experts))
    call = lambda: oracle.rearrange(w.kind, w.scales, w.offs)
    return (call, in_bytes_of(w) + call().size,
            "the %s workload (%s scales, %d groups)" % (w.name, "x".join(map(str, w.scales.shape)), w.num_groups))


def _time_calls(call, seconds, threads):
    """Runs `call` in `threads` threads for about `seconds`; returns (calls, elapsed seconds)."""
    import threading

    stop = time.perf_counter() + seconds
    counts = [0] * threads

    def worker(k):
        while True:
            call()
            counts[k] += 1
            if time.perf_counter() >= stop:
                break

    t0 = time.perf_counter()
    ts = [threading.Thread(target=worker, args=(k,)) for k in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return sum(counts), time.perf_counter() - t0


def _threaded_call(w, threads):
    """One call of the oracle on the whole of workload w, shared among `threads` host threads, or None
    when the oracle has no threaded form for this kind of workload."""
    import oracle

    if w.kind not in ("M", "K"):
        return None
    return lambda: oracle.rearrange(w.kind, w.scales, w.offs, threads=threads)


def cpu_baseline(name, seconds, all_core_seconds=3.0):
    """The CPU oracle as it is, on (a bounded sample of) the same workload: single-threaded for about
    `seconds`; then, for about `all_core_seconds`, one call of the whole workload shared among one
    thread per host core (at most MAX_CPU_THREADS) over its (group, 128-row block) pieces, or, for
    workloads without that form, independent single-threaded copies run at once. Same byte
    convention as the GPU figure."""
    import workloads

    w = workloads.make(name)
    call, nbytes, what = _oracle_job(w)
    model, ncores = host_cpu()
    reps, el = _time_calls(call, seconds, 1)
    res = {
        "value": round(nbytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d runs over %s in %.1f s, single-threaded C oracle" % (reps, what, el),
        "us_per_call": round(el / reps * 1e6, 1),
        "host_cpu": model,
        "host_cores": ncores,
    }
    threads = min(ncores, MAX_CPU_THREADS)
    if all_core_seconds <= 0 or threads <= 1:
        return res
    one_call = _threaded_call(w, threads)
    if one_call is not None:
        one_call()   # first touch of the output pages outside the timed calls, as for the 1-core figure
        reps_mt, el_mt = _time_calls(one_call, all_core_seconds, 1)
        res["all_cores"] = {
            "value": round(nbytes * reps_mt / el_mt / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "us_per_call": round(el_mt / reps_mt * 1e6, 1),
            "sample": "%d calls over %s in %.1f s, each call shared among %d threads over its (group, "
                      "128-row block) pieces" % (reps_mt, what, el_mt, threads),
        }
    else:
        reps_mt, el_mt = _time_calls(call, all_core_seconds, threads)
        res["all_cores_copies"] = {
            "value": round(nbytes * reps_mt / el_mt / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "sample": "%d runs of the same sample, %d at a time (one thread each, unchanged oracle) in %.1f s"
                      % (reps_mt, threads, el_mt),
        }
    return res


def _counter_means(csv_path, counter, kernel_substring):
    """Mean per-dispatch value of `counter` over the dispatches whose name contains kernel_substring."""
    import csv

    vals = []
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and kernel_substring in row["Kernel_Name"]:
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise ValueError("no %s values for %s in %s" % (counter, kernel_substring, csv_path))
    return sum(vals) / len(vals), len(vals)


def summarize_pmc(name, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, commands):
    """HBM bytes per launch of the rearrange kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE runs.

    Each counter (KiB per dispatch) is scaled by what it reads for a plain
    device copy of known size (the --copy-calibration run), so the result is in
    bytes whatever the counter's unit or coverage on this GPU.
    """
    import workloads

    w = workloads.make(name)
    copy_bytes = in_bytes_of(w)
    kname = KERNEL_NAMES[name].split("<")[0]
    kfetch, nk = _counter_means(fetch_csv, "FETCH_SIZE", kname)
    kwrite, _ = _counter_means(write_csv, "WRITE_SIZE", kname)
    cfetch, nc = _counter_means(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cwrite, _ = _counter_means(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    fetch_scale = copy_bytes / cfetch      # bytes per counter unit
    write_scale = copy_bytes / cwrite
    read = kfetch * fetch_scale
    written = kwrite * write_scale
    import group_scale_factor_amd as gsf

    out_bytes = out_bytes_of(gsf, w)
    d = {
        "workload": name,
        "kernel": KERNEL_NAMES.get(name),
        "kernel_source": os.path.basename(kernel_source(name)),
        "kernel_source_sha256_16": kernel_source_digest(name),
        "dispatches_averaged": nk,
        "FETCH_SIZE_kib_per_dispatch": round(kfetch, 1),
        "WRITE_SIZE_kib_per_dispatch": round(kwrite, 1),
        "copy_calibration": {"bytes_read": copy_bytes, "bytes_written": copy_bytes, "dispatches": nc,
                             "FETCH_SIZE_kib": round(cfetch, 1), "WRITE_SIZE_kib": round(cwrite, 1),
                             "fetch_bytes_per_unit": round(fetch_scale, 2),
                             "write_bytes_per_unit": round(write_scale, 2)},
        "hbm_read_bytes_per_launch": round(read),
        "hbm_write_bytes_per_launch": round(written),
        "hbm_bytes_per_launch": round(read + written),
        "algorithmic_bytes_per_launch": copy_bytes + out_bytes,
        "traffic_over_algorithmic": round((read + written) / (copy_bytes + out_bytes), 4),
        "commands": commands,
    }
    path = os.path.join(PROFILES, "pmc_%s.json" % name)
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d))


def hbm_traffic(name, kind):
    """Measured HBM bytes per launch from the committed counter profile, if it matches this kernel."""
    path = os.path.join(PROFILES, "pmc_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_digest(name):
        return None
    return d.get("hbm_bytes_per_launch")


def config_of(w, job, args):
    """The `config` object of a workload's line."""
    return {
        "workload": w.name,
        "kind": {"3d": "per-expert", "quant": "MXFP8 dim0 cast, M-groups blocked scales",
                 "pad": "per-group row padding of MXFP8 data (M groups)",
                 "quant_k": "MXFP8 dim1 cast (tokens x features), K-groups blocked scales",
                 "inv_M": "inverse rearrangement (blocked -> row-major), M groups",
                 "inv_K": "inverse rearrangement (blocked -> row-major), K groups",
                 "quant_3d": "MXFP8 dim1 cast of stacked expert weights, per-expert codes and blocked scales"}.get(
            w.kind, "%s-groups" % w.kind),
        {"quant": "x_shape", "quant_k": "x_shape", "pad": "data_shape", "quant_3d": "w_shape"}.get(
            w.kind, "scales_shape"):
            [w.rows, w.K] if w.kind in ("quant", "quant_k") else (
                [w.experts, w.K, w.N] if w.kind == "quant_3d" else (
                    [w.rows, w.cols] if w.kind in ("pad",) + INVERSE else list(w.scales.shape))),
        "num_groups": w.experts if w.kind in ("3d", "quant_3d") else w.num_groups,
        "bytes_per_step": job.bytes_per_step,
        "rotating_copies": job.copies,
        "launch": "eager" if args.eager else "hip_graph",
        "parallelism": "single_gpu",
    }


def measure(name, K, W, args, spinner, floor_us, flush=None):
    """Times K launches of workload `name` (after W warm-up launches); returns (result fields, kind).
    With a flush buffer it also takes the cold figure."""
    import torch

    job = Job(name, rotate_bytes=args.rotate_mib << 20)
    gpu_s, wall, enqueue_s, warm_launches = timed_launches(job, K, W, spinner, eager=args.eager,
                                                           warm_ms=args.warm_ms)
    us_per_launch = gpu_s / K * 1e6
    achieved = job.bytes_per_step / (gpu_s / K) / 1e9
    warm = None if args.eager or args.no_warm else warm_figure(job, K, spinner)
    cold = None
    if flush is not None:
        cold = cold_figure(job, COLD_LAUNCHES_LARGE if job.bytes_per_step > (256 << 20) else COLD_LAUNCHES, flush)
    ideal_us = job.bytes_per_step / HBM_PEAK_GBPS / 1e3
    pages_us = PAGES_US.get(name)
    res = {
        "value": round(achieved, 2),
        "ms_per_step": round(us_per_launch / 1e3, 6),
        "us_per_launch": round(us_per_launch, 3),
        "steps": K,
        "warmup": W,
        "warmup_launches_run": warm_launches,
        "wall_ms": round(wall * 1e3, 3),
        "first_enqueue_us": round(enqueue_s * 1e6, 1) if enqueue_s is not None else None,
        "vs_baseline": round(pages_us / us_per_launch, 3) if pages_us else None,
        "config": config_of(job.w, job, args),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": hbm_traffic(name, job.kind),
            "kernel": KERNEL_NAMES.get(name),
            "avg_launch_us": round(us_per_launch, 3),
            "launch_floor_us": round(floor_us, 3) if floor_us is not None else None,
            "frac_ceiling": round(ideal_us / (floor_us + ideal_us), 4) if floor_us is not None else None,
        },
        "warm": warm,
        "cold": cold,
    }
    kind = job.kind
    del job
    torch.cuda.empty_cache()
    return res, kind


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--secondary", default=",".join(SECONDARY),
                    help="comma-separated workloads timed after the headline and reported in `configs` ('' for none)")
    ap.add_argument("--secondary-min-steps", type=int, default=200,
                    help="launches timed for each secondary workload: max(--steps, this)")
    ap.add_argument("--rotate-mib", type=int, default=1024, help="bytes of input+output rotated over")
    ap.add_argument("--warm-ms", type=float, default=20.0,
                    help="GPU time of the warm-up rotation passes before each timed region (at least one pass)")
    ap.add_argument("--eager", action="store_true", help="launch each step from Python instead of a graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time for the oracle baseline (0: skip)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the secondary cache-resident timing, the cold launches and the launch floor "
                         "(profiling runs: only the timed launches)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the secondary figure of launches with the caches flushed before each one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time torch's plain device copy of the workload's input size instead "
                         "(reference kernel of known traffic for the HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/pmc_<workload>.json from rocprofv3 counter_collection.csv files")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help="commands that produced the csv files")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc, commands=args.pmc_commands)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the rearrangement has no multi-GPU path "
              "(each GPU converts its own groups independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch

    from group_scale_factor_amd import _build

    if not os.path.exists(_build.LIBRARY):
        _build.build()
    import group_scale_factor_amd  # noqa: F401  (fails loudly if the HIP library is missing)

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args)
        return
    K, W = args.steps, args.warmup
    spinner = Spinner()
    # the fixed cost of one graph-replayed launch (outside every timed region; skipped when profiling)
    floor = launch_floor_us(spinner) if not args.eager and not args.no_warm else None
    # the buffer rewritten before each cold launch (outside every timed region of the main figure)
    flush = (torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
             if not args.no_warm and not args.no_cold else None)
    head, kind = measure(args.workload, K, W, args, spinner, floor, flush)
    configs = {}
    for name in [n for n in args.secondary.split(",") if n and n != args.workload]:
        r, _ = measure(name, max(K, args.secondary_min_steps), W, args, spinner, floor, flush)
        cfg = r["config"]
        configs[name] = {"us_per_launch": r["us_per_launch"], "value": r["value"], "unit": "GB/s",
                         "frac": r["roofline"]["frac"], "frac_ceiling": r["roofline"]["frac_ceiling"],
                         "traffic": r["roofline"]["traffic"], "kernel": r["roofline"]["kernel"],
                         "steps": r["steps"], "warmup": r["warmup"], "vs_baseline": r["vs_baseline"],
                         "scales_shape": cfg.get("scales_shape"), "num_groups": cfg["num_groups"],
                         "bytes_per_step": cfg["bytes_per_step"], "rotating_copies": cfg["rotating_copies"],
                         "cold": r["cold"]}
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "warmup_launches_run": head["warmup_launches_run"],
        "ms_per_step": head["ms_per_step"],
        "us_per_launch": head["us_per_launch"],
        "wall_ms": head["wall_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": head["vs_baseline"],
        "dtype": "bf16->e4m3 (f32 arithmetic)" if kind in ("quant", "quant_k", "quant_3d") else "u8",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "configs": configs,
        "warm": head["warm"],
        "cold": head["cold"],
        "first_enqueue_us": head["first_enqueue_us"],
        "cpu_baseline": None,
    }
    if not args.no_cpu and args.cpu_seconds > 0 and int(os.environ.get("RANK", "0")) == 0:
        res["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
