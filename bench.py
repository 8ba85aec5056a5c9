#!/usr/bin/env python3
"""Benchmark of the grouped MXFP8 scale rearrangement on one MI355X.

A step is one rearrangement launch over one batch of synthetic scales (group
scan, lookup, strip load, in-tile interleave, zero padding, stores and tail
fill all happen inside that launch). The default workload is the M-groups
skinny case: scales (131072, 44) with 44-byte rows, 8 groups. `--workload`
selects any of the other named workloads, including the per-expert (3-D)
weight scales, where a step is one launch over all experts.

Timing: inputs are resident in HBM before the timed region. Steps rotate over
enough copies of input and output (1 GiB by default, four times the 256 MB
Infinity Cache) that each step reads its input from HBM rather than from a
cache. The K timed steps are captured once in a HIP graph (the pages' own
K-groups benchmark timed CUDA graphs of 1000 launches) and replayed once
between two synchronisations; `--eager` launches them one by one instead.

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
DEFAULT_WORKLOAD = "m_groups_skinny"
# The pages' own figure for the same scale shape and operation, M groups at (131072, 44):
# 19.46 us for the fallback CUDA kernel ("[mxfp8 moe training] fallback cuda kernel for when
# input doesn't meet 2d TMA constraints", Benchmarks table). GPU not named on the page.
PAGES_US = {"m_groups_skinny": 19.46, "k_groups": 49.08, "k_groups_large": 315.47}
# kernel instantiation per staging mode: 0 = M flat strips, 1 = M row segments,
# 3 = M narrow row segments, 2 = K column windows of rows on 128-byte lines (6: rows at
# any other alignment), 4 = per-expert row segments, 5 = the same with 512 threads (grids
# of more than 2048 units)
KERNEL_NAMES = {"m_groups_tiny": "rearrange_kernel<3>", "m_groups_skinny": "rearrange_kernel<0>",
                "m_groups_experts": "rearrange_kernel<3>", "k_groups": "rearrange_kernel<2>",
                "k_groups_large": "rearrange_kernel<2>", "experts_3d_small": "rearrange_kernel<4>",
                "experts_3d_e16": "rearrange_kernel<4>", "experts_3d_e64": "rearrange_kernel<5>",
                "quant_m_groups_small": "quantize_dim0_kernel", "quant_m_groups": "quantize_dim0_kernel",
                "quant_m_groups_skinny": "quantize_dim0_kernel",
                "quant_k_groups_small": "quantize_dim1_kernel", "quant_k_groups": "quantize_dim1_kernel",
                "pad_m_groups_small": "pad_kernel<true, true, true>", "pad_m_groups": "pad_kernel<true, true, true>",
                "inverse_m_groups_skinny": "unrearrange_kernel<false, true>",
                "inverse_k_groups_large": "unrearrange_kernel<true, true>",
                "quant_3d_small": "quantize_dim1_kernel", "quant_3d_e16": "quantize_dim1_kernel"}
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


def blocked_bytes_of(lib, w):
    """Size of the blocked buffer the inverse reads (the forward layout's allocation)."""
    size_fn = lib.mx_rearrange_M_groups_out_bytes if w.kind == "inv_M" else lib.mx_rearrange_K_groups_out_bytes
    return int(size_fn(w.rows, w.cols, w.num_groups))


def out_bytes_of(lib, w):
    """Bytes written per launch: the whole output allocation(s)."""
    if w.kind in INVERSE:
        return w.rows * w.cols
    if w.kind == "pad":
        return int(lib.mx_pad_M_groups_out_rows(w.rows, w.num_groups)) * w.cols
    if w.kind == "quant":
        return w.rows * w.K + int(lib.mx_quantize_dim0_M_groups_scale_bytes(w.rows, w.K, w.num_groups))
    if w.kind == "quant_k":
        return w.rows * w.K + int(lib.mx_quantize_dim1_K_groups_scale_bytes(w.rows, w.K, w.num_groups))
    if w.kind == "quant_3d":
        return w.experts * w.N * w.K + int(lib.mx_quantize_dim1_3d_scale_bytes(w.experts, w.K, w.N))
    if w.kind == "3d":
        return int(lib.mx_rearrange_3d_out_bytes(w.experts, w.rows, w.cols))
    size_fn = lib.mx_rearrange_M_groups_out_bytes if w.kind == "M" else lib.mx_rearrange_K_groups_out_bytes
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
        self.out_bytes = out_bytes_of(lib, w)
        self.in_bytes = in_bytes_of(w)
        self.bytes_per_step = self.in_bytes + self.out_bytes
        self.copies = max(1, min(max_copies, math.ceil(rotate_bytes / max(self.bytes_per_step, 1))))
        self.in_alloc = blocked_bytes_of(lib, w) if w.kind in INVERSE else self.in_bytes
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
    """A HIP graph of `count` launches starting at step `first`."""
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


def launch_floor_us(count=500):
    """Graph-replay cost of an empty launch on this GPU (torch's spin kernel told to spin 0 cycles),
    timed like the workload's launches; None when torch offers no such kernel."""
    import torch

    if not hasattr(torch.cuda, "_sleep"):
        return None
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


def cpu_baseline(name, seconds, all_core_seconds=2.0):
    """The CPU oracle as it is, on (a bounded sample of) the same workload: single-threaded for about
    `seconds`, then one copy per host core at once for about `all_core_seconds` (independent runs of
    the unchanged oracle; their aggregate rate). Same byte convention as the GPU figure."""
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
    if all_core_seconds > 0 and threads > 1:
        reps_mt, el_mt = _time_calls(call, all_core_seconds, threads)
        res["all_cores"] = {
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

    out_bytes = out_bytes_of(gsf.library(), w)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate-mib", type=int, default=1024, help="bytes of input+output rotated over")
    ap.add_argument("--eager", action="store_true", help="launch each step from Python instead of a graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time for the oracle baseline (0: skip)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the secondary cache-resident timing (profiling runs: only the timed launches)")
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

    import torch

    from group_scale_factor_amd import _build

    if not os.path.exists(_build.LIBRARY):
        _build.build()
    import group_scale_factor_amd  # noqa: F401  (fails loudly if the HIP library is missing)

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args)
        return
    job = Job(args.workload, rotate_bytes=args.rotate_mib << 20)
    K, W = args.steps, args.warmup

    if args.eager:
        warm_launches = W
        for i in range(W):
            job.step(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for i in range(W, W + K):
            job.step(i)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # One graph covers one pass over the rotating copies (its first replay
        # is part of the warm-up); the timed region replays it back to back.
        chunk = min(job.copies, K)
        g = capture(job, 0, chunk)
        rem = K % chunk
        g_rem = capture(job, 0, rem) if rem else None
        warm_replays = max(1, math.ceil(W / chunk))
        for _ in range(warm_replays):
            g.replay()
        if g_rem is not None:
            g_rem.replay()
        warm_launches = warm_replays * chunk + rem
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(K // chunk):
            g.replay()
        if g_rem is not None:
            g_rem.replay()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    warm = None
    if not args.eager and not args.no_warm and K > 0:
        # secondary figure: the same launches back to back on one input/output
        # copy, which stays in the MALL/L2 when it fits (256 MB + 8 x 4 MB)
        n_warm = min(K, 200)
        g_warm = capture_same(job, n_warm)
        g_warm.replay()
        torch.cuda.synchronize()
        ew0, ew1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ew0.record()
        g_warm.replay()
        ew1.record()
        torch.cuda.synchronize()
        warm_us = ew0.elapsed_time(ew1) * 1e3 / n_warm
        warm = {"us_per_launch": round(warm_us, 3), "GBps": round(job.bytes_per_step / warm_us / 1e3, 2),
                "launches": n_warm, "note": "one input/output copy reused: cache-resident when it fits, "
                                            "not an HBM figure"}
    # the fixed cost of one graph-replayed launch, and the fraction of peak one launch of these bytes could
    # reach even if it moved them at the full peak rate (outside the timed region; skipped when profiling)
    floor = launch_floor_us() if not args.eager and not args.no_warm and K > 0 else None
    us_per_launch = gpu_s / K * 1e6
    value = job.bytes_per_step * K / wall / 1e9
    achieved = job.bytes_per_step / (gpu_s / K) / 1e9
    pages_us = PAGES_US.get(args.workload)
    w = job.w
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "warmup_launches_run": warm_launches,
        "ms_per_step": round(wall / K * 1e3, 6),
        "us_per_launch": round(us_per_launch, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(pages_us / (wall / K * 1e6), 3) if pages_us else None,
        "dtype": "bf16->e4m3 (f32 arithmetic)" if w.kind in ("quant", "quant_k", "quant_3d") else "u8",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
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
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": hbm_traffic(args.workload, w.kind),
            "kernel": KERNEL_NAMES.get(args.workload),
            "avg_launch_us": round(us_per_launch, 3),
            "launch_floor_us": round(floor, 3) if floor is not None else None,
            "frac_ceiling": (round((job.bytes_per_step / HBM_PEAK_GBPS / 1e3) /
                                   (floor + job.bytes_per_step / HBM_PEAK_GBPS / 1e3), 4)
                             if floor is not None else None),
        },
        "warm": warm,
        "cpu_baseline": None,
    }
    if not args.no_cpu and args.cpu_seconds > 0 and int(os.environ.get("RANK", "0")) == 0:
        res["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
