"""Calls from several host threads at once, each on its own stream, give the oracle's bytes (GPU).

The headers state that calls are thread-safe. The library's host code keeps
per-device caches (the occupancy answer that picks a grid order) and raises the
LDS allowance of the kernels that stage more than 64 KB (the 512-column K
windows, the paired dim1 cast of expert weights) on first use. This test runs in
a fresh process, so those caches start empty and the first calls of every entry
point race one another: eight threads, each on its own torch stream, call every
entry point in a different order, three times over outputs poisoned before each
call, and compare every result byte for byte with the C oracle's. ctypes drops
the GIL for the duration of each library call, so the calls overlap on the host.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))

THREADED_CALLS = r"""
import sys
import threading

import numpy as np
import torch

import group_scale_factor_amd as gsf
import oracle
import pins
import workloads

THREADS, REPEATS = 8, 3
dev = torch.device("cuda")
cases = []          # (label, launch(outs), output shapes, wanted numpy arrays)


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16(bits):
    return gpu(bits.view(np.int16)).view(torch.bfloat16)


def add(label, launch, wants):
    cases.append((label, launch, [tuple(w.shape) for w in wants], [gpu(w) for w in wants]))


def strided(a, ld):
    # (rows, cols) uint8 on the GPU with row stride ld
    rows, cols = a.shape
    full = np.zeros((rows, ld), np.uint8)
    full[:, :cols] = a
    return gpu(full)[:, :cols]


# M and K groups on every staging path: packed flat strips, narrow chunks, wide row segments, the
# 512-column K windows of a one-pass grid (LDS allowance raised), 256-column and unaligned windows
rng = np.random.default_rng(2024)
for name in ("m_groups_skinny", "m_groups_experts", "k_groups"):
    w = workloads.make(name)
    s, o = gpu(w.scales), gpu(w.offs)
    fn = gsf.mx_block_rearrange_M_groups if w.kind == "M" else gsf.mx_block_rearrange_K_groups
    add(name, (lambda fn, s, o: lambda outs: fn(s, o, out=outs[0]))(fn, s, o),
        [oracle.rearrange(w.kind, np.ascontiguousarray(w.scales), w.offs)])
for kind, rows, cols, ld, G in (("M", 3000, 300, 307, 5), ("K", 1000, 1024, 1024, 7), ("K", 900, 1500, 1503, 9)):
    a = np.ascontiguousarray(workloads.random_scales(rng, rows, cols))
    total = rows if kind == "M" else cols
    offs = workloads.random_offsets(rng, total, G)
    s, o = strided(a, ld), gpu(offs)
    fn = gsf.mx_block_rearrange_M_groups if kind == "M" else gsf.mx_block_rearrange_K_groups
    add("%s %dx%d ld %d" % (kind, rows, cols, ld), (lambda fn, s, o: lambda outs: fn(s, o, out=outs[0]))(fn, s, o),
        [oracle.rearrange(kind, a, offs)])

w = workloads.make("experts_3d_small")
e3 = gpu(w.scales)
add("experts_3d_small", lambda outs: gsf.mx_block_rearrange_3d(e3, out=outs[0]),
    [oracle.rearrange_3d(np.ascontiguousarray(w.scales))])

# casts: dim0 into M groups, dim1 into K groups, dim1 of expert weights with paired feature blocks
w = workloads.make("quant_m_groups_small")
x0, o0 = bf16(w.x), gpu(w.offs)
add("dim0 cast", lambda outs: gsf.mx_quantize_dim0_M_groups(x0, o0, q=outs[0], scales=outs[1]),
    list(oracle.quantize_dim0_M_groups(w.x, w.offs)))
w = workloads.make("quant_k_groups_small")
x1, o1 = bf16(w.x), gpu(w.offs)
add("dim1 cast", lambda outs: gsf.mx_quantize_dim1_K_groups(x1, o1, qT=outs[0], scales=outs[1]),
    list(oracle.quantize_dim1_K_groups(w.x, w.offs)))
E, K, N = 3, 256, 300
wb = np.zeros((E, K, 304), np.uint16)
for e in range(E):
    wb[e, :, :N] = pins.random_bf16_rows(rng, K, N)
wt = bf16(wb)[:, :, :N]
add("dim1 cast of experts (paired blocks)", lambda outs: gsf.mx_quantize_dim1_3d(wt, q=outs[0], scales=outs[1]),
    list(oracle.quantize_dim1_3d(np.ascontiguousarray(wb[:, :, :N]))))

# pad and unpad of data rows, inverse rearrangement of both groupings
w = workloads.make("pad_m_groups_small")
d, od = gpu(w.data), gpu(w.offs)
padded = oracle.pad_M_groups(w.data, w.offs)
pg = gpu(padded)
add("pad", lambda outs: gsf.mx_pad_M_groups(d, od, out=outs[0]), [padded])
prows = w.rows
add("unpad", lambda outs: gsf.mx_unpad_M_groups(pg, prows, od, out=outs[0]),
    [oracle.unpad_M_groups(padded, prows, w.offs)])
for name in ("m_groups_experts", "k_groups"):
    f = workloads.make(name)
    blocked = oracle.rearrange(f.kind, np.ascontiguousarray(f.scales), f.offs)
    b, ob = gpu(blocked), gpu(f.offs)
    inv = gsf.mx_block_unrearrange_M_groups if f.kind == "M" else gsf.mx_block_unrearrange_K_groups
    add("inverse " + name, (lambda inv, b, ob, r, c: lambda outs: inv(b, r, c, ob, out=outs[0]))(
        inv, b, ob, f.rows, f.cols), [oracle.unrearrange(f.kind, blocked, f.rows, f.cols, f.offs)])

streams = [torch.cuda.Stream() for _ in range(THREADS)]
outs = [[[torch.empty(shape, dtype=torch.uint8, device=dev) for shape in c[2]] for c in cases]
        for _ in range(THREADS)]
torch.cuda.synchronize()
failures = []
start = threading.Barrier(THREADS)
count_lock = threading.Lock()
done = [0]


def worker(t):
    try:
        run(t)
    except BaseException as exc:   # a thread that dies must fail the run, not vanish
        failures.append("thread %d raised %r" % (t, exc))


def run(t):
    order = [(t * 5 + k) % len(cases) for k in range(len(cases))]
    if t % 2:
        order.reverse()
    with torch.cuda.stream(streams[t]):
        start.wait(timeout=120)
        for rep in range(REPEATS):
            for i in order:
                label, launch, _, wants = cases[i]
                for o in outs[t][i]:
                    o.fill_((0x5A + 17 * t + rep) & 0xFF)
                launch(outs[t][i])
                with count_lock:
                    done[0] += 1
            streams[t].synchronize()
            for i in order:
                label, _, _, wants = cases[i]
                for k, (o, want) in enumerate(zip(outs[t][i], wants)):
                    if not torch.equal(o, want):
                        failures.append("thread %d repeat %d %s output %d" % (t, rep, label, k))


threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
for th in threads:
    th.start()
for th in threads:
    th.join()
torch.cuda.synchronize()
print("threads %d, cases %d, repeats %d, calls %d" % (THREADS, len(cases), REPEATS, done[0]))
if failures or done[0] != THREADS * REPEATS * len(cases):
    print("\n".join(failures[:20]))
    sys.exit(1)
print("threaded calls: ok")
"""


def test_calls_from_many_threads_match_the_oracle():
    from group_scale_factor_amd import _build

    if not os.path.exists(_build.LIBRARY):
        _build.build()
    print("case threaded calls in a fresh process", flush=True)
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([ROOT, TESTS, os.environ.get("PYTHONPATH", "")]))
    res = subprocess.run([sys.executable, "-c", THREADED_CALLS], capture_output=True, text=True, timeout=300,
                         env=env, cwd=ROOT)
    print(res.stdout[-3000:])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert res.stdout.strip().endswith("threaded calls: ok")
