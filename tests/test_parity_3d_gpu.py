"""Parity of the per-expert (3-D) entry point with the CPU oracle, byte for byte (GPU).

Every case prints its shape and strides before touching the GPU. The output
buffer is prefilled with 0xAB and followed by guard bytes, so each case also
shows that the kernel writes every byte of its output and nothing past it.
"""

import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GUARD = 4096
POISON = 0xAB


@pytest.fixture(scope="module")
def env():
    import torch

    from group_scale_factor_amd import _build
    import oracle

    if not os.path.exists(_build.LIBRARY):
        _build.build()
    if not os.path.exists(oracle.LIBRARY):
        oracle.build()
    import group_scale_factor_amd as gsf

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return gsf, oracle, torch


def host_experts(rng, E, rows, cols, ld=None, es=None):
    """(E, rows, cols) bytes in [1, 255] as a strided view with row stride ld and expert stride es."""
    ld = cols if ld is None else ld
    es = rows * ld if es is None else es
    n = max((E - 1) * es + rows * ld, 1) if E > 0 else 1
    base = rng.integers(1, 256, size=n, dtype=np.uint8)
    return np.lib.stride_tricks.as_strided(base, shape=(E, rows, cols), strides=(es, ld, 1))


def device_experts(torch, A, misalign=0):
    E, rows, cols = A.shape
    ld = max(A.strides[1] if rows > 1 else cols, cols)
    es = A.strides[0] if E > 1 else rows * ld
    span = (E - 1) * es + rows * ld if E * rows * cols > 0 else 0
    flat = np.zeros(misalign + span + 64, np.uint8)
    if span:
        np.lib.stride_tricks.as_strided(flat[misalign:], shape=(E, rows, cols), strides=(es, ld, 1))[...] = A
    buf = torch.from_numpy(flat).cuda()
    return torch.as_strided(buf, (E, rows, cols), (es, ld, 1), misalign)


def run_3d(env, A, misalign=0, label="", dev=None):
    gsf, oracle, torch = env
    E, rows, cols = A.shape
    print("case", label, "E", E, "rows", rows, "cols", cols, "strides", A.strides[:2], "misalign", misalign,
          flush=True)
    want = oracle.rearrange_3d(A)
    n = want.size
    if dev is None:
        dev = device_experts(torch, A, misalign)
    buf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    out = gsf.mx_block_rearrange_3d(dev, out=buf[:n])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert n == 0 or out.data_ptr() == buf.data_ptr()
    assert (got[n:] == POISON).all(), "%s: bytes past the output were written" % label
    if not np.array_equal(got[:n], want):
        bad = np.nonzero(got[:n] != want)[0]
        raise AssertionError("%s: %d of %d bytes differ, first at %d (got %d want %d)"
                             % (label, bad.size, n, bad[0], got[bad[0]], want[bad[0]]))
    return got[:n]


@pytest.mark.parametrize("name", ["experts_3d_small", "experts_3d_e16", "experts_3d_e64"])
def test_workload_bit_exact(env, name):
    import workloads

    w = workloads.make(name)
    run_3d(env, w.scales, label=name)


def test_brute_force_small_shapes(env):
    rng = np.random.default_rng(31)
    for E in (1, 2, 3):
        for rows in (1, 5, 127, 128, 129, 300):
            for cols in (1, 3, 4, 5, 8, 17, 44, 45, 160, 161):
                run_3d(env, host_experts(rng, E, rows, cols), label="brute")


def test_fuzz_strides_and_alignment(env):
    rng = np.random.default_rng(32)
    for it in range(120):
        E = int(rng.integers(1, 6))
        rows = int(rng.integers(1, 700))
        cols = int(rng.integers(1, 400))
        ld = cols + int(rng.choice([0, 0, 1, 3, 13, 64]))
        es = rows * ld + int(rng.choice([0, 0, 5, 64, 1000]))
        A = host_experts(rng, E, rows, cols, ld, es)
        run_3d(env, A, misalign=int(rng.integers(0, 16)), label="fuzz%d" % it)


def test_random_sweep(env):
    """Random per-expert cases (a fifth of MX_SWEEP_CASES, default 400): up to 9 experts, rows up to 1300,
    widths up to 700, padded row and expert strides, base alignments 0..15."""
    rng = np.random.default_rng(2028)
    for it in range(int(os.environ.get("MX_SWEEP_CASES", "2000")) // 5):
        E = int(rng.integers(1, 10))
        rows = int(rng.choice([1, 2, 127, 128, 129, 300, 1300]))
        cols = int(rng.integers(1, 700))
        ld = cols + int(rng.choice([0, 0, 1, 3, 13, 64]))
        es = rows * ld + int(rng.choice([0, 0, 5, 64, 1000]))
        A = host_experts(rng, E, rows, cols, ld, es)
        run_3d(env, A, misalign=int(rng.integers(0, 16)), label="sweep%d" % it)


def test_wide_rows_and_many_experts(env):
    rng = np.random.default_rng(33)
    # the last two run more than 2048 units (the 512-thread instantiation), with ragged rows in the last
    for E, rows, cols in [(1, 256, 1000), (2, 130, 4096), (128, 128, 160), (300, 3, 7), (1, 20000, 12),
                          (20, 16384, 8), (3, 100001, 45)]:
        run_3d(env, host_experts(rng, E, rows, cols), label="wide")


@pytest.mark.parametrize("E,rows,cols", [(24, 8192, 160), (96, 8192, 160)])
def test_multi_pass_grids(env, E, rows, cols):
    # 1536 units of 256 threads and 6144 units of 512 threads: more than the GPU holds at once, so
    # their row blocks are dealt to the XCDs in turn
    rng = np.random.default_rng(44)
    run_3d(env, host_experts(rng, E, rows, cols), label="multi-pass grid")


def test_experts_sharing_one_matrix(env):
    # expert stride 0: every expert reads the same matrix (an expanded view)
    gsf, oracle, torch = env
    rng = np.random.default_rng(34)
    one = rng.integers(1, 256, size=(1, 200, 37), dtype=np.uint8)
    A = np.broadcast_to(one, (4, 200, 37))
    dev = torch.from_numpy(np.ascontiguousarray(one)).cuda().expand(4, 200, 37)
    assert dev.stride(0) == 0
    got = run_3d(env, A, label="stride0", dev=dev)
    per = got.size // 4
    for e in range(1, 4):
        assert np.array_equal(got[e * per:(e + 1) * per], got[:per])


def test_empty_inputs(env):
    gsf, oracle, torch = env
    for shape in [(0, 5, 5), (3, 0, 5), (3, 5, 0), (0, 0, 0)]:
        print("case empty", shape, flush=True)
        dev = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        out = gsf.mx_block_rearrange_3d(dev)
        torch.cuda.synchronize()
        assert out.numel() == 0


def test_rejects_misaligned_out(env):
    gsf, oracle, torch = env
    print("case misaligned out", flush=True)
    dev = torch.ones((2, 4, 4), dtype=torch.uint8, device="cuda")
    buf = torch.zeros(2 * 512 + 32, dtype=torch.uint8, device="cuda")
    with pytest.raises(gsf.RearrangeError):
        gsf.mx_block_rearrange_3d(dev, out=buf[4:4 + 1024])


def test_repeat_and_side_stream(env):
    gsf, oracle, torch = env
    import workloads

    w = workloads.make("experts_3d_small")
    print("case repeat/side stream experts_3d_small", flush=True)
    want = oracle.rearrange_3d(w.scales)
    dev = device_experts(torch, w.scales)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = gsf.mx_block_rearrange_3d(dev)
        b = gsf.mx_block_rearrange_3d(dev)
    s.synchronize()
    assert np.array_equal(a.cpu().numpy(), want)
    assert np.array_equal(b.cpu().numpy(), want)
