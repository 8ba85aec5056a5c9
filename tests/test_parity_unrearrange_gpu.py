"""Parity of the inverse rearrangement (blocked -> row-major) with the CPU oracle, byte for byte (GPU).

The blocked input is random bytes everywhere, padding included, so a kernel
that read a padding byte into the output would differ from the oracle. The
row-major output is a strided view (row stride >= cols, base at any alignment)
inside a buffer prefilled with 0xAB: the bytes between rows and past the last
row must keep that value. Every case prints its name before touching the GPU.
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


def run_inverse(env, kind, blocked_np, rows, cols, offs, ld=None, misalign=0, label=""):
    """GPU inverse of `blocked_np` into a poisoned strided view; returns the (rows, cols) result."""
    gsf, oracle, torch = env
    offs = np.asarray(offs, np.int32)
    ld = cols if ld is None else ld
    print("case inverse", label, kind, "rows", rows, "cols", cols, "ld", ld, "G", len(offs), "misalign", misalign,
          flush=True)
    want = oracle.unrearrange(kind, blocked_np, rows, cols, offs)
    blocked = torch.from_numpy(np.ascontiguousarray(blocked_np)).cuda()
    span = misalign + rows * ld
    buf = torch.full((span + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    out = torch.as_strided(buf, (rows, cols), (ld, 1), misalign)
    fn = gsf.mx_block_unrearrange_M_groups if kind == "M" else gsf.mx_block_unrearrange_K_groups
    fn(blocked, rows, cols, torch.from_numpy(offs).cuda(), out=out)
    torch.cuda.synchronize()
    flat = buf.cpu().numpy()
    got = np.lib.stride_tricks.as_strided(flat[misalign:], shape=(rows, cols), strides=(ld, 1)).copy()
    mask = np.ones(flat.size, bool)
    if rows and cols:
        np.lib.stride_tricks.as_strided(mask[misalign:], shape=(rows, cols), strides=(ld, 1))[...] = False
    assert (flat[mask] == POISON).all(), "%s: bytes outside the output rows were written" % label
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        r, c = bad[0]
        raise AssertionError("%s: %d of %d bytes differ, first at (%d, %d) (got %d want %d)"
                             % (label, len(bad), want.size, r, c, got[r, c], want[r, c]))
    return got


def random_blocked(rng, oracle, kind, rows, cols, G):
    n = oracle.out_bytes(kind, rows, cols, G)
    return rng.integers(0, 256, size=n, dtype=np.uint8)


# --------------------------------------------------------------------------
# the rearrangement workloads at full size, and round trips
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["m_groups_tiny", "m_groups_skinny", "m_groups_experts", "k_groups", "k_groups_large"])
def test_workload_round_trip(env, name):
    """rearrange (oracle) then inverse (GPU) gives the scales back, zeros where no group."""
    import workloads

    gsf, oracle, torch = env
    w = workloads.make(name)
    rows, cols = w.scales.shape
    blocked = oracle.rearrange(w.kind, w.scales, w.offs)
    got = run_inverse(env, w.kind, blocked, rows, cols, w.offs, label=name)
    end = int(w.offs[-1])
    keep = got[:end] if w.kind == "M" else got[:, :end]
    assert np.array_equal(keep, np.ascontiguousarray(w.scales)[:end] if w.kind == "M" else w.scales[:, :end])
    assert not (got[end:] if w.kind == "M" else got[:, end:]).any()


@pytest.mark.parametrize("name", ["m_groups_experts", "k_groups"])
def test_workload_random_blocked(env, name):
    import workloads

    gsf, oracle, torch = env
    w = workloads.make(name)
    rows, cols = w.scales.shape
    rng = np.random.default_rng(61)
    run_inverse(env, w.kind, random_blocked(rng, oracle, w.kind, rows, cols, len(w.offs)), rows, cols, w.offs,
                label=name + " random")


def test_gpu_forward_then_inverse(env):
    import workloads

    gsf, oracle, torch = env
    for name in ("m_groups_tiny", "k_groups"):
        w = workloads.make(name)
        rows, cols = w.scales.shape
        print("case forward+inverse", name, flush=True)
        s = torch.from_numpy(np.ascontiguousarray(w.scales)).cuda()
        o = torch.from_numpy(w.offs).cuda()
        fwd = gsf.mx_block_rearrange_M_groups if w.kind == "M" else gsf.mx_block_rearrange_K_groups
        inv = gsf.mx_block_unrearrange_M_groups if w.kind == "M" else gsf.mx_block_unrearrange_K_groups
        back = inv(fwd(s, o), rows, cols, o)
        torch.cuda.synchronize()
        end = int(w.offs[-1])
        want = np.zeros((rows, cols), np.uint8)
        if w.kind == "M":
            want[:end] = w.scales[:end]
        else:
            want[:, :end] = w.scales[:, :end]
        assert np.array_equal(back.cpu().numpy(), want)


# --------------------------------------------------------------------------
# seeded fuzz: shapes, output strides and alignments, empty and many groups
# --------------------------------------------------------------------------

def _fuzz(env, kind, seed, n):
    import workloads

    gsf, oracle, torch = env
    rng = np.random.default_rng(seed)
    row_choices = [1, 2, 31, 127, 128, 129, 255, 300, 513, 1000, 2049]
    col_choices = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 44, 45, 63, 64, 111, 112, 113, 129, 160, 224, 225, 300, 1031]
    for i in range(n):
        rows = int(rng.choice(row_choices))
        cols = int(rng.choice(col_choices))
        ld = cols + int(rng.choice([0, 0, 1, 3, 4, 12, 16, 64]))
        misalign = int(rng.choice([0, 0, 1, 2, 4, 8, 12, 15]))
        G = int(rng.choice([1, 2, 3, 8, 16, 63, 64, 65, 130]))
        total = rows if kind == "M" else cols
        offs = workloads.random_offsets(rng, total, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.3))
        run_inverse(env, kind, random_blocked(rng, oracle, kind, rows, cols, G), rows, cols, offs, ld=ld,
                    misalign=misalign, label="fuzz%s-%d" % (kind, i))


@pytest.mark.parametrize("kind,rows,cols,G", [("M", 1 << 20, 44, 8), ("K", 14336, 8192, 100)])
def test_multi_pass_grids(env, kind, rows, cols, G):
    # 8200 M units of 128 threads; 7168 K windows of 128 columns (the table of 100 groups in LDS):
    # more than the GPU holds at once, so row blocks are dealt to the XCDs in turn
    import workloads

    gsf, oracle, torch = env
    rng = np.random.default_rng(63)
    offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G, p_empty=0.25)
    run_inverse(env, kind, random_blocked(rng, oracle, kind, rows, cols, G), rows, cols, offs,
                label="multi-pass grid")


def test_multi_pass_fuzz(env):
    """Seeded random shapes whose inverse grids take more than one pass over the GPU: ragged row counts,
    output strides and bases of every kind, group tables in registers and in LDS. M units run 128 threads
    (more than 4096 units), K windows 512 or 256 threads (more than 1024 and 2048 units)."""
    import workloads

    gsf, oracle, torch = env
    rng = np.random.default_rng(64)
    for i in range(6):
        kind = "M" if i % 2 == 0 else "K"
        G = int(rng.choice([1, 8, 64, 65, 300]))
        if kind == "M":
            rows, cols = int(rng.integers(530_000, 800_000)), int(rng.choice([17, 44, 60, 100, 160]))
            assert rows // 128 > 4096
        else:
            rows, cols = int(rng.integers(10240, 16000)), int(rng.integers(6000, 8300))
            assert (rows // 128) * (cols // 256) > 1024
        ld = cols + int(rng.choice([0, 1, 4, 16, 128 - cols % 128]))
        misalign = int(rng.choice([0, 1, 4, 16, 128]))
        offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G, p_empty=0.25,
                                        short_total=bool(rng.random() < 0.2))
        run_inverse(env, kind, random_blocked(rng, oracle, kind, rows, cols, G), rows, cols, offs, ld=ld,
                    misalign=misalign, label="multi-pass fuzz %d" % i)


def test_fuzz_M(env):
    _fuzz(env, "M", 62, 100)


def test_fuzz_K(env):
    _fuzz(env, "K", 63, 100)


def test_random_sweep(env):
    """Random inverse cases (half of MX_SWEEP_CASES, default 1000): both groupings, rows up to 3000, widths
    up to 1300, output strides and base alignments of every kind, up to 300 groups, empty groups and short
    totals; every output byte and the poisoned bytes around the output rows checked."""
    import workloads

    gsf, oracle, torch = env
    rng = np.random.default_rng(2027)
    for i in range(int(os.environ.get("MX_SWEEP_CASES", "2000")) // 2):
        kind = "K" if i % 2 else "M"
        rows = int(rng.choice([1, 2, 63, 127, 128, 129, 300, 700, 3000]))
        cols = int(rng.integers(1, 1300))
        ld = cols + int(rng.choice([0, 0, 1, 3, 16, 128 - cols % 128]))
        G = int(rng.choice([1, 2, 3, 8, 16, 64, 65, 300]))
        offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G,
                                        p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.2))
        run_inverse(env, kind, random_blocked(rng, oracle, kind, rows, cols, G), rows, cols, offs, ld=ld,
                    misalign=int(rng.integers(0, 16)) if rng.random() < 0.5 else 0, label="sweep%d" % i)


def test_brute_force_tiny(env):
    import itertools

    gsf, oracle, torch = env
    rng = np.random.default_rng(64)
    for kind, total_dim in (("M", 0), ("K", 1)):
        for rows, cols in [(5, 3), (6, 9), (129, 7), (1, 9)]:
            total = (rows, cols)[total_dim]
            for G in (1, 2, 3):
                if total <= 12:
                    cases = itertools.combinations_with_replacement(range(total + 1), G)
                else:   # every split point would be too many launches: a seeded sample of them
                    cases = (np.sort(rng.integers(0, total + 1, size=G)) for _ in range(60))
                for offs in cases:
                    run_inverse(env, kind, random_blocked(rng, oracle, kind, rows, cols, G), rows, cols, offs,
                                label="brute")


def test_no_group_covers_anything(env):
    gsf, oracle, torch = env
    rng = np.random.default_rng(65)
    for kind in ("M", "K"):
        got = run_inverse(env, kind, random_blocked(rng, oracle, kind, 300, 45, 3), 300, 45, [0, 0, 0],
                          ld=47, misalign=3, label="all empty")
        assert not got.any()


def test_invalid_offsets_are_clamped(env):
    gsf, oracle, torch = env
    rng = np.random.default_rng(66)
    rows, cols = 300, 45
    for kind in ("M", "K"):
        limit = rows if kind == "M" else cols
        for raw in ([50, 20, 400], [-5, 10, 10**6], [300, 0, 0], [2**31 - 1] * 3, [-(2**31)] * 2):
            clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw, np.int64), 0)), limit)
            blocked = random_blocked(rng, oracle, kind, rows, cols, len(raw))
            want = oracle.unrearrange(kind, blocked, rows, cols, clamped.astype(np.int32))
            print("case inverse invalid offsets", kind, raw, flush=True)
            buf = torch.full((rows * cols + GUARD,), POISON, dtype=torch.uint8, device="cuda")
            fn = gsf.mx_block_unrearrange_M_groups if kind == "M" else gsf.mx_block_unrearrange_K_groups
            fn(torch.from_numpy(blocked).cuda(), rows, cols, torch.tensor(raw, dtype=torch.int32, device="cuda"),
               out=buf[: rows * cols].view(rows, cols))
            torch.cuda.synchronize()
            got = buf.cpu().numpy()
            assert (got[rows * cols:] == POISON).all()
            assert np.array_equal(got[: rows * cols].reshape(rows, cols), want)


def test_errors(env):
    gsf, oracle, torch = env
    o = torch.tensor([4], dtype=torch.int32, device="cuda")
    buf = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    with pytest.raises(gsf.RearrangeError) as e:   # blocked base not 16-byte aligned
        gsf.mx_block_unrearrange_M_groups(buf[4:], 4, 4, o)
    assert e.value.status == -4
    with pytest.raises(ValueError):                 # blocked smaller than the forward output
        gsf.mx_block_unrearrange_M_groups(buf[:100], 4, 4, o)
    assert gsf.mx_block_unrearrange_K_groups(buf, 0, 4, o).shape == (0, 4)


def test_bench_launch_configuration(env):
    """The exact launches bench.py times (its buffers, pitches and stream) give the oracle's bytes."""
    import bench

    gsf, oracle, torch = env
    for name in ("inverse_m_groups_skinny", "inverse_k_groups_large"):
        print("case bench config", name, flush=True)
        job = bench.Job(name, rotate_bytes=0)  # one copy: both launches write the same output
        job.step(0)
        job.step(1)
        torch.cuda.synchronize()
        w = job.w
        want = oracle.unrearrange(w.kind[-1], w.blocked(job.in_alloc), w.rows, w.cols, w.offs)
        assert np.array_equal(job.outs[0].cpu().numpy().reshape(w.rows, w.cols), want)
