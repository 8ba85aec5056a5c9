"""Parity of the HIP library with the CPU oracle, byte for byte (GPU).

Every case prints its name before touching the GPU. The output buffer is
prefilled with 0xAB and followed by guard bytes, so a test also shows that the
kernel writes every byte of its output and nothing past it.
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


def _device_scales(torch, scales_np, misalign=0):
    """Upload a (rows, cols) host view (any row stride) to a device view whose base is misaligned by `misalign`."""
    rows, cols = scales_np.shape
    ld = scales_np.strides[0] if rows > 1 else cols
    ld = max(ld, cols)
    flat = np.zeros(misalign + rows * ld + 64, np.uint8)
    if rows and cols:
        dst = np.lib.stride_tricks.as_strided(flat[misalign:], shape=(rows, cols), strides=(ld, 1))
        dst[...] = scales_np
    buf = torch.from_numpy(flat).cuda()
    if rows == 0:
        return buf[misalign:misalign].view(0, cols) if cols else buf[:0].view(0, 0)
    return torch.as_strided(buf, (rows, cols), (ld, 1), misalign)


def run_case(env, kind, scales_np, offs_np, misalign=0, label=""):
    gsf, oracle, torch = env
    rows, cols = scales_np.shape
    G = len(offs_np)
    print("case", label, kind, "rows", rows, "cols", cols, "ld", scales_np.strides[0] if rows > 1 else cols,
          "G", G, "misalign", misalign, flush=True)
    want = oracle.rearrange(kind, scales_np, offs_np)
    n = want.size
    dev = _device_scales(torch, scales_np, misalign)
    offs = torch.from_numpy(np.asarray(offs_np, np.int32)).cuda()
    buf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    fn = gsf.mx_block_rearrange_M_groups if kind == "M" else gsf.mx_block_rearrange_K_groups
    out = fn(dev, offs, out=buf[:n])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert n == 0 or out.data_ptr() == buf.data_ptr()
    assert (got[n:] == POISON).all(), "%s: bytes past the output were written" % label
    if not np.array_equal(got[:n], want):
        bad = np.nonzero(got[:n] != want)[0]
        raise AssertionError("%s: %d of %d bytes differ, first at %d (got %d want %d)"
                             % (label, bad.size, n, bad[0], got[bad[0]], want[bad[0]]))
    return got[:n]


# --------------------------------------------------------------------------
# the five workloads, full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["m_groups_tiny", "m_groups_skinny", "m_groups_experts", "k_groups", "k_groups_large"])
def test_workload_bit_exact(env, name):
    import workloads

    w = workloads.make(name)
    run_case(env, w.kind, w.scales, w.offs, label=name)


# --------------------------------------------------------------------------
# hand-worked cases and tiny brute force
# --------------------------------------------------------------------------

def test_hand_worked_cases(env):
    import pins

    rng = np.random.default_rng(21)
    for case in pins.load_positions():
        A = rng.integers(1, 256, size=(case["rows"], case["cols"]), dtype=np.uint8)
        run_case(env, case["kind"], A, np.array(case["offs"], np.int32), label=case["name"])


def test_brute_force_tiny(env):
    import itertools

    rng = np.random.default_rng(22)
    for kind, total_dim in (("M", 0), ("K", 1)):
        for rows, cols in [(5, 3), (6, 9), (129, 7), (1, 9)]:
            total = (rows, cols)[total_dim]
            A = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
            for G in (1, 2, 3):
                for offs in itertools.combinations_with_replacement(range(total + 1), G):
                    run_case(env, kind, A, np.array(offs, np.int32), label="brute")


# --------------------------------------------------------------------------
# seeded fuzz: shapes, strides, misaligned bases, empty groups, many groups
# --------------------------------------------------------------------------

def _fuzz(env, kind, seed, n):
    import workloads

    rng = np.random.default_rng(seed)
    row_choices = [0, 1, 2, 31, 127, 128, 129, 255, 300, 513, 1000, 2049]
    col_choices = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 44, 45, 63, 64, 129, 160, 255, 256, 257, 300, 513, 1031]
    for i in range(n):
        rows = int(rng.choice(row_choices))
        cols = int(rng.choice(col_choices))
        extra = int(rng.choice([0, 0, 1, 3, 12, 13, 64]))
        ld = cols + extra
        G = int(rng.choice([1, 2, 3, 8, 16, 63, 64, 65, 130]))
        total = rows if kind == "M" else cols
        offs = workloads.random_offsets(rng, total, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.2))
        A = workloads.random_scales(rng, rows, cols, ld)
        run_case(env, kind, A, offs, misalign=int(rng.integers(0, 16)), label="fuzz%s-%d" % (kind, i))


def test_fuzz_M(env):
    _fuzz(env, "M", 31, 120)


def test_fuzz_K(env):
    _fuzz(env, "K", 32, 120)


def test_fuzz_K_line_aligned_rows(env):
    """K groups over rows that start on 128-byte lines (the streaming window path): widths spanning
    several column windows, group starts at any column (tiles straddling window edges), up to 130 groups."""
    import workloads

    rng = np.random.default_rng(34)
    for i in range(60):
        rows = int(rng.choice([1, 5, 127, 128, 129, 300, 1000]))
        cols = int(rng.choice([3, 100, 255, 256, 257, 259, 300, 513, 768, 1031, 2000, 4097]))
        ld = (cols + 127) // 128 * 128 + 128 * int(rng.choice([0, 0, 1, 7]))
        G = int(rng.choice([1, 2, 3, 8, 16, 64, 65, 130]))
        offs = workloads.random_offsets(rng, cols, G, p_empty=float(rng.choice([0.0, 0.3])),
                                        short_total=bool(rng.random() < 0.2))
        A = workloads.random_scales(rng, rows, cols, ld)
        run_case(env, "K", A, offs, misalign=0, label="fuzzK-lines-%d" % i)


def test_wide_random_sweep(env):
    """Thousands of random M and K cases (MX_SWEEP_CASES, default 2000): rows up to 3000, widths up to 2049,
    half of them on rows that start on 128-byte lines and half at any stride and base alignment, up to 300
    groups with empty groups and short totals; every byte and the guard bytes checked."""
    import workloads

    gsf, oracle, torch = env
    rng = np.random.default_rng(2026)
    cases = int(os.environ.get("MX_SWEEP_CASES", "2000"))
    print("case sweep of", cases, "random cases, seed 2026", flush=True)
    for i in range(cases):
        kind = "K" if i % 3 else "M"
        rows = int(rng.choice([1, 2, 63, 127, 128, 129, 255, 256, 300, 700, 1300, 3000]))
        if rng.random() < 0.7:
            cols = int(rng.integers(1, 1200))
        else:
            cols = int(rng.choice([255, 256, 257, 259, 511, 512, 513, 1024, 2049]))
        if rng.random() < 0.5:
            ld, misalign = (cols + 127) // 128 * 128 + 128 * int(rng.integers(0, 3)), 0
        else:
            ld, misalign = cols + int(rng.integers(0, 40)), int(rng.integers(0, 16))
        G = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 65, 100, 300]))
        offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G,
                                        p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.2))
        A = workloads.random_scales(rng, rows, cols, ld)
        want = oracle.rearrange(kind, A, offs)
        n = want.size
        dev = _device_scales(torch, A, misalign)
        buf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        fn = gsf.mx_block_rearrange_M_groups if kind == "M" else gsf.mx_block_rearrange_K_groups
        fn(dev, torch.from_numpy(offs).cuda(), out=buf[:n])
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        assert (got[n:] == POISON).all() and np.array_equal(got[:n], want), \
            "sweep case %d: %s rows %d cols %d ld %d misalign %d G %d" % (i, kind, rows, cols, ld, misalign, G)


@pytest.mark.parametrize("line_aligned", [True, False])
def test_k_window_edges(env, line_aligned):
    """K groups at the edges of the column windows, on rows that start on 128-byte lines and on rows that do
    not: a tile straddling a window edge, more than 64 groups inside one window, group starts on both sides of
    window boundaries, and windows that hold no group (offsets ending before the last column)."""
    import workloads

    rng = np.random.default_rng(35)
    cases = [
        (129, 259, [253, 259]),                                   # tile 253..256 straddles the first edge
        (130, 512, list(range(1, 201)) + [512]),                  # 200 one-column groups in the first window
        (128, 1000, [255, 256, 257, 511, 513, 1000]),             # starts on either side of 256 and 512
        (200, 700, [3, 3, 3, 130]),                               # windows past the last group
        (1, 300, [0, 0, 299]),                                    # one row, empty leading groups
        (257, 2049, [1, 2049]),                                   # every tile of the big group misaligned by 1
    ]
    for rows, cols, offs in cases:
        ld = ((cols + 127) // 128 * 128) if line_aligned else cols + 5
        A = workloads.random_scales(rng, rows, cols, ld)
        run_case(env, "K", A, np.array(offs, np.int32), misalign=0 if line_aligned else 3,
                 label="k-window-edges-%s" % ("lines" if line_aligned else "any"))


def test_k_wide_windows(env):
    """Shapes whose 256-column window grid needs a small second pass over the workgroups an MI355X holds at
    once (3 per CU) while the 512-column grid fits in one (2 per CU), so the library takes 512-column windows:
    random group widths, starts on either side of the 512-column window edges, tiles straddling them, empty
    groups, short totals, strided rows on 128-byte lines."""
    import workloads

    rng = np.random.default_rng(36)
    cases = [
        (7168, 4096, 4096, "random", 8),
        (7168, 3600, 3712, "random", 8),
        (6400, 4096, 4096, "random", 40),
        (5760, 4608, 4608, "random", 16),
        (7040, 4000, 4096, "edges", 0),
        (7168, 4096, 4224, "short", 8),
    ]
    for rows, cols, ld, how, G in cases:
        if how == "random":
            offs = workloads.random_offsets(rng, cols, G, p_empty=0.2, short_total=False)
        elif how == "edges":   # starts at, just before and just after multiples of 512, a 1-column group, empty ones
            offs = np.array([511, 512, 513, 1023, 1024, 1024, 1537, 1538, 2047, 2560, 3071, 3584, 3585, cols],
                            np.int32)
        else:
            offs = workloads.random_offsets(rng, cols, G, p_empty=0.0, short_total=True)
        A = workloads.random_scales(rng, rows, cols, ld)
        run_case(env, "K", A, offs, misalign=0, label="k-wide-windows-%dx%d-%s" % (rows, cols, how))


@pytest.mark.parametrize("kind", ["M", "K"])
def test_wide_and_odd_shapes(env, kind):
    rng = np.random.default_rng(33)
    for rows, cols, offs in [(300, 4097, [1000, 1000, 4097]), (130, 129, [64, 129]), (257, 4097, [4097]),
                             (1, 1, [1]), (128, 1025, [3, 700, 1025]), (1000, 600, [1, 2, 3, 599])]:
        offs = np.array(offs, np.int32)
        if kind == "M":
            offs = np.minimum(offs * rows // max(cols, 1), rows).astype(np.int32)
        A = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        run_case(env, kind, A, offs, misalign=int(rng.integers(0, 16)), label="wide")


def test_empty_inputs(env):
    gsf, oracle, torch = env
    # M with no rows: all groups empty, output all zero
    run_case(env, "M", np.zeros((0, 6), np.uint8), np.array([0, 0, 0], np.int32), label="M rows=0")
    # K with no columns: output all zero
    run_case(env, "K", np.zeros((5, 0), np.uint8), np.array([0, 0], np.int32), label="K cols=0")
    # nothing to write
    out = gsf.mx_block_rearrange_M_groups(torch.zeros((5, 0), dtype=torch.uint8, device="cuda"),
                                          torch.tensor([5], dtype=torch.int32, device="cuda"))
    assert out.numel() == 0


# --------------------------------------------------------------------------
# offsets that break the preconditions: clamped, never out of bounds
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["M", "K"])
def test_invalid_offsets_are_clamped(env, kind):
    rng = np.random.default_rng(34)
    for raw in ([50, 20, 400], [-5, 10, 10**6], [300, 0, 0], [2**31 - 1] * 3, [-(2**31)] * 2):
        rows, cols = 300, 45
        A = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        limit = rows if kind == "M" else cols
        clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw, np.int64), 0)), limit).astype(np.int32)
        gsf, oracle, torch = env
        want = oracle.rearrange(kind, A, clamped)
        n = want.size
        buf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        fn = gsf.mx_block_rearrange_M_groups if kind == "M" else gsf.mx_block_rearrange_K_groups
        print("case invalid offsets", kind, raw, flush=True)
        fn(torch.from_numpy(A).cuda(), torch.tensor(raw, dtype=torch.int32, device="cuda"), out=buf[:n])
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        assert (got[n:] == POISON).all()
        assert np.array_equal(got[:n], want)


# --------------------------------------------------------------------------
# determinism, streams, errors
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# launches that move more than 256 MiB run kernels whose stores also carry sc1
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind,rows,cols", [
    ("M", 1 << 20, 160),     # row segments, 336 MB per launch
    ("M", 6291456, 44),      # flat strips of packed 44-byte rows, 554 MB
    ("K", 20480, 8196),      # windows of rows that do not start on 128-byte lines, 336 MB
])
def test_launches_past_the_mall_size(env, kind, rows, cols):
    import workloads

    gsf, oracle, torch = env
    G = 8
    rng = np.random.default_rng(41)
    offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G, p_empty=0.25)
    size = gsf.mx_rearrange_M_groups_out_bytes if kind == "M" else gsf.mx_rearrange_K_groups_out_bytes
    assert rows * cols + size(rows, cols, G) > (256 << 20), "the case must take the kernels built for large launches"
    scales = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    run_case(env, kind, scales, offs, label="past the MALL size")


# --------------------------------------------------------------------------
# grids of more than one pass over the GPU (row blocks dealt to the XCDs in
# turn), below the size that takes the sc1 stores
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind,rows,cols,ld", [
    ("M", 1 << 18, 160, 160),    # row segments, 4112 units of 256 threads
    ("M", 1 << 20, 44, 44),      # flat strips, 8200 units
    ("M", 1 << 20, 32, 32),      # narrow row segments, 8200 units
    ("K", 14336, 8192, 8192),    # 256-column windows of line-aligned rows, 3696 units, 235 MB
    ("K", 8192, 8196, 8196),     # 128-column windows of other rows, 4224 units
])
def test_multi_pass_grids(env, kind, rows, cols, ld):
    import workloads

    gsf, oracle, torch = env
    G = 8
    rng = np.random.default_rng(43)
    offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G, p_empty=0.25)
    size = gsf.mx_rearrange_M_groups_out_bytes if kind == "M" else gsf.mx_rearrange_K_groups_out_bytes
    assert rows * cols + size(rows, cols, G) <= (256 << 20), "the case must stay below the sc1-store size"
    run_case(env, kind, workloads.random_scales(rng, rows, cols, ld), offs, label="multi-pass grid")


def test_multi_pass_fuzz(env):
    """Seeded random shapes whose grids take more than one pass over the GPU (row blocks dealt to the XCDs
    in turn): ragged row counts, packed and strided rows, bases off 16-byte and 128-byte lines, 1 to 200
    groups (tables past 64 groups), empty groups and short totals. A grid is multi-pass for certain when it
    has more units than 256 CUs x 2048 threads / its workgroup size; each case checks a lower bound on its
    unit count against that."""
    import workloads

    rng = np.random.default_rng(46)
    layouts = ["M flat", "M packed", "M strided", "K line-aligned", "K other"] * 2
    for i, layout in enumerate(layouts):
        kind = layout[0]
        G = int(rng.choice([1, 5, 8, 64, 65, 200]))
        misalign = int(rng.choice([0, 1, 4, 16, 128]))
        if kind == "M":
            # flat strips (packed rows of <= 60 bytes, not whole 16-byte pieces), packed rows of whole
            # pieces (row segments, narrow when chunked), rows with a stride
            cols = int(rng.choice({"M flat": [20, 33, 44, 60], "M packed": [32, 48, 96, 160],
                                   "M strided": [17, 44, 100, 160]}[layout]))
            ld = cols + (int(rng.choice([1, 4, 16, 36])) if layout == "M strided" else 0)
            rows = int(rng.integers(530_000, 800_000))
            assert rows // 128 > 4096
        else:
            cols = int(rng.integers(6000, 8300))
            rows = int(rng.integers(10240, 16000))
            if layout == "K line-aligned":
                ld, misalign = (cols + 127) // 128 * 128, int(rng.choice([0, 128]))
            else:
                ld = cols + int(rng.choice([0, 1, 5, 16]))
                if (ld % 128 == 0) and misalign % 128 == 0:
                    misalign = 4
            # more than 512 windows of 512 columns (so not the one-pass wide windows), hence more than
            # 1024 of 256 columns (512 threads) and 2048 of 128 columns (256 threads)
            assert (rows // 128) * (cols // 512) > 512
        offs = workloads.random_offsets(rng, rows if kind == "M" else cols, G, p_empty=0.25,
                                        short_total=bool(rng.random() < 0.2))
        run_case(env, kind, workloads.random_scales(rng, rows, cols, ld), offs, misalign=misalign,
                 label="multi-pass fuzz %d (%s)" % (i, layout))


def test_repeat_is_deterministic(env):
    import workloads

    gsf, oracle, torch = env
    for name in ("m_groups_experts", "k_groups"):
        w = workloads.make(name)
        print("case repeat", name, flush=True)
        s = torch.from_numpy(w.scales).cuda()
        o = torch.from_numpy(w.offs).cuda()
        fn = gsf.mx_block_rearrange_M_groups if w.kind == "M" else gsf.mx_block_rearrange_K_groups
        outs = [fn(s, o) for _ in range(3)]
        torch.cuda.synchronize()
        for x in outs[1:]:
            assert torch.equal(x, outs[0])


def test_side_stream(env):
    import workloads

    gsf, oracle, torch = env
    w = workloads.make("m_groups_tiny")
    print("case side stream", flush=True)
    s = torch.from_numpy(w.scales).cuda()
    o = torch.from_numpy(w.offs).cuda()
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        out = gsf.mx_block_rearrange_M_groups(s, o)
    st.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.rearrange("M", w.scales, w.offs))


def test_misaligned_out_is_rejected(env):
    gsf, oracle, torch = env
    s = torch.ones((4, 4), dtype=torch.uint8, device="cuda")
    o = torch.tensor([4], dtype=torch.int32, device="cuda")
    buf = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(gsf.RearrangeError) as e:
        gsf.mx_block_rearrange_M_groups(s, o, out=buf[8:])
    assert e.value.status == -4


def test_bench_launch_configuration(env):
    """The exact launches bench.py times (rotating buffers, its stream) give the oracle's bytes."""
    import bench

    gsf, oracle, torch = env
    for name in ("m_groups_skinny", "k_groups_large", "experts_3d_e64"):
        print("case bench config", name, flush=True)
        job = bench.Job(name, rotate_bytes=0)  # one copy: both launches write the same output
        job.step(0)
        job.step(1)
        torch.cuda.synchronize()
        if job.w.kind == "3d":
            want = oracle.rearrange_3d(job.w.scales)
        else:
            want = oracle.rearrange(job.w.kind, job.w.scales, job.w.offs)
        for k in range(min(2, job.copies)):
            assert np.array_equal(job.outs[k].cpu().numpy(), want)
