"""Sizes at the documented limits, byte for byte against the oracle (GPU).

The largest row stride each entry point accepts (and the first one it rejects),
thousands of groups (the group table scanned in many 64-lane slices), very wide
K rows and the largest group count of the casts. Every case prints its name
before touching the GPU; outputs carry poisoned guard bytes.
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


def strided(rng, rows, cols, ld):
    """(flat bytes, (rows, cols) view of them with row stride ld)."""
    base = rng.integers(0, 256, size=max((rows - 1) * ld + cols, 1), dtype=np.uint8)
    return base, np.lib.stride_tricks.as_strided(base, shape=(rows, cols), strides=(ld, 1))


def rearrange_case(env, kind, base_and_view, offs, label):
    gsf, oracle, torch = env
    base, scales = base_and_view
    rows, cols = scales.shape
    ld = scales.strides[0] if rows > 1 else cols
    print("case limits", label, kind, "rows", rows, "cols", cols, "ld", ld, "G", len(offs), flush=True)
    want = oracle.rearrange(kind, scales, np.asarray(offs, np.int32))
    n = want.size
    dev = torch.as_strided(torch.from_numpy(base).cuda(), (rows, cols), (ld, 1))
    buf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    fn = gsf.mx_block_rearrange_M_groups if kind == "M" else gsf.mx_block_rearrange_K_groups
    fn(dev, torch.tensor(np.asarray(offs, np.int32), device="cuda"), out=buf[:n])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert (got[n:] == POISON).all(), label
    assert np.array_equal(got[:n], want), label


def test_largest_row_stride(env):
    gsf, oracle, torch = env
    rng = np.random.default_rng(101)
    ld = 1 << 24                                       # the largest stride the rearrangement accepts
    for kind, offs in (("M", [1, 3]), ("K", [2, 7])):
        rearrange_case(env, kind, strided(rng, 3, 7, ld), offs, "row stride 2^24")
    s = torch.zeros(16, dtype=torch.uint8, device="cuda")
    o = torch.tensor([2], dtype=torch.int32, device="cuda")
    out = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    lib = gsf.library()
    for fn in (lib.mx_block_rearrange_M_groups, lib.mx_block_rearrange_K_groups):
        assert fn(s.data_ptr(), 2, 4, (1 << 24) + 1, o.data_ptr(), 1, out.data_ptr(), None) == -2


def test_thousands_of_groups(env):
    rng = np.random.default_rng(102)
    # M: 10000 groups over 3000 rows, most of them empty
    ends = np.sort(rng.integers(0, 3001, size=10000)).astype(np.int32)
    ends[-1] = 3000
    rearrange_case(env, "M", strided(rng, 3000, 13, 13), ends, "M 10000 groups")
    # K: 5000 groups over 6000 scale columns of 130 rows
    ends = np.sort(rng.integers(0, 6001, size=5000)).astype(np.int32)
    ends[-1] = 6000
    rearrange_case(env, "K", strided(rng, 130, 6000, 6003), ends, "K 5000 groups")


def test_very_wide_k_rows(env):
    rng = np.random.default_rng(103)
    rearrange_case(env, "K", strided(rng, 129, 65537, 65541), [1, 30001, 30001, 65537], "K 65537 columns")
    # rows on 128-byte lines (the streaming window path): 257 windows per row block
    rearrange_case(env, "K", strided(rng, 129, 65539, 65664), [1, 30001, 30002, 65539], "K 65539 columns, lines")


def test_inverse_most_groups(env):
    """The inverse calls at their group limit (4096): the scanned table of more than 64 groups sits in LDS
    beside the strip, and most groups are empty."""
    gsf, oracle, torch = env
    rng = np.random.default_rng(105)
    for kind, rows, cols in (("M", 3000, 13), ("K", 130, 6000)):
        n = rows if kind == "M" else cols
        ends = np.sort(rng.integers(0, n + 1, size=4096)).astype(np.int32)
        ends[-1] = n
        blocked = rng.integers(0, 256, size=oracle.out_bytes(kind, rows, cols, 4096), dtype=np.uint8)
        want = oracle.unrearrange(kind, blocked, rows, cols, ends)
        print("case limits inverse", kind, "4096 groups", flush=True)
        fn = gsf.mx_block_unrearrange_M_groups if kind == "M" else gsf.mx_block_unrearrange_K_groups
        got = fn(torch.from_numpy(blocked).cuda(), rows, cols, torch.from_numpy(ends).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), want), kind


def test_inverse_and_pad_largest_strides(env):
    gsf, oracle, torch = env
    rng = np.random.default_rng(104)
    rows, cols, ld = 3, 9, (1 << 22) + 5               # a large, odd output row stride
    offs = np.array([1, 3], np.int32)
    for kind in ("M", "K"):
        o = offs if kind == "M" else np.array([4, 9], np.int32)
        blocked = rng.integers(0, 256, size=oracle.out_bytes(kind, rows, cols, 2), dtype=np.uint8)
        want = oracle.unrearrange(kind, blocked, rows, cols, o)
        print("case limits inverse", kind, "ld", ld, flush=True)
        buf = torch.full(((rows - 1) * ld + cols + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        out = torch.as_strided(buf, (rows, cols), (ld, 1))
        fn = gsf.mx_block_unrearrange_M_groups if kind == "M" else gsf.mx_block_unrearrange_K_groups
        fn(torch.from_numpy(blocked).cuda(), rows, cols, torch.from_numpy(o).cuda(), out=out)
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        for r in range(rows):
            assert np.array_equal(got[r * ld: r * ld + cols], want[r]), (kind, r)
        keep = np.ones(got.size, bool)
        for r in range(rows):
            keep[r * ld: r * ld + cols] = False
        assert (got[keep] == POISON).all(), kind
    # pad: input rows 2^22 + 5 bytes apart
    base, data = strided(rng, 3, 9, ld)
    want = oracle.pad_M_groups(data, offs)
    print("case limits pad ld", ld, flush=True)
    got = gsf.mx_pad_M_groups(torch.as_strided(torch.from_numpy(base).cuda(), (3, 9), (ld, 1)),
                              torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


def test_cast_group_limits(env):
    gsf, oracle, torch = env
    import pins

    rng = np.random.default_rng(105)
    # dim1 cast: the largest group count (2048), many of them empty; one past it is rejected
    T, N = 64 * 32, 40
    x = pins.random_bf16_rows(rng, T, N, ld=48)
    ends = (32 * np.sort(rng.integers(0, T // 32 + 1, size=2048))).astype(np.int32)
    ends[-1] = T
    want_q, want_s = oracle.quantize_dim1_K_groups(x, ends)
    print("case limits dim1 2048 groups", flush=True)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    q, s = gsf.mx_quantize_dim1_K_groups(xd, torch.from_numpy(ends).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), want_q) and np.array_equal(s.cpu().numpy(), want_s)
    too_many = torch.from_numpy(np.full(2049, T, np.int32)).cuda()
    with pytest.raises(gsf.RearrangeError) as e:
        gsf.mx_quantize_dim1_K_groups(xd, too_many)
    assert e.value.status == -3


def test_grid_stride_loop(env):
    """More than 2^20 work units: the grid is capped and each workgroup loops over several units (with a
    barrier between them). One-column matrices keep the bytes modest: M groups (flat strips), K groups (the
    window path) and per-expert matrices, each checked byte for byte."""
    gsf, oracle, torch = env
    rng = np.random.default_rng(106)
    # M: ceil(rows/128) + G row blocks = 1048582 units
    rows = 128 * (1 << 20) + 300
    scales = rng.integers(1, 256, size=(rows, 1), dtype=np.uint8)
    rearrange_case(env, "M", (scales.reshape(-1), scales), [1000, 70000000, rows], "M grid-stride")
    del scales
    # K: 524289 row blocks x (1 window + 1 tail unit) = 1048578 units
    rows = (1 << 26) + 7
    scales = rng.integers(1, 256, size=(rows, 2), dtype=np.uint8)
    rearrange_case(env, "K", (scales.reshape(-1), scales), [1, 2], "K grid-stride")
    del scales
    # per-expert: one expert of 1048577 row blocks
    rows = 128 * (1 << 20) + 3
    A = rng.integers(1, 256, size=(1, rows, 1), dtype=np.uint8)
    print("case limits 3-D grid-stride rows", rows, flush=True)
    want = oracle.rearrange_3d(A)
    buf = torch.full((want.size + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    gsf.mx_block_rearrange_3d(torch.from_numpy(A).cuda(), out=buf[:want.size])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert (got[want.size:] == POISON).all() and np.array_equal(got[:want.size], want), "3-D grid-stride"
