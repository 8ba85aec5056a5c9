"""Parity of per-group row padding and unpadding with the CPU oracle, byte for byte (GPU).

Every case prints its shape before touching the GPU; outputs are prefilled with
0xAB and followed by guard bytes (every byte written, none past it).
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


def upload(torch, data, ld=None, misalign=0):
    """(rows, cols) bytes as a device view with row stride ld and base misaligned by `misalign`."""
    rows, cols = data.shape
    ld = cols if ld is None else ld
    flat = np.zeros(misalign + max(rows, 1) * ld + 64, np.uint8)
    if rows and cols:
        np.lib.stride_tricks.as_strided(flat[misalign:], shape=(rows, cols), strides=(ld, 1))[...] = data
    buf = torch.from_numpy(flat).cuda()
    return torch.as_strided(buf, (rows, cols), (ld, 1), misalign)


def compare(label, got, want):
    if not np.array_equal(got, want):
        bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
        raise AssertionError("%s: %d of %d bytes differ, first at %d" % (label, bad.size, want.size, bad[0]))


def run_pad(env, data, offs, ld=None, misalign=0, label=""):
    gsf, oracle, torch = env
    rows, cols = data.shape
    offs = np.asarray(offs, np.int32)
    print("case pad", label, "rows", rows, "cols", cols, "ld", ld or cols, "G", len(offs), "misalign", misalign,
          flush=True)
    want = oracle.pad_M_groups(data, offs)
    n = want.size
    buf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    out = buf[:n].view(want.shape)
    dev_offs = torch.from_numpy(offs).cuda()
    gsf.mx_pad_M_groups(upload(torch, data, ld, misalign), dev_offs, out=out)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert (got[n:] == POISON).all(), "%s: bytes past the padded output were written" % label
    compare(label + " pad", got[:n], want.reshape(-1))
    # and back: unpad into a strided, misaligned view
    print("case unpad", label, flush=True)
    base_ld = ld or cols
    uld = base_ld if (misalign == 0 and base_ld % 16 == 0) else base_ld + 3   # 16-byte path or byte path
    ubuf = torch.full((misalign + max(rows, 1) * uld + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    uview = torch.as_strided(ubuf, (rows, cols), (uld, 1), misalign)
    gsf.mx_unpad_M_groups(out, rows, dev_offs, out=uview)
    torch.cuda.synchronize()
    got_u = ubuf.cpu().numpy()
    want_u = oracle.unpad_M_groups(want, rows, offs)
    if rows and cols:
        view = np.lib.stride_tricks.as_strided(got_u[misalign:], shape=(rows, cols), strides=(uld, 1))
        compare(label + " unpad", np.ascontiguousarray(view), want_u)
    # bytes outside the rows' cols stay untouched
    mask = np.ones(got_u.size, bool)
    if rows and cols:
        idx = misalign + (np.arange(rows)[:, None] * uld + np.arange(cols)[None, :]).reshape(-1)
        mask[idx] = False
    assert (got_u[mask] == POISON).all(), "%s: unpad wrote outside its rows" % label


@pytest.mark.parametrize("name", ["pad_m_groups_small", "pad_m_groups"])
def test_workloads(env, name):
    import workloads

    w = workloads.make(name)
    run_pad(env, w.data, w.offs, label=name)


@pytest.mark.parametrize("ld,G", [(5120, 80), (5123, 8)])
def test_multi_pass_grids(env, ld, G):
    # (16640, 5120) rows with 80 groups (table in LDS) on the 16-byte path, and 8 groups with a row stride
    # that takes the byte path: more workgroups than the GPU holds at once, dealt to the XCDs in turn
    import workloads

    rng = np.random.default_rng(62)
    data = rng.integers(0, 256, size=(16640, 5120), dtype=np.uint8)
    offs = workloads.random_offsets(rng, 16640, G, p_empty=0.25)
    run_pad(env, data, offs, ld=ld, label="multi-pass grid")


def test_fuzz_aligned_and_unaligned(env):
    import workloads

    rng = np.random.default_rng(80)
    for i in range(60):
        rows = int(rng.choice([0, 1, 2, 127, 128, 129, 300, 700]))
        cols = int(rng.choice([1, 5, 16, 48, 100, 1024, 1040, 2049, 5120]))
        aligned = rng.random() < 0.6
        ld = (cols + 15) // 16 * 16 + 16 * int(rng.integers(0, 3)) if aligned else cols + int(rng.integers(0, 5))
        misalign = 0 if aligned else int(rng.integers(0, 16))
        G = int(rng.choice([1, 2, 3, 8, 16, 64, 65, 100]))
        offs = workloads.random_offsets(rng, rows, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.3))
        data = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        run_pad(env, data, offs, ld=ld, misalign=misalign, label="fuzz%d" % i)


def test_random_sweep(env):
    """Random pad/unpad cases (a fifth of MX_SWEEP_CASES, default 400): rows up to 3000, widths up to
    5120, 16-byte aligned and unaligned strides and bases, up to 300 groups, empty groups, short totals."""
    import workloads

    rng = np.random.default_rng(2029)
    for i in range(int(os.environ.get("MX_SWEEP_CASES", "2000")) // 5):
        rows = int(rng.choice([0, 1, 2, 127, 128, 129, 300, 700, 3000]))
        cols = int(rng.integers(1, 5121)) if rng.random() < 0.5 else int(rng.choice([16, 48, 1024, 5120]))
        aligned = rng.random() < 0.5
        ld = (cols + 15) // 16 * 16 + 16 * int(rng.integers(0, 3)) if aligned else cols + int(rng.integers(0, 5))
        misalign = 0 if aligned else int(rng.integers(0, 16))
        G = int(rng.choice([1, 2, 3, 8, 16, 64, 65, 300]))
        offs = workloads.random_offsets(rng, rows, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.3))
        data = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        run_pad(env, data, offs, ld=ld, misalign=misalign, label="sweep%d" % i)


def test_invalid_offsets_are_clamped(env):
    gsf, oracle, torch = env
    rng = np.random.default_rng(81)
    rows, cols = 300, 64
    data = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    for raw in ([50, 20, 400], [-5, 10, 10**6], [300, 0, 0], [2**31 - 1] * 3, [-(2**31)] * 2):
        clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw, np.int64), 0)), rows).astype(np.int32)
        want = oracle.pad_M_groups(data, clamped)
        print("case pad invalid offsets", raw, flush=True)
        out = gsf.mx_pad_M_groups(upload(torch, data), torch.tensor(raw, dtype=torch.int32).cuda())
        torch.cuda.synchronize()
        compare("clamped pad", out.cpu().numpy(), want)


def test_float8_input(env):
    gsf, oracle, torch = env
    rng = np.random.default_rng(82)
    data = rng.integers(0, 0x7E, size=(200, 96), dtype=np.uint8)   # finite E4M3 codes
    print("case pad float8 view", flush=True)
    x = torch.from_numpy(data).cuda().view(torch.float8_e4m3fn)
    out = gsf.mx_pad_M_groups(x, torch.tensor([77, 200], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    compare("float8 pad", out.cpu().numpy(), oracle.pad_M_groups(data, [77, 200]))


def test_bench_launch_configuration(env):
    import bench

    gsf, oracle, torch = env
    print("case bench config pad_m_groups_small", flush=True)
    job = bench.Job("pad_m_groups_small", rotate_bytes=0)
    job.step(0)
    job.step(1)
    torch.cuda.synchronize()
    want = oracle.pad_M_groups(job.w.data, job.w.offs)
    compare("bench pad", job.outs[0].cpu().numpy(), want.reshape(-1))
