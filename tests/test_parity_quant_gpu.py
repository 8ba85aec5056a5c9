"""Parity of the MXFP8 dim0 cast (codes and blocked scales) with the CPU oracle, byte for byte (GPU).

Every case prints its shape before touching the GPU. Both outputs are prefilled
with 0xAB and followed by guard bytes: every byte must be written, none past it.
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


def device_bf16(torch, x_bits, ld=None):
    """Upload (rows, K) bf16 bit patterns as a torch.bfloat16 view with row stride ld elements."""
    rows, K = x_bits.shape
    ld = K if ld is None else ld
    buf = np.zeros((max(rows, 1), ld), np.uint16)
    buf[:rows, :K] = x_bits
    t = torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)
    return t[:rows, :K]


def run_quant(env, x_bits, offs, ld=None, label="", want=None):
    """Runs the GPU cast; compares q and the blocked scales with the oracle (or with `want`)."""
    gsf, oracle, torch = env
    rows, K = x_bits.shape
    offs = np.asarray(offs, np.int32)
    print("case", label, "rows", rows, "K", K, "ld", ld or K, "G", len(offs), flush=True)
    if want is None:
        want = oracle.quantize_dim0_M_groups(x_bits, offs)
    want_q, want_s = want
    x = device_bf16(torch, x_bits, ld)
    n = want_s.size
    qbuf = torch.full((rows * K + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    q, s = gsf.mx_quantize_dim0_M_groups(x, torch.from_numpy(offs).cuda(), q=qbuf[: rows * K].view(rows, K),
                                         scales=sbuf[:n])
    torch.cuda.synchronize()
    gq, gs = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (gq[rows * K:] == POISON).all(), "%s: bytes past q were written" % label
    assert (gs[n:] == POISON).all(), "%s: bytes past the scales were written" % label
    _compare(label + " codes", gq[: rows * K], want_q.reshape(-1))
    _compare(label + " scales", gs[:n], want_s)


def _compare(label, got, want):
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError("%s: %d of %d bytes differ, first at %d (got %#x want %#x)"
                             % (label, bad.size, want.size, bad[0], got[bad[0]], want[bad[0]]))


def compare_slices(label, tasks):
    """Compares GPU codes with the oracle slice by slice, the oracle slices computed in parallel host
    threads (the C oracle runs without the GIL). tasks: (slice label, want() -> codes, got codes)."""
    from concurrent.futures import ThreadPoolExecutor

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    print("  %s: %d slices on %d host threads" % (label, len(tasks), threads), flush=True)
    with ThreadPoolExecutor(threads) as pool:
        futures = [(name, pool.submit(want), got) for name, want, got in tasks]
        for name, fut, got in futures:
            _compare("%s %s" % (label, name), np.ascontiguousarray(got).reshape(-1), fut.result().reshape(-1))


def test_workload_small_bit_exact(env):
    import workloads

    w = workloads.make("quant_m_groups_small")
    run_quant(env, w.x, w.offs, label=w.name)


@pytest.mark.parametrize("name", ["quant_m_groups", "quant_m_groups_skinny"])
def test_workload_full_size(env, name):
    """(16640, 5120) and (131072, 1408): every scale byte and every code against the oracle (the codes
    in slices of 1024 rows, computed in parallel)."""
    gsf, oracle, torch = env
    import workloads

    w = workloads.make(name)
    print("case %s full size" % name, flush=True)
    x = device_bf16(torch, w.x)
    q, s = gsf.mx_quantize_dim0_M_groups(x, torch.from_numpy(w.offs).cuda())
    torch.cuda.synchronize()
    want_s = oracle.rearrange("M", oracle.scales_dim0(w.x), w.offs)
    _compare("full-size scales", s.cpu().numpy(), want_s)
    got = q.cpu().numpy()
    step = 1024
    compare_slices("full-size codes", [
        ("rows %d..%d" % (r, min(r + step, w.rows)),
         (lambda r=r: oracle.quantize_dim0(np.ascontiguousarray(w.x[r:r + step]))[0]), got[r:r + step])
        for r in range(0, w.rows, step)])


def test_every_scale_and_code(env):
    """Every scale exponent s in [-127, 119], and for each one every E4M3-relevant y = x / 2^s
    (1 + m/128) * 2^e, |y| <= 256, e >= -12, both signs, whenever x is exact in bf16; plus
    blocks whose largest magnitude is each bf16 subnormal."""
    gsf, oracle, torch = env
    vals = []
    ys = np.array([(1 + m / 128.0) * 2.0 ** e for e in range(-12, 8) for m in range(128)] + [256.0])
    ys = np.concatenate([ys, -ys])
    for s in range(-127, 120):
        x = ys * 2.0 ** s
        x32 = x.astype(np.float32)
        ok = (x32.astype(np.float64) == x) & ((x32.view(np.uint32) & 0xFFFF) == 0) & (x32 != 0)
        xs = x32[ok]
        amax = np.float32(2.0 ** (s + 8))
        for i in range(0, xs.size, 31):
            blk = np.zeros(32, np.float32)
            blk[0] = amax if (i // 31) % 2 == 0 else -amax
            blk[1: 1 + min(31, xs.size - i)] = xs[i: i + 31]
            vals.append(blk)
    sub = np.arange(1, 128, dtype=np.uint32)           # bf16 subnormal magnitudes
    for m in sub:
        blk = (np.concatenate([[m], np.arange(32 - 1) % m]) << 16).astype(np.uint32).view(np.float32)
        vals.append(blk)
    blocks = np.stack(vals)
    bits = (blocks.view(np.uint32) >> 16).astype(np.uint16)
    nb = bits.shape[0]
    per_row = 16
    rows = (nb + per_row - 1) // per_row
    x = np.zeros((rows * per_row, 32), np.uint16)
    x[:nb] = bits
    x = x.reshape(rows, per_row * 32)
    run_quant(env, x, [rows], label="every scale and code")


def test_hand_worked_blocks(env):
    import pins

    blocks = pins.load_mxfp8_blocks()
    x = np.stack([b["x"] for b in blocks]).reshape(1, -1)
    x = np.repeat(x, 3, axis=0)
    q = np.stack([b["q"] for b in blocks]).reshape(1, -1).repeat(3, axis=0)
    s = np.array([b["scale"] for b in blocks], np.uint8)
    gsf, oracle, torch = env
    want = oracle.quantize_dim0_M_groups(x, [3])
    assert np.array_equal(want[0], q)   # the oracle agrees with the hand-worked values
    assert np.array_equal(oracle.scales_dim0(x)[0], s)
    run_quant(env, x, [3], label="hand-worked", want=want)


def test_fuzz(env):
    import pins
    import workloads

    rng = np.random.default_rng(51)
    for i in range(60):
        rows = int(rng.choice([0, 1, 2, 31, 127, 128, 129, 200, 255, 300, 513, 700]))
        K = 32 * int(rng.choice([1, 2, 3, 4, 5, 7, 15, 16, 17, 31, 33, 50]))
        ld = K + 8 * int(rng.choice([0, 0, 1, 4, 9]))
        G = int(rng.choice([1, 2, 3, 8, 16, 63, 64, 65, 80]))
        offs = workloads.random_offsets(rng, rows, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.2))
        x = pins.random_bf16_rows(rng, rows, K) if rows else np.zeros((0, K), np.uint16)
        if rows and rng.random() < 0.3:   # a few non-finite elements
            for _ in range(3):
                x[rng.integers(0, rows), rng.integers(0, K)] = rng.choice([0x7F80, 0xFF80, 0x7FC0])
        run_quant(env, x, offs, ld=ld, label="fuzz%d" % i)


def test_random_sweep(env):
    """Random dim0 and dim1 casts (a tenth of MX_SWEEP_CASES each, default 200): rows/tokens up to 700,
    K/N up to 1600 and 1300, padded strides, up to 200 groups, empty groups, short totals (dim1: ends at any
    token, not only multiples of 32), sprinkled non-finite values."""
    import pins
    import workloads

    rng = np.random.default_rng(2030)
    n = int(os.environ.get("MX_SWEEP_CASES", "2000")) // 10
    for i in range(n):
        rows = int(rng.choice([1, 2, 31, 127, 128, 129, 300, 700]))
        K = 32 * int(rng.integers(1, 51))
        G = int(rng.choice([1, 2, 3, 8, 16, 64, 65, 200]))
        offs = workloads.random_offsets(rng, rows, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.2))
        x = pins.random_bf16_rows(rng, rows, K)
        if rng.random() < 0.3:
            x[rng.integers(0, rows), rng.integers(0, K)] = rng.choice([0x7F80, 0xFF80, 0x7FC0])
        run_quant(env, x, offs, ld=K + 8 * int(rng.choice([0, 0, 1, 9])), label="sweep dim0 %d" % i)
    for i in range(n):
        T = 32 * int(rng.choice([1, 2, 3, 4, 5, 8, 13, 21]))
        N = int(rng.integers(1, 1300))
        G = int(rng.choice([1, 2, 3, 8, 16, 64, 65, 200]))
        offs = workloads.random_offsets(rng, T, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                        short_total=bool(rng.random() < 0.2))
        x = pins.random_bf16_rows(rng, T, N)
        if rng.random() < 0.3:
            x[rng.integers(0, T), rng.integers(0, N)] = rng.choice([0x7F80, 0xFF80, 0x7FC0])
        run_dim1(env, x, offs, ld=_ld8(N, int(rng.choice([0, 0, 1, 5]))), label="sweep dim1 %d" % i)


def test_many_groups(env):
    import pins
    import workloads

    rng = np.random.default_rng(52)
    for rows, K, G in [(5000, 64, 4096), (3000, 96, 1000), (64, 32, 4096)]:
        offs = workloads.random_offsets(rng, rows, G, p_empty=0.5)
        run_quant(env, pins.random_bf16_rows(rng, rows, K), offs, label="many groups")


def test_multi_pass_grid_many_groups(env):
    # 2500 quantising workgroups, more than the GPU holds at once (row blocks dealt to the XCDs in
    # turn), with the group table of 80 groups in LDS
    import pins
    import workloads

    rng = np.random.default_rng(61)
    rows, K = 40000, 512
    offs = workloads.random_offsets(rng, rows, 80, p_empty=0.25)
    run_quant(env, pins.random_bf16_rows(rng, rows, K), offs, label="multi-pass grid, 80 groups")


def test_multi_pass_fuzz(env):
    """Seeded random casts whose grids take more than one pass over the GPU (128-row blocks dealt to the
    XCDs in turn): ragged row counts, K not a multiple of 512 (a partial last unit of each row), row strides,
    group tables in registers and in LDS. Each case has more than 2048 quantising workgroups of 256 threads
    (16 units of 512 elements each), more than the GPU holds at once."""
    import pins
    import workloads

    rng = np.random.default_rng(65)
    for i, K in enumerate([96, 544, 1408, 2048]):
        chunks = (K + 511) // 512
        rows = int(rng.integers(40_000 // chunks + 2000, 40_000 // chunks + 12_000))
        assert rows * chunks // 16 > 2048
        ld = K + 8 * int(rng.choice([0, 0, 1, 5]))
        G = int(rng.choice([1, 8, 65, 200]))
        offs = workloads.random_offsets(rng, rows, G, p_empty=0.25, short_total=bool(rng.random() < 0.2))
        run_quant(env, pins.random_bf16_rows(rng, rows, K), offs, ld=ld, label="multi-pass fuzz %d" % i)


def test_invalid_offsets_are_clamped(env):
    import pins

    gsf, oracle, torch = env
    rng = np.random.default_rng(53)
    rows, K = 300, 96
    x = pins.random_bf16_rows(rng, rows, K)
    for raw in ([50, 20, 400], [-5, 10, 10**6], [300, 0, 0], [2**31 - 1] * 3, [-(2**31)] * 2):
        clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw, np.int64), 0)), rows).astype(np.int32)
        want = oracle.quantize_dim0_M_groups(x, clamped)
        print("case invalid offsets", raw, flush=True)
        n = want[1].size
        sbuf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        q, _ = gsf.mx_quantize_dim0_M_groups(device_bf16(torch, x), torch.tensor(raw, dtype=torch.int32).cuda(),
                                             scales=sbuf[:n])
        torch.cuda.synchronize()
        got = sbuf.cpu().numpy()
        assert (got[n:] == POISON).all()
        _compare("clamped scales", got[:n], want[1])
        _compare("clamped codes", q.cpu().numpy().reshape(-1), want[0].reshape(-1))


def test_empty_shapes(env):
    gsf, oracle, torch = env
    run_quant(env, np.zeros((0, 64), np.uint16), [0, 0], label="rows=0")
    print("case K=0", flush=True)
    q, s = gsf.mx_quantize_dim0_M_groups(torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda"),
                                         torch.tensor([5], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert q.numel() == 0 and s.numel() == 0


def test_codes_read_back_as_float8(env):
    """The codes are torch float8_e4m3fn values: dequantised, they lie within half an E4M3 step of x / 2^s."""
    gsf, oracle, torch = env
    import workloads

    w = workloads.make("quant_m_groups_small")
    print("case float8 view", flush=True)
    q, s = gsf.mx_quantize_dim0_M_groups(device_bf16(torch, w.x), torch.from_numpy(w.offs).cuda())
    torch.cuda.synchronize()
    deq = q.view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy()
    sc = oracle.scales_dim0(w.x).astype(np.int64) - 127
    y = np.clip((np.asarray(w.x, np.uint32) << 16).view(np.float32).astype(np.float64)
                / np.repeat(2.0 ** sc, 32, axis=1), -448, 448)
    ay = np.abs(y)
    step = 2.0 ** (np.maximum(np.floor(np.log2(np.where(ay > 0, ay, 1.0))), -6) - 3)
    assert np.all(np.abs(deq - y) <= step / 2)


def test_bench_launch_configuration(env):
    """The exact launches bench.py times give the oracle's bytes."""
    import bench

    gsf, oracle, torch = env
    print("case bench config quant_m_groups_small", flush=True)
    job = bench.Job("quant_m_groups_small", rotate_bytes=0)
    job.step(0)
    job.step(1)
    torch.cuda.synchronize()
    w = job.w
    want_q, want_s = oracle.quantize_dim0_M_groups(w.x, w.offs)
    out = job.outbuf.cpu().numpy()
    _compare("bench codes", out[: w.rows * w.K], want_q.reshape(-1))
    _compare("bench scales", out[job.q_pitch: job.q_pitch + want_s.size], want_s)


# --------------------------------------------------------------------------
# dim1 cast: blocks of 32 tokens, codes transposed, K-groups blocked scales
# --------------------------------------------------------------------------


def run_dim1(env, x_bits, offs, ld=None, label="", want=None):
    gsf, oracle, torch = env
    T, N = x_bits.shape
    offs = np.asarray(offs, np.int32)
    print("case dim1", label, "T", T, "N", N, "ld", ld or N, "G", len(offs), flush=True)
    if want is None:
        want = oracle.quantize_dim1_K_groups(x_bits, offs)
    want_q, want_s = want
    x = device_bf16(torch, x_bits, ld)
    n = want_s.size
    qbuf = torch.full((N * T + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    gsf.mx_quantize_dim1_K_groups(x, torch.from_numpy(offs).cuda(), qT=qbuf[: N * T].view(N, T), scales=sbuf[:n])
    torch.cuda.synchronize()
    gq, gs = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (gq[N * T:] == POISON).all(), "%s: bytes past qT were written" % label
    assert (gs[n:] == POISON).all(), "%s: bytes past the scales were written" % label
    _compare(label + " codes", gq[: N * T], want_q.reshape(-1))
    _compare(label + " scales", gs[:n], want_s)


def _ld8(N, extra=0):
    return (N + 7) // 8 * 8 + 8 * extra


def test_dim1_workload_small(env):
    import workloads

    w = workloads.make("quant_k_groups_small")
    run_dim1(env, w.x, w.offs, ld=_ld8(w.K), label=w.name)


def test_dim1_workload_full_size(env):
    """(131072, 7168): every scale byte and every code against the oracle (the codes in slices of 64
    feature columns, computed in parallel)."""
    gsf, oracle, torch = env
    import workloads

    w = workloads.make("quant_k_groups")
    print("case dim1 quant_k_groups full size", flush=True)
    x = device_bf16(torch, w.x)
    qT, s = gsf.mx_quantize_dim1_K_groups(x, torch.from_numpy(w.offs).cuda())
    torch.cuda.synchronize()
    del x
    want_s = oracle.rearrange("K", oracle.scales_dim1(w.x), w.offs // 32)
    _compare("dim1 full-size scales", s.cpu().numpy(), want_s)
    got = qT.cpu().numpy()
    del qT, s
    step = 64
    compare_slices("dim1 full-size codes", [
        ("features %d..%d" % (f, min(f + step, w.K)),
         (lambda f=f: oracle.quantize_dim1(np.ascontiguousarray(w.x[:, f:f + step]))[0]), got[f:f + step])
        for f in range(0, w.K, step)])


def test_dim1_hand_worked_blocks(env):
    import pins

    gsf, oracle, torch = env
    blocks = pins.load_mxfp8_blocks()
    col = np.concatenate([b["x"] for b in blocks])            # one feature: the blocks one after another in tokens
    x = np.stack([col, col[::-1].copy(), col], axis=1)          # (T, 3)
    T = x.shape[0]
    want = oracle.quantize_dim1_K_groups(x, [T])
    codes = np.concatenate([b["q"] for b in blocks])
    assert np.array_equal(want[0][0], codes) and np.array_equal(want[0][2], codes)
    run_dim1(env, x, [T], ld=8, label="hand-worked", want=want)


def test_dim1_every_scale_and_code(env):
    """The exhaustive value set of the dim0 sweep, one 32-token block per feature column."""
    vals = []
    ys = np.array([(1 + m / 128.0) * 2.0 ** e for e in range(-12, 8) for m in range(128)] + [256.0])
    ys = np.concatenate([ys, -ys])
    for s in range(-127, 120, 3):
        x = ys * 2.0 ** s
        x32 = x.astype(np.float32)
        ok = (x32.astype(np.float64) == x) & ((x32.view(np.uint32) & 0xFFFF) == 0) & (x32 != 0)
        xs = x32[ok]
        for i in range(0, xs.size, 31):
            blk = np.zeros(32, np.float32)
            blk[0] = np.float32(2.0 ** (s + 8))
            blk[1: 1 + min(31, xs.size - i)] = xs[i: i + 31]
            vals.append(blk)
    bits = (np.stack(vals).view(np.uint32) >> 16).astype(np.uint16)   # (blocks, 32)
    x = np.ascontiguousarray(bits.T)                                     # (32 tokens, features)
    run_dim1(env, x, [32], ld=_ld8(x.shape[1]), label="every scale and code")


def test_dim1_fuzz(env):
    import pins
    import workloads

    rng = np.random.default_rng(61)
    for i in range(50):
        T = 32 * int(rng.choice([0, 1, 2, 3, 4, 5, 7, 8, 13, 40]))
        N = int(rng.choice([1, 2, 7, 8, 127, 128, 129, 300, 513]))
        ld = _ld8(N, int(rng.choice([0, 0, 1, 5])))
        G = int(rng.choice([1, 2, 3, 8, 16, 63, 64, 65, 80]))
        offs = 32 * workloads.random_offsets(rng, T // 32, G, p_empty=float(rng.choice([0.0, 0.3, 0.7])),
                                             short_total=bool(rng.random() < 0.3))
        x = pins.random_bf16_rows(rng, max(T, 1), N)[:T] if T else np.zeros((0, N), np.uint16)
        if T and rng.random() < 0.3:
            for _ in range(3):
                x[rng.integers(0, T), rng.integers(0, N)] = rng.choice([0x7F80, 0xFF80, 0x7FC0])
        run_dim1(env, x, offs.astype(np.int32), ld=ld, label="fuzz%d" % i)


def test_dim1_offsets_not_multiples_of_32(env):
    import pins

    rng = np.random.default_rng(62)
    x = pins.random_bf16_rows(rng, 320, 70)
    for offs in ([33, 100, 320], [31, 31, 290], [1, 2, 3, 300]):
        run_dim1(env, x, offs, ld=72, label="offsets %s" % offs)


def test_dim1_many_groups(env):
    import pins
    import workloads

    rng = np.random.default_rng(63)
    for T, N, G in [(32 * 300, 40, 2048), (32 * 100, 130, 100)]:
        offs = 32 * workloads.random_offsets(rng, T // 32, G, p_empty=0.5)
        run_dim1(env, pins.random_bf16_rows(rng, T, N), offs.astype(np.int32), ld=_ld8(N), label="many groups")


def test_dim1_invalid_offsets_are_clamped(env):
    import pins

    gsf, oracle, torch = env
    rng = np.random.default_rng(64)
    T, N = 320, 96
    x = pins.random_bf16_rows(rng, T, N)
    for raw in ([64, 32, 400], [-32, 96, 10**6], [320, 0, 0], [2**31 - 1] * 3, [-(2**31)] * 2):
        clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw, np.int64), 0)), T).astype(np.int32)
        want = oracle.quantize_dim1_K_groups(x, clamped)
        print("case dim1 invalid offsets", raw, flush=True)
        n = want[1].size
        sbuf = torch.full((n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        qT, _ = gsf.mx_quantize_dim1_K_groups(device_bf16(torch, x), torch.tensor(raw, dtype=torch.int32).cuda(),
                                              scales=sbuf[:n])
        torch.cuda.synchronize()
        got = sbuf.cpu().numpy()
        assert (got[n:] == POISON).all()
        _compare("dim1 clamped scales", got[:n], want[1])
        _compare("dim1 clamped codes", qT.cpu().numpy().reshape(-1), want[0].reshape(-1))


def test_dim1_empty_shapes(env):
    gsf, oracle, torch = env
    run_dim1(env, np.zeros((0, 40), np.uint16), [0, 0], ld=40, label="T=0")
    print("case dim1 N=0", flush=True)
    qT, s = gsf.mx_quantize_dim1_K_groups(torch.zeros((64, 0), dtype=torch.bfloat16, device="cuda"),
                                          torch.tensor([64], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert qT.numel() == 0 and s.numel() == 0


def test_dim1_bench_launch_configuration(env):
    import bench

    gsf, oracle, torch = env
    print("case bench config quant_k_groups_small", flush=True)
    job = bench.Job("quant_k_groups_small", rotate_bytes=0)
    job.step(0)
    job.step(1)
    torch.cuda.synchronize()
    w = job.w
    want_q, want_s = oracle.quantize_dim1_K_groups(w.x, w.offs)
    out = job.outbuf.cpu().numpy()
    _compare("dim1 bench codes", out[: w.rows * w.K], want_q.reshape(-1))
    _compare("dim1 bench scales", out[job.q_pitch: job.q_pitch + want_s.size], want_s)


# --------------------------------------------------------------------------
# dim1 cast of stacked expert weights: per-expert codes and blocked scales
# --------------------------------------------------------------------------

def device_bf16_3d(torch, w_bits, es, ld):
    """An (E, K, N) bf16 device view with expert stride es and row stride ld (elements) of host bit patterns."""
    E, K, N = w_bits.shape
    n = (E - 1) * es + (K - 1) * ld + N if E * K * N > 0 else 0
    flat = np.zeros(n + 64, np.uint16)
    if E * K * N > 0:
        np.lib.stride_tricks.as_strided(flat, shape=(E, K, N), strides=(2 * es, 2 * ld, 2))[...] = w_bits
    buf = torch.from_numpy(flat.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.as_strided(buf, (E, K, N), (es, ld, 1))


def run_dim1_3d(env, w_bits, es=None, ld=None, label=""):
    gsf, oracle, torch = env
    E, K, N = w_bits.shape
    ld = _ld8(N) if ld is None else ld
    es = K * ld if es is None else es
    print("case dim1 3d", label, "E", E, "K", K, "N", N, "ld", ld, "expert stride", es, flush=True)
    want_q, want_s = oracle.quantize_dim1_3d(w_bits)
    w = device_bf16_3d(torch, w_bits, es, ld)
    nq, ns = E * N * K, want_s.size
    qbuf = torch.full((nq + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((ns + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    gsf.mx_quantize_dim1_3d(w, q=qbuf[:nq].view(E, N, K), scales=sbuf[:ns])
    torch.cuda.synchronize()
    gq, gs = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (gq[nq:] == POISON).all(), "%s: bytes past the codes were written" % label
    assert (gs[ns:] == POISON).all(), "%s: bytes past the scales were written" % label
    _compare(label + " codes", gq[:nq], want_q.reshape(-1))
    _compare(label + " scales", gs[:ns], want_s)


def test_dim1_3d_workload_small(env):
    import workloads

    w = workloads.make("quant_3d_small")
    es, ld = w.w.strides[0] // 2, w.w.strides[1] // 2
    run_dim1_3d(env, w.w, es=es, ld=ld, label=w.name)


def test_dim1_3d_fuzz(env):
    import pins

    rng = np.random.default_rng(95)
    for i in range(40):
        E = int(rng.choice([1, 2, 3, 5, 8]))
        K = int(rng.choice([32, 64, 96, 128, 160, 256, 320]))   # multiples of 128 take the diagonal unit order
        N = int(rng.choice([1, 5, 8, 40, 127, 128, 129, 300]))
        ld = _ld8(N, int(rng.integers(0, 3)))
        es = 0 if rng.random() < 0.1 else K * ld + 8 * int(rng.integers(0, 4))
        one = pins.random_bf16_rows(rng, K * (1 if es == 0 else E), N)
        w = np.broadcast_to(one, (E, K, N)) if es == 0 else one.reshape(E, K, N)
        run_dim1_3d(env, w, es=es, ld=ld, label="fuzz%d" % i)


def test_dim1_3d_many_experts(env):
    import pins

    rng = np.random.default_rng(96)
    w = pins.random_bf16_rows(rng, 70 * 32, 40).reshape(70, 32, 40)   # more than 64 groups: table in LDS
    run_dim1_3d(env, w, label="70 experts")
    w = pins.random_bf16_rows(rng, 66 * 128, 136).reshape(66, 128, 136)
    run_dim1_3d(env, w, label="66 experts of 128 tokens")


def test_dim1_3d_empty_shapes(env):
    gsf, oracle, torch = env
    for E, K, N in [(0, 64, 8), (3, 0, 8), (3, 64, 0)]:
        print("case dim1 3d empty", E, K, N, flush=True)
        w = torch.zeros((E, K, N), dtype=torch.bfloat16, device="cuda")
        q, s = gsf.mx_quantize_dim1_3d(w)
        torch.cuda.synchronize()
        assert q.shape == (E, N, K) and s.numel() == oracle.out_bytes_3d(E, N, K // 32)


def test_dim1_3d_full_size_and_bench_launch(env):
    """The launches bench.py times on the (16, 5120, 8192) weights: every scale byte and every code
    against the oracle (the codes in slices of one expert x 1024 features, computed in parallel)."""
    import bench

    gsf, oracle, torch = env
    print("case dim1 3d full size quant_3d_e16 (bench launch)", flush=True)
    job = bench.Job("quant_3d_e16", rotate_bytes=0)
    job.step(0)
    torch.cuda.synchronize()
    w = job.w
    E, K, N = w.experts, w.K, w.N
    out = job.outs[0].cpu().numpy()
    q = out[: E * N * K].reshape(E, N, K)
    scales = np.stack([oracle.scales_dim1(w.w[e]) for e in range(E)])        # (E, N, K/32)
    _compare("quant_3d_e16 scales", out[job.q_pitch: job.q_pitch + oracle.out_bytes_3d(E, N, K // 32)],
             oracle.rearrange_3d(scales))
    step = 1024
    compare_slices("quant_3d_e16 codes", [
        ("expert %d features %d..%d" % (e, f, min(f + step, N)),
         (lambda e=e, f=f: oracle.quantize_dim1(np.ascontiguousarray(w.w[e][:, f:f + step]))[0]), q[e, f:f + step])
        for e in range(E) for f in range(0, N, step)])


def test_dim0_cast_of_stacked_experts_gives_the_3d_layout(env):
    """Expert weights cast along their last dimension through the M-groups cast with equal group ends: the
    codes are the row-wise cast, the first E*ru(N,128)*ru(K/32,4) scale bytes the per-expert (3-D) layout of
    the oracle, and the rest of the allocation zero."""
    gsf, oracle, torch = env
    import pins

    rng = np.random.default_rng(97)
    for E, N, K in [(3, 200, 96), (4, 128, 64), (2, 129, 160)]:
        print("case dim0 stacked experts", E, N, K, flush=True)
        x = pins.random_bf16_rows(rng, E * N, K)
        offs = (np.arange(1, E + 1) * N).astype(np.int32)
        q, s = gsf.mx_quantize_dim0_M_groups(device_bf16(torch, x), torch.from_numpy(offs).cuda())
        torch.cuda.synchronize()
        want_q, scales = oracle.quantize_dim0(x)                      # (E*N, K/32) scales
        want_3d = oracle.rearrange_3d(scales.reshape(E, N, K // 32))
        got_s = s.cpu().numpy()
        _compare("stacked experts codes", q.cpu().numpy().reshape(-1), want_q.reshape(-1))
        _compare("stacked experts 3-D scales", got_s[:want_3d.size], want_3d)
        assert not got_s[want_3d.size:].any()
