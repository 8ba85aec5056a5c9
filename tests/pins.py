"""Checks that pin the CPU oracle to something other than itself.

Nothing here calls the oracle's formula again. The checks are:

* hand-worked byte positions (``golden/blocked_layout_positions.txt``);
* the inverse direction: every output byte is decoded back to the input element
  it must hold (or to padding) from the tile geometry alone, and compared with
  the source of that byte measured by running the oracle on index-coded inputs;
* a textbook reshape/transpose formulation of a single blocked matrix, which
  M groups with one group, and K groups with at most 128 rows, reduce to;
* the output size that reproduces the bandwidth figures printed on the pages
  (``golden/k_groups_bandwidth.txt``).

Each check takes an ``Oracle``-like object (``out_bytes``, ``rearrange``), so
the same checks also run against deliberately broken copies of the oracle.
"""

import os
import shutil
import tempfile

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def ru(x, m):
    return (x + m - 1) // m * m


# --------------------------------------------------------------------------
# measuring where each output byte comes from
# --------------------------------------------------------------------------

def source_map(orc, kind, rows, cols, ld, offs):
    """Linear input index (row*ld + col) held by each output byte, or -1 for padding.

    The rearrangement moves bytes without looking at them, so running it on
    three byte planes of the linear index plus an all-ones plane recovers the
    whole map.
    """
    offs = np.asarray(offs, dtype=np.int32)
    n = max(rows * ld, 1)
    assert n < (1 << 24)
    idx = np.arange(n, dtype=np.int64)
    planes = []
    for k in range(3):
        buf = ((idx >> (8 * k)) & 0xFF).astype(np.uint8)
        planes.append(_strided(buf, rows, cols, ld))
    ones = _strided(np.ones(n, np.uint8), rows, cols, ld)
    outs = [orc.rearrange(kind, p, offs).astype(np.int64) for p in planes]
    valid = orc.rearrange(kind, ones, offs)
    src = outs[0] | (outs[1] << 8) | (outs[2] << 16)
    src[valid == 0] = -1
    return src


def _strided(buf, rows, cols, ld):
    return np.lib.stride_tricks.as_strided(buf, shape=(rows, cols), strides=(ld, 1))


# --------------------------------------------------------------------------
# the inverse direction, from the tile geometry
# --------------------------------------------------------------------------

def _tile_coords(b):
    """Split byte offsets inside blocked storage into (tile, row in tile, col in tile)."""
    t, o = b // 512, b % 512
    i = o // 16          # 16 bytes per group of four row-words
    q = (o % 16) // 4    # which 32-row quarter of the tile
    c = o % 4
    return t, 32 * q + i, c


def decode_M(rows, cols, ld, offs, n_out):
    offs = np.asarray(offs, dtype=np.int64)
    Cp = ru(cols, 4)
    src = np.full(n_out, -1, dtype=np.int64)
    if Cp == 0:
        return src
    b = np.arange(n_out, dtype=np.int64)
    t, r, c = _tile_coords(b)
    out_row = (t // (Cp // 4)) * 128 + r
    col = (t % (Cp // 4)) * 4 + c
    start, first_out_row = 0, 0
    for end in offs:
        size = int(end) - start
        padded = ru(size, 128)
        local = out_row - first_out_row
        hit = (local >= 0) & (local < size) & (col < cols)
        src[hit] = (start + local[hit]) * ld + col[hit]
        first_out_row += padded
        start = int(end)
    return src


def decode_K(rows, cols, ld, offs, n_out):
    offs = np.asarray(offs, dtype=np.int64)
    Rp = ru(rows, 128)
    src = np.full(n_out, -1, dtype=np.int64)
    start, first_col = 0, 0
    for end in offs:
        width = int(end) - start
        W = ru(width, 4)
        lo, hi = Rp * first_col, Rp * (first_col + W)
        if W > 0:
            b = np.arange(lo, hi, dtype=np.int64)
            t, r, c = _tile_coords(b - lo)
            row = (t // (W // 4)) * 128 + r
            col = (t % (W // 4)) * 4 + c
            hit = (row < rows) & (col < width)
            src[b[hit]] = row[hit] * ld + start + col[hit]
        first_col += W
        start = int(end)
    return src


def decode(kind, rows, cols, ld, offs, n_out):
    return (decode_M if kind == "M" else decode_K)(rows, cols, ld, offs, n_out)


# --------------------------------------------------------------------------
# one blocked matrix, written as array reshapes
# --------------------------------------------------------------------------

def to_blocked_reshape(A):
    """Blocked layout of an (R, C) uint8 matrix, R % 128 == 0, C % 4 == 0.

    View each 128x4 tile's rows as (4 quarters, 32 rows) and store the tile as
    [row in quarter][quarter][column]; tiles go row-major.
    """
    R, C = A.shape
    x = A.reshape(R // 128, 128, C // 4, 4).transpose(0, 2, 1, 3)      # (rb, cb, 128, 4)
    x = x.reshape(R // 128, C // 4, 4, 32, 4).transpose(0, 1, 3, 2, 4)  # (rb, cb, 32, 4, 4)
    return np.ascontiguousarray(x).reshape(-1)


def pad_to(A, R, C):
    P = np.zeros((R, C), dtype=np.uint8)
    P[: A.shape[0], : A.shape[1]] = A
    return P


# --------------------------------------------------------------------------
# golden files
# --------------------------------------------------------------------------

def load_positions():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "blocked_layout_positions.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                kv = dict(t.split("=") for t in tok[3:])
                cur = {"name": tok[1], "kind": tok[2], "rows": int(kv["rows"]), "cols": int(kv["cols"]),
                       "offs": [int(v) for v in kv["offs"].split(",")], "out_bytes": int(kv["out_bytes"]),
                       "at": [], "copied": None}
                cases.append(cur)
            elif tok[0] == "at":
                cur["at"].append(tuple(int(v) for v in tok[1:4]))
            elif tok[0] == "copied":
                cur["copied"] = int(tok[1])
    return cases


def load_bandwidth_rows():
    rows = []
    with open(os.path.join(GOLDEN, "k_groups_bandwidth.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            src, r, c, g, us, gb = [t.strip() for t in line.split("|")]
            rows.append((src, int(r), int(c), int(g), float(us), gb))
    return rows


def printed_precision(s):
    return 10.0 ** -(len(s.split(".")[1])) if "." in s else 1.0


def bandwidth_matches(rows, cols, G, us, gb_str, written):
    """Does (rows*cols + written) / t reproduce the printed GB/s, given both roundings?"""
    gb = float(gb_str)
    got = (rows * cols + written) / (us * 1e3)
    tol = 0.5 * printed_precision(gb_str) + got * (0.005 / us) + 1e-9
    return abs(got - gb) <= tol


# --------------------------------------------------------------------------
# the pin checks (each returns a list of failure strings)
# --------------------------------------------------------------------------

def check_positions(orc):
    fails = []
    for case in load_positions():
        kind, rows, cols, offs = case["kind"], case["rows"], case["cols"], case["offs"]
        n = orc.out_bytes(kind, rows, cols, len(offs))
        if n != case["out_bytes"]:
            fails.append("%s: out_bytes %d != %d" % (case["name"], n, case["out_bytes"]))
            continue
        src = source_map(orc, kind, rows, cols, cols, offs)
        for r, c, b in case["at"]:
            if src[b] != r * cols + c:
                fails.append("%s: (%d,%d) expected at byte %d, byte holds %d" % (case["name"], r, c, b, src[b]))
        if int((src >= 0).sum()) != case["copied"]:
            fails.append("%s: %d bytes copied, expected %d" % (case["name"], int((src >= 0).sum()), case["copied"]))
    return fails


def check_inverse(orc, kind, rows, cols, ld, offs):
    n = orc.out_bytes(kind, rows, cols, len(offs))
    src = source_map(orc, kind, rows, cols, ld, offs)
    want = decode(kind, rows, cols, ld, offs, n)
    if src.shape != want.shape or not np.array_equal(src, want):
        bad = np.nonzero(src != want)[0] if src.shape == want.shape else [-1]
        return ["%s rows=%d cols=%d ld=%d offs=%s: %d bytes differ from the decoded map (first %d)"
                % (kind, rows, cols, ld, list(offs), len(bad), bad[0])]
    # each input element appears at most once
    s = src[src >= 0]
    if np.unique(s).size != s.size:
        return ["%s rows=%d cols=%d offs=%s: an input byte appears twice" % (kind, rows, cols, list(offs))]
    return []


def check_single_matrix(orc, rng):
    """M with one group and K with <= 128 rows reduce to one blocked matrix."""
    fails = []
    for rows, cols in [(1, 1), (128, 4), (200, 7), (300, 12), (513, 3)]:
        A = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        out = orc.rearrange("M", A, [rows])
        Rp, Cp = ru(rows, 128), ru(cols, 4)
        want = np.zeros(orc.out_bytes("M", rows, cols, 1), np.uint8)
        want[: Rp * Cp] = to_blocked_reshape(pad_to(A, Rp, Cp))
        if not np.array_equal(out, want):
            fails.append("M single group %dx%d differs from the reshape layout" % (rows, cols))
    for rows, cols, offs in [(128, 8, [8]), (77, 10, [3, 3, 10]), (5, 13, [1, 6, 13]), (128, 9, [0, 9])]:
        A = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        out = orc.rearrange("K", A, offs)
        pieces, start = [], 0
        for end in offs:
            pieces.append(pad_to(A[:, start:end], 128, ru(end - start, 4)))
            start = end
        cat = np.concatenate(pieces, axis=1)
        want = np.zeros(orc.out_bytes("K", rows, cols, len(offs)), np.uint8)
        if cat.shape[1]:
            want[: cat.size] = to_blocked_reshape(cat)
        if not np.array_equal(out, want):
            fails.append("K rows=%d cols=%d offs=%s differs from the reshape layout" % (rows, cols, offs))
    return fails


def check_bandwidth_tables(orc):
    fails = []
    for src, rows, cols, G, us, gb in load_bandwidth_rows():
        written = orc.out_bytes("K", rows, cols, G)
        if not bandwidth_matches(rows, cols, G, us, gb, written):
            fails.append("%s (%d,%d) G=%d: %.3f GB/s vs printed %s"
                         % (src, rows, cols, G, (rows * cols + written) / (us * 1e3), gb))
    return fails


def random_case(rng, kind, max_rows=700, max_cols=40, max_groups=6):
    from workloads import random_offsets
    rows = int(rng.integers(0, max_rows + 1))
    cols = int(rng.integers(0, max_cols + 1))
    ld = cols + int(rng.choice([0, 0, 1, 3, 13]))
    G = int(rng.integers(1, max_groups + 1))
    total = rows if kind == "M" else cols
    offs = random_offsets(rng, total, G, p_empty=0.3, short_total=rng.random() < 0.3)
    return rows, cols, ld, offs


# --------------------------------------------------------------------------
# per-expert (3-D) weight scales: one blocked matrix per expert
# --------------------------------------------------------------------------

def strided_3d(buf, experts, rows, cols, es, ld):
    return np.lib.stride_tricks.as_strided(buf, shape=(experts, rows, cols), strides=(es, ld, 1))


def source_map_3d(orc, experts, rows, cols, es, ld):
    """Linear input index (e*es + row*ld + col) held by each output byte, or -1."""
    n = max(experts * es + rows * ld, 1)
    assert n < (1 << 24)
    idx = np.arange(n, dtype=np.int64)
    outs = []
    for k in range(3):
        buf = ((idx >> (8 * k)) & 0xFF).astype(np.uint8)
        outs.append(orc.rearrange_3d(strided_3d(buf, experts, rows, cols, es, ld)).astype(np.int64))
    valid = orc.rearrange_3d(strided_3d(np.ones(n, np.uint8), experts, rows, cols, es, ld))
    src = outs[0] | (outs[1] << 8) | (outs[2] << 16)
    src[valid == 0] = -1
    return src


def decode_3d(experts, rows, cols, es, ld):
    """Inverse map from the tile geometry: expert e owns bytes [e*Rp*Cp, (e+1)*Rp*Cp)."""
    Rp, Cp = ru(rows, 128), ru(cols, 4)
    n = experts * Rp * Cp
    src = np.full(n, -1, dtype=np.int64)
    if n == 0:
        return src
    b = np.arange(n, dtype=np.int64)
    e, local = b // (Rp * Cp), b % (Rp * Cp)
    t, r, c = _tile_coords(local)
    row = (t // (Cp // 4)) * 128 + r
    col = (t % (Cp // 4)) * 4 + c
    hit = (row < rows) & (col < cols)
    src[hit] = e[hit] * es + row[hit] * ld + col[hit]
    return src


def check_inverse_3d(orc, experts, rows, cols, es, ld):
    n = orc.out_bytes_3d(experts, rows, cols)
    src = source_map_3d(orc, experts, rows, cols, es, ld)
    want = decode_3d(experts, rows, cols, es, ld)
    if n != want.size or src.shape != want.shape or not np.array_equal(src, want):
        return ["3d E=%d rows=%d cols=%d es=%d ld=%d: output differs from the decoded map"
                % (experts, rows, cols, es, ld)]
    return []


def check_3d_reshape(orc, rng):
    """Each expert's slice is the reshape layout of that expert's padded matrix."""
    fails = []
    for E, rows, cols in [(1, 1, 1), (1, 128, 4), (3, 200, 7), (2, 256, 12), (4, 77, 13), (5, 128, 160)]:
        A = rng.integers(1, 256, size=(E, rows, cols), dtype=np.uint8)
        out = orc.rearrange_3d(A)
        Rp, Cp = ru(rows, 128), ru(cols, 4)
        want = np.concatenate([to_blocked_reshape(pad_to(A[e], Rp, Cp)) for e in range(E)])
        if not np.array_equal(out, want):
            fails.append("3d E=%d %dx%d differs from the per-expert reshape layout" % (E, rows, cols))
    return fails


def random_case_3d(rng, max_experts=5, max_rows=300, max_cols=40):
    E = int(rng.integers(0, max_experts + 1))
    rows = int(rng.integers(0, max_rows + 1))
    cols = int(rng.integers(0, max_cols + 1))
    ld = cols + int(rng.choice([0, 0, 1, 3, 13]))
    es = rows * ld + int(rng.choice([0, 0, 5, 64]))
    return E, rows, cols, es, ld


# --------------------------------------------------------------------------
# deliberately broken copies of the oracle
# --------------------------------------------------------------------------

def check_dim1_3d(orc, rng):
    """The dim1 cast of stacked expert weights (E, K, N) equals the dim1 cast of the experts stacked
    into one (E*K, N) token matrix with E equal token groups: the codes of expert e are the token
    columns [eK, (e+1)K) of that cast's transposed codes, and the per-expert blocked scales are the
    first bytes of its K-groups blocked scales (each group one blocked matrix at ru(N,128)*C_g, C_g =
    e*ru(K/32,4)), the rest of which is zero. Any expert and row strides."""
    fails = []
    for E, K, N, ld_pad, es_pad in [(1, 32, 5, 0, 0), (3, 64, 40, 3, 17), (4, 96, 130, 0, 0), (2, 160, 7, 1, 5),
                                    (5, 32, 129, 2, 0), (0, 64, 8, 0, 0), (3, 0, 8, 0, 0)]:
        ld = N + ld_pad
        es = K * ld + es_pad
        base = random_bf16_rows(rng, max(E * es // max(ld, 1) + 2, 1), ld).reshape(-1)
        x3 = np.lib.stride_tricks.as_strided(base, shape=(E, K, N), strides=(2 * es, 2 * ld, 2))
        q, blocked = orc.quantize_dim1_3d(x3)
        if q.shape != (E, N, K) or blocked.size != orc.out_bytes_3d(E, N, K // 32):
            fails.append("E=%d K=%d N=%d: shapes %s %d" % (E, K, N, q.shape, blocked.size))
            continue
        if E == 0 or K == 0 or N == 0:
            continue
        packed = np.ascontiguousarray(x3).reshape(E * K, N)
        offs = np.arange(1, E + 1, dtype=np.int32) * K
        qT2, blocked2 = orc.quantize_dim1_K_groups(packed, offs)
        for e in range(E):
            if not np.array_equal(q[e], qT2[:, e * K:(e + 1) * K]):
                fails.append("E=%d K=%d N=%d: codes of expert %d" % (E, K, N, e))
        if not np.array_equal(blocked2[:blocked.size], blocked) or blocked2[blocked.size:].any():
            fails.append("E=%d K=%d N=%d: blocked scales" % (E, K, N))
    # expert stride 0: every expert is the same matrix
    x = random_bf16_rows(rng, 64, 24)
    x3 = np.lib.stride_tricks.as_strided(x.reshape(-1), shape=(3, 64, 24), strides=(0, 48, 2))
    q, blocked = orc.quantize_dim1_3d(x3)
    one = blocked.size // 3
    if not (np.array_equal(q[0], q[1]) and np.array_equal(q[0], q[2]) and
            np.array_equal(blocked[:one], blocked[one:2 * one]) and np.array_equal(blocked[:one], blocked[2 * one:])):
        fails.append("expert stride 0: experts differ")
    return fails


def with_mutant(old, new, fn):
    """Build a copy of the oracle source with `old` replaced by `new`, call fn(oracle), clean up."""
    import oracle

    src = open(oracle.SOURCE).read()
    assert old in src, old
    tmp = tempfile.mkdtemp()
    try:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(tmp, "libmutant.so")
        oracle.compile_library(path, lib)
        return fn(oracle.Oracle(lib))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


# --------------------------------------------------------------------------
# MXFP8 dim0 cast
# --------------------------------------------------------------------------

def load_mxfp8_blocks():
    """Hand-worked blocks: list of (name, x bits uint16[32], scale byte, codes uint8[32])."""
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, "mxfp8_dim0_blocks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "block":
                cur = {"name": tok[1], "x": np.zeros(32, np.uint16), "q": np.zeros(32, np.uint8), "scale": None}
                blocks.append(cur)
            elif tok[0] == "scale":
                cur["scale"] = int(tok[1], 16)
            elif tok[0] == "x":
                i = int(tok[1])
                cur["x"][i] = int(tok[2], 16)
                cur["q"][i] = int(tok[3], 16)
    for b in blocks:
        if b["scale"] == 0xFF:   # a non-finite block: every code is NaN, listed or not
            b["q"][:] = 0x7F
    return blocks


def bf16_bits(values):
    """bf16 bit patterns of float values that are exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert not (bits & 0xFFFF).any(), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_e4m3_values():
    """Value of every E4M3 code according to torch's float8_e4m3fn (a library routine)."""
    import torch

    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(values_f32):
    import torch

    return torch.from_numpy(np.asarray(values_f32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_e4m3_table(orc):
    want = torch_e4m3_values()
    fails = []
    for c in range(256):
        got = orc.lib.oracle_e4m3_value(c)
        if np.isnan(want[c]):
            if c & 0x7F != 0x7F:
                fails.append("torch says code %#x is NaN" % c)
            continue
        if got != want[c] or np.signbit(got) != np.signbit(want[c]):
            fails.append("code %#x: oracle %r, torch %r" % (c, got, want[c]))
    return fails


def e4m3_test_values(rng):
    """binary32 values in [-448, 448]: every code's value, every midpoint, one binary32 step either side
    of each midpoint, and log-uniform random values."""
    vals = torch_e4m3_values()
    pos = np.unique(vals[(vals >= 0) & np.isfinite(vals)])
    mids = (pos[1:] + pos[:-1]) / 2
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(np.inf))
    down = np.nextafter(mids32, np.float32(-np.inf))
    rnd = (rng.choice([-1.0, 1.0], 4000) * 2.0 ** rng.uniform(-12, np.log2(448), 4000)).astype(np.float32)
    v = np.concatenate([pos, mids32, up, down, rnd]).astype(np.float32)
    v = np.concatenate([v, -v, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -11, 2.0 ** -30])])
    return v[np.abs(v) <= 448]


def check_e4m3_encode(orc, rng):
    v = e4m3_test_values(rng)
    want = torch_e4m3_encode(v)
    got = np.array([orc.lib.oracle_e4m3_encode(float(x)) for x in v], np.uint8)
    bad = np.nonzero(got != want)[0]
    return ["encode(%r): oracle %#x, torch %#x" % (float(v[i]), got[i], want[i]) for i in bad[:5]]


def check_scale_closed_form(orc):
    """amax = m * 2^k with 1 <= m < 2 gives byte clamp(k - 8, -127, 127) + 127; amax 0 gives 0."""
    fails = []
    for k in range(-149, 128):
        for m in (1.0, 1.5, 1.9921875):
            amax = m * 2.0 ** k
            want = min(max(k - 8, -127), 127) + 127
            if orc.lib.oracle_e8m0_of_amax(amax) != want:
                fails.append("amax %r: byte %d, want %d" % (amax, orc.lib.oracle_e8m0_of_amax(amax), want))
    if orc.lib.oracle_e8m0_of_amax(0.0) != 0:
        fails.append("amax 0 must give byte 0")
    return fails


def check_golden_blocks(orc):
    fails = []
    blocks = load_mxfp8_blocks()
    x = np.stack([b["x"] for b in blocks])
    q, s = orc.quantize_dim0(x.reshape(1, -1))
    for i, b in enumerate(blocks):
        if s[0, i] != b["scale"]:
            fails.append("%s: scale %#x, want %#x" % (b["name"], s[0, i], b["scale"]))
        got = q[0, 32 * i: 32 * i + 32]
        for j in np.nonzero(got != b["q"])[0]:
            fails.append("%s[%d]: code %#x, want %#x" % (b["name"], j, got[j], b["q"][j]))
    return fails


def random_bf16_rows(rng, rows, K, ld=None, zero_block_p=0.05):
    """bf16 bit patterns: normal values times 2^U{-40..40} per block, some zero blocks, some -0."""
    ld = K if ld is None else ld
    v = rng.standard_normal((rows, ld)).astype(np.float32)
    v *= (2.0 ** rng.integers(-40, 41, size=(rows, ld // 32 + 1))).repeat(32, axis=1)[:, :ld].astype(np.float32)
    zb = rng.random((rows, ld // 32 + 1)) < zero_block_p
    v[zb.repeat(32, axis=1)[:, :ld]] = 0.0
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)   # truncation to bf16
    bits[rng.random((rows, ld)) < 0.01] = 0x8000
    return bits[:, :K]


def check_round_trip(orc, rng, rows=64, K=256):
    """Properties of any correct result: the scale puts the block's largest |y| in [256, 512) (unless
    clamped), every code is within half an E4M3 step of y = x / 2^s (saturated at 448), signs agree."""
    fails = []
    x = random_bf16_rows(rng, rows, K)
    q, s = orc.quantize_dim0(x)
    xv = bf16_to_f64(x).reshape(rows, K // 32, 32)
    qv = torch_e4m3_values()[q].reshape(rows, K // 32, 32)
    sexp = s.astype(np.int64) - 127
    y = xv / (2.0 ** sexp)[:, :, None]
    ymax = np.abs(y).max(axis=2)
    nz = ymax > 0
    clamped_low = sexp == -127
    if not np.all(((ymax >= 256) & (ymax < 512)) | ~nz | (clamped_low & (ymax < 256))):
        fails.append("a block's scale does not put its largest |y| in [256, 512)")
    if np.any(s[~nz] != 0):
        fails.append("zero block with non-zero scale")
    yc = np.clip(y, -448, 448)
    ay = np.abs(yc)
    step = 2.0 ** (np.maximum(np.floor(np.log2(np.where(ay > 0, ay, 1.0))), -6) - 3)
    err = np.abs(qv - yc)
    if np.any(err > step / 2 + 0.0):
        i = np.argmax(err - step / 2)
        fails.append("a code is more than half a step from y (%r vs %r)" % (qv.flat[i], yc.flat[i]))
    sign_bad = (np.signbit(qv) != np.signbit(y))
    if np.any(sign_bad):
        fails.append("%d codes with the wrong sign" % int(sign_bad.sum()))
    return fails


def check_nonfinite(orc):
    x = np.zeros((1, 96), np.uint16)
    x[0, :] = bf16_bits([1.0])[0]
    x[0, 5] = 0x7F80        # +inf in block 0
    x[0, 40] = 0x7FC1       # NaN in block 1
    q, s = orc.quantize_dim0(x)
    fails = []
    if list(s[0]) != [0xFF, 0xFF, 119]:   # block 2: amax 1.0, s = -8
        fails.append("scales of non-finite blocks: %s" % list(s[0]))
    if not (q[0, :64] == 0x7F).all():
        fails.append("codes of non-finite blocks are not all NaN")
    if not (q[0, 64:] == 0x78).all():     # 1.0 / 2^-8 = 256 = 2^8: exponent field 15, mantissa 0
        fails.append("a finite block next to non-finite ones is wrong")
    return fails


def check_blocked_scales(orc, rng):
    """The blocked scales equal the M-groups layout of the row-major scales, decoded from the tile geometry."""
    fails = []
    for rows, K, offs in [(200, 96, [200]), (300, 128, [0, 77, 77, 300]), (5, 32, [2, 5]), (129, 160, [129]),
                          (260, 64, [1, 130, 259])]:
        x = random_bf16_rows(rng, rows, K)
        q, s = orc.quantize_dim0(x)
        q2, blocked = orc.quantize_dim0_M_groups(x, offs)
        if not np.array_equal(q, q2):
            fails.append("codes differ between the two entry points")
        src = decode_M(rows, K // 32, K // 32, offs, blocked.size)
        want = np.where(src >= 0, s.reshape(-1)[np.maximum(src, 0)], 0).astype(np.uint8)
        if not np.array_equal(blocked, want):
            fails.append("blocked scales rows=%d K=%d offs=%s differ from the decoded layout" % (rows, K, offs))
    return fails


def check_dim1_transpose(orc, rng):
    """The dim1 cast of x is the dim0 cast of x transposed (tokens become the blocked dimension)."""
    fails = []
    for T, N, pad in [(32, 1, 0), (96, 50, 0), (64, 129, 7), (160, 33, 3), (0, 5, 0)]:
        base = random_bf16_rows(rng, max(T, 1), N + pad)[:T]
        x = base[:, :N]
        qT, s = orc.quantize_dim1(x)
        q0, s0 = orc.quantize_dim0(np.ascontiguousarray(x.T))
        if not (np.array_equal(qT, q0) and np.array_equal(s, s0)):
            fails.append("dim1 of (%d, %d) differs from dim0 of the transpose" % (T, N))
    return fails


def check_dim1_blocked(orc, rng):
    """dim1 blocked scales: the K-groups layout of the scales, group g = columns [offs[g-1]/32, offs[g]/32)."""
    fails = []
    for T, N, offs in [(256, 40, [64, 64, 256]), (320, 130, [32, 288]), (96, 5, [96]), (128, 300, [0, 40, 100, 128]),
                       (192, 7, [64, 190])]:
        x = random_bf16_rows(rng, T, N)
        try:
            qT, blocked = orc.quantize_dim1_K_groups(x, offs)
        except ValueError as e:
            fails.append(repr(e))
            continue
        _, s = orc.quantize_dim1(x)
        scale_offs = [o // 32 for o in offs]
        src = decode_K(N, T // 32, T // 32, scale_offs, blocked.size)
        want = np.where(src >= 0, s.reshape(-1)[np.maximum(src, 0)], 0).astype(np.uint8)
        if blocked.size != orc.out_bytes("K", N, T // 32, len(offs)) or not np.array_equal(blocked, want):
            fails.append("dim1 blocked scales T=%d N=%d offs=%s differ from the decoded layout" % (T, N, offs))
    return fails


# --------------------------------------------------------------------------
# per-group row padding of data
# --------------------------------------------------------------------------

def m_layout_row_sources(orc, rows, offs):
    """For each output row of the M-groups layout, the input row it holds (or -1), measured by running
    the M-groups scale oracle on a one-column index-coded matrix and reading rows off the tile geometry."""
    n = orc.out_bytes("M", rows, 1, len(offs))
    src = source_map(orc, "M", rows, 1, 1, offs)          # linear index = row (ld = 1)
    b = np.arange(n, dtype=np.int64)
    t, r, c = _tile_coords(b)
    out_row = t * 128 + r                                  # one tile column: tile index = row block
    sources = np.full(n // 4, -1, dtype=np.int64)
    hit = (c == 0) & (src >= 0)
    sources[out_row[hit]] = src[hit]
    return sources


def check_pad_placement(orc, rng):
    fails = []
    for rows, cols, offs in [(6, 3, [2, 2, 6]), (300, 5, [0, 129, 129, 250]), (129, 16, [129]), (0, 4, [0, 0]),
                             (257, 7, [1, 2, 3, 257])]:
        data = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        padded = orc.pad_M_groups(data, offs)
        sources = m_layout_row_sources(orc, rows, offs)
        want = np.zeros_like(padded)
        for R, s in enumerate(sources):
            if s >= 0:
                want[R] = data[s]
        if padded.shape[0] != rows + 128 * len(offs) or not np.array_equal(padded, want):
            fails.append("pad rows=%d cols=%d offs=%s: rows not where the M-groups layout puts them" % (rows, cols, offs))
    return fails


def check_unpad_round_trip(orc, rng):
    from workloads import random_offsets

    fails = []
    for _ in range(30):
        rows = int(rng.integers(0, 400))
        cols = int(rng.integers(1, 40))
        G = int(rng.integers(1, 8))
        offs = random_offsets(rng, rows, G, p_empty=0.3, short_total=bool(rng.random() < 0.3))
        data = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        back = orc.unpad_M_groups(orc.pad_M_groups(data, offs), rows, offs)
        end = int(offs[-1]) if len(offs) else 0
        if not (np.array_equal(back[:end], data[:end]) and not back[end:].any()):
            fails.append("unpad(pad(x)) != x for rows=%d offs=%s" % (rows, list(offs)))
    return fails


# --------------------------------------------------------------------------
# the inverse rearrangement
# --------------------------------------------------------------------------

def check_unrearrange(orc, kind, rows, cols, ld, offs, rng):
    """The inverse reads each byte from where the decoded map says the forward put it, zero elsewhere,
    and undoes the forward oracle."""
    offs = np.asarray(offs, np.int32)
    n = orc.out_bytes(kind, rows, cols, len(offs))
    blocked = rng.integers(0, 256, size=max(n, 1), dtype=np.uint8)[:n]
    got = orc.unrearrange(kind, blocked, rows, cols, offs)
    src = decode(kind, rows, cols, cols, offs, n)            # output byte -> input index (row*cols + col)
    want = np.zeros(rows * cols, np.uint8)
    hit = src >= 0
    want[src[hit]] = blocked[hit]
    fails = []
    if not np.array_equal(got.reshape(-1), want):
        fails.append("%s rows=%d cols=%d offs=%s: inverse differs from the decoded map" % (kind, rows, cols, list(offs)))
    A = random_scales(rng, rows, cols, ld)
    back = orc.unrearrange(kind, orc.rearrange(kind, A, offs), rows, cols, offs)
    end = int(offs[-1]) if len(offs) else 0
    keep = A[:end] if kind == "M" else A[:, :end]
    got_keep = back[:end] if kind == "M" else back[:, :end]
    rest = back[end:] if kind == "M" else back[:, end:]
    if not (np.array_equal(got_keep, keep) and not rest.any()):
        fails.append("%s rows=%d cols=%d offs=%s: inverse(forward(x)) != x" % (kind, rows, cols, list(offs)))
    return fails


def random_scales(rng, rows, cols, ld):
    from workloads import random_scales as rs

    return rs(rng, rows, cols, ld, lo=0, hi=255)
