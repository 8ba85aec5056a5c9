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
