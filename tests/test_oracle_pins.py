"""Pins of the CPU oracle (no GPU).

The oracle is checked against hand-worked positions, the inverse map derived
from the tile geometry, brute force over every offset vector of tiny shapes, a
reshape formulation of a single blocked matrix, the pages' printed bandwidth
figures (which fix the K-groups output size), and whole-workload invariants.
Deliberately broken copies of the oracle must fail these same pins.
"""

import itertools

import numpy as np
import pytest

import oracle
import pins
import workloads


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


def test_hand_worked_positions(orc):
    assert pins.check_positions(orc) == []


def test_hand_worked_zero_counts(orc):
    # with every input byte non-zero, the zeros are exactly the padding
    for case in pins.load_positions():
        rows, cols = case["rows"], case["cols"]
        A = np.full((rows, cols), 200, dtype=np.uint8)
        out = orc.rearrange(case["kind"], A, case["offs"])
        assert int((out == 0).sum()) == case["out_bytes"] - case["copied"], case["name"]
        assert int((out == 200).sum()) == case["copied"], case["name"]


def test_pad_in_tile_bytes_exact(orc):
    A = np.array([[11, 12, 13], [21, 22, 23]], dtype=np.uint8)
    out = orc.rearrange("M", A, [2])
    want = np.zeros(520, np.uint8)
    want[0:3] = [11, 12, 13]
    want[16:19] = [21, 22, 23]
    assert np.array_equal(out, want)


@pytest.mark.parametrize("kind", ["M", "K"])
def test_inverse_map_random(orc, kind):
    rng = np.random.default_rng(100 if kind == "M" else 200)
    fails = []
    for _ in range(60):
        rows, cols, ld, offs = pins.random_case(rng, kind)
        fails += pins.check_inverse(orc, kind, rows, cols, ld, offs)
    assert fails == []


def _nondecreasing(total, G):
    return [list(c) for c in itertools.combinations_with_replacement(range(total + 1), G)]


def test_brute_force_M_tiny(orc):
    fails = []
    for rows in range(0, 7):
        for cols in (1, 3, 4, 5):
            for G in (1, 2, 3):
                for offs in _nondecreasing(rows, G):
                    fails += pins.check_inverse(orc, "M", rows, cols, cols + (rows % 2), offs)
    assert fails == []


def test_brute_force_M_crossing_blocks(orc):
    # group boundaries on and around multiples of 128
    fails = []
    cuts = [0, 1, 127, 128, 129, 255, 256, 300]
    for a, b in itertools.combinations_with_replacement(cuts, 2):
        fails += pins.check_inverse(orc, "M", 300, 5, 7, [a, b, 300])
    assert fails == []


def test_brute_force_K_tiny(orc):
    fails = []
    for cols in range(0, 10):
        for rows in (1, 5, 129):
            for G in (1, 2, 3):
                for offs in _nondecreasing(cols, G):
                    fails += pins.check_inverse(orc, "K", rows, cols, cols + 2, offs)
    assert fails == []


def test_single_matrix_reductions(orc):
    assert pins.check_single_matrix(orc, np.random.default_rng(7)) == []


def test_M_and_K_single_group_agree(orc):
    rng = np.random.default_rng(8)
    for rows, cols in [(1, 1), (130, 6), (256, 8), (77, 13)]:
        A = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        m = orc.rearrange("M", A, [rows])
        k = orc.rearrange("K", A, [cols])
        used = pins.ru(rows, 128) * pins.ru(cols, 4)
        assert np.array_equal(m[:used], k[:used])
        assert not m[used:].any() and not k[used:].any()


def test_K_output_size_reproduces_printed_bandwidth(orc):
    assert pins.check_bandwidth_tables(orc) == []


def test_bandwidth_pin_rejects_other_sizes():
    # the printed figures single out the column term of the byte count: the
    # obvious alternatives fail. (Every printed shape has a multiple of 128 rows,
    # so the figures cannot tell row padding apart; the hand-worked cases do.)
    rows_tab = pins.load_bandwidth_rows()
    assert all(r % 128 == 0 for _, r, _, _, _, _ in rows_tab)
    alternatives = {
        "no padding": lambda r, c, G: r * c,
        "no group padding": lambda r, c, G: pins.ru(r, 128) * c,
        "padding of 3 per group": lambda r, c, G: pins.ru(r, 128) * (c + 3 * G),
        "padding of 8 per group": lambda r, c, G: pins.ru(r, 128) * (c + 8 * G),
    }
    for name, fn in alternatives.items():
        misses = sum(not pins.bandwidth_matches(r, c, G, us, gb, fn(r, c, G)) for _, r, c, G, us, gb in rows_tab)
        assert misses > 0, name


def test_rejects_invalid_input(orc):
    A = np.ones((10, 4), np.uint8)
    for kind, offs in [("M", [5, 3]), ("M", [11]), ("M", [-1, 10]), ("K", [5]), ("K", [2, 1])]:
        with pytest.raises(ValueError):
            orc.rearrange(kind, A, offs)
    with pytest.raises(ValueError):
        orc.rearrange("M", A, np.zeros(0, np.int32))


def test_empty_shapes(orc):
    # rows = 0 (M): all groups empty, 128*G*Cp zero bytes
    out = orc.rearrange("M", np.zeros((0, 6), np.uint8), [0, 0])
    assert out.size == 256 * 8 and not out.any()
    # cols = 0: M writes nothing; K writes Rp*4G zeros
    assert orc.rearrange("M", np.zeros((5, 0), np.uint8), [5]).size == 0
    out = orc.rearrange("K", np.zeros((5, 0), np.uint8), [0, 0, 0])
    assert out.size == 128 * 12 and not out.any()
    assert orc.rearrange("K", np.zeros((0, 7), np.uint8), [7]).size == 0


@pytest.mark.parametrize("name", ["m_groups_tiny", "m_groups_skinny", "m_groups_experts", "k_groups"])
def test_workload_invariants(orc, name):
    w = workloads.make(name)
    out = orc.rearrange(w.kind, w.scales, w.offs)
    assert out.size == orc.out_bytes(w.kind, w.rows, w.cols, w.num_groups)
    # a permutation of the input plus zeros: histograms agree byte value by byte value
    hist_in = np.bincount(w.scales.reshape(-1), minlength=256)
    hist_out = np.bincount(out, minlength=256)
    assert hist_in[0] == 0
    assert np.array_equal(hist_out[1:], hist_in[1:])
    assert hist_out[0] == out.size - w.rows * w.cols


def test_workload_m_tiny_inverse(orc):
    w = workloads.make("m_groups_tiny")
    assert pins.check_inverse(orc, "M", w.rows, w.cols, w.cols, w.offs) == []


def test_3d_inverse_map_random(orc):
    rng = np.random.default_rng(300)
    fails = []
    for _ in range(60):
        fails += pins.check_inverse_3d(orc, *pins.random_case_3d(rng))
    assert fails == []


def test_3d_brute_force_tiny(orc):
    fails = []
    for E in (0, 1, 2, 3):
        for rows in (0, 1, 5, 127, 128, 129):
            for cols in range(0, 7):
                for ld_pad, es_pad in ((0, 0), (2, 0), (1, 9)):
                    ld = cols + ld_pad
                    fails += pins.check_inverse_3d(orc, E, rows, cols, rows * ld + es_pad, ld)
    assert fails == []


def test_3d_per_expert_reshape(orc):
    assert pins.check_3d_reshape(orc, np.random.default_rng(9)) == []


def test_3d_is_m_groups_of_equal_size(orc):
    # experts of N rows each are M groups of N rows: same bytes over the 3-D output
    rng = np.random.default_rng(10)
    for E, N, C in [(1, 5, 3), (3, 128, 8), (4, 200, 13), (2, 1, 1)]:
        A = rng.integers(1, 256, size=(E, N, C), dtype=np.uint8)
        out = orc.rearrange_3d(A)
        m = orc.rearrange("M", A.reshape(E * N, C), [N * (e + 1) for e in range(E)])
        assert np.array_equal(out, m[: out.size])
        assert not m[out.size:].any()


def test_3d_sizes_and_errors(orc):
    assert orc.out_bytes_3d(64, 8192, 160) == 64 * 8192 * 160
    assert orc.out_bytes_3d(3, 129, 5) == 3 * 256 * 8
    assert orc.out_bytes_3d(0, 100, 100) == 0
    assert orc.rearrange_3d(np.zeros((2, 0, 5), np.uint8)).size == 0
    out = orc.rearrange_3d(np.zeros((2, 3, 0), np.uint8))
    assert out.size == 0
    rc = orc.lib.oracle_3d(None, 1, 4, 4, 16, 3, None)  # ld < cols
    assert rc != 0


@pytest.mark.parametrize("name", ["experts_3d_small", "experts_3d_e16", "experts_3d_e64"])
def test_3d_workload_invariants(orc, name):
    w = workloads.make(name)
    out = orc.rearrange_3d(w.scales)
    hist_in = np.bincount(w.scales.reshape(-1), minlength=256)
    hist_out = np.bincount(out, minlength=256)
    assert hist_in[0] == 0
    assert np.array_equal(hist_out[1:], hist_in[1:])
    assert hist_out[0] == out.size - w.scales.size


# --------------------------------------------------------------------------
# planted mistakes: each broken copy of the oracle must fail at least one pin
# --------------------------------------------------------------------------

MUTANTS = {
    # each replacement keeps every write inside the output buffer
    "swapped in-tile strides": ("return (r % 32) * 16 + (r / 32) * 4 + c;",
                                "return (r / 32) * 16 + (r % 32) * 4 + c;"),
    "tile index drops the column block": ("int64_t tile = (i / 128) * (ncols / 4) + (j / 4);",
                                          "int64_t tile = (i / 128) * (ncols / 4);"),
    "M groups not advanced": ("        out_row += padded_rows;\n", "\n"),
    "M rows padded to 64": ("int64_t padded_rows = round_up(size, 128);",
                            "int64_t padded_rows = round_up(size, 64);"),
    "K one global matrix": ("group_out[blocked_byte(padded_width, i, j)] = v;",
                            "out[blocked_byte((cols + 4 * (int64_t)num_groups) / 4 * 4, i, out_col + j)] = v;"),
    "K source column off by one": ("v = scales[i * ld + group_start + j];",
                                   "v = scales[i * ld + group_start + j + (j + 1 < width)];"),
    "K output size without group padding": ("return round_up(rows, 128) * (cols + 4 * (int64_t)num_groups);",
                                            "return round_up(rows, 128) * (cols + 3 * (int64_t)num_groups);"),
    "M row stride taken as cols": ("v = scales[(group_start + i) * ld + j];",
                                   "v = scales[(group_start + i) * cols + j];"),
    "3-D expert stride ignored": ("v = scales[e * expert_stride + i * ld + j];",
                                  "v = scales[e * rows * ld + i * ld + j];"),
    "3-D experts packed without row padding": ("uint8_t *expert_out = out + e * padded_rows * padded_cols;",
                                               "uint8_t *expert_out = out + e * rows * padded_cols;"),
    "3-D columns not padded": ("expert_out[blocked_byte(padded_cols, i, j)] = v;",
                               "expert_out[blocked_byte(cols, i, j)] = v;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]

    def all_pins(mut):
        rng = np.random.default_rng(3)
        fails = pins.check_positions(mut)
        fails += pins.check_bandwidth_tables(mut)
        for kind in ("M", "K"):
            for _ in range(10):
                rows, cols, ld, offs = pins.random_case(rng, kind)
                try:
                    fails += pins.check_inverse(mut, kind, rows, cols, ld, offs)
                except (AssertionError, ValueError, IndexError) as e:
                    fails.append(repr(e))
        for _ in range(10):
            fails += pins.check_inverse_3d(mut, *pins.random_case_3d(rng))
        fails += pins.check_3d_reshape(mut, rng)
        return fails

    assert pins.with_mutant(old, new, all_pins), "mutant '%s' passed every pin" % name


@pytest.mark.parametrize("kind", ["M", "K"])
def test_unrearrange_inverts_and_follows_the_map(orc, kind):
    rng = np.random.default_rng(90 if kind == "M" else 91)
    fails = []
    for _ in range(40):
        rows, cols, ld, offs = pins.random_case(rng, kind)
        fails += pins.check_unrearrange(orc, kind, rows, cols, ld, offs, rng)
    assert fails == []


UNREARRANGE_MUTANTS = {
    "inverse M reads unpadded rows": ("scales[(group_start + i) * ld + j] = blocked[blocked_byte(padded_cols, out_row + i, j)];",
                                      "scales[(group_start + i) * ld + j] = blocked[blocked_byte(padded_cols, group_start + i, j)];"),
    "inverse K group matrix unpadded width": ("scales[i * ld + group_start + j] = group_in[blocked_byte(padded_width, i, j)];",
                                              "scales[i * ld + group_start + j] = group_in[blocked_byte(width, i, j)];"),
}


@pytest.mark.parametrize("name", sorted(UNREARRANGE_MUTANTS))
def test_unrearrange_planted_mistake_is_caught(name):
    old, new = UNREARRANGE_MUTANTS[name]

    def all_pins(mut):
        rng = np.random.default_rng(92)
        fails = []
        for kind in ("M", "K"):
            for _ in range(15):
                rows, cols, ld, offs = pins.random_case(rng, kind)
                fails += pins.check_unrearrange(mut, kind, rows, cols, ld, offs, rng)
        return fails

    assert pins.with_mutant(old, new, all_pins), "mutant '%s' passed every pin" % name


@pytest.mark.parametrize("kind", ["M", "K"])
def test_threaded_call_equals_the_definition(orc, kind):
    # the CPU baseline's all-core form of one call: the same bytes as the single-threaded definition
    # (itself pinned above), on random shapes, strides, empty groups and short totals, for several
    # thread counts, and on the large named workload of each kind
    rng = np.random.default_rng(300 if kind == "M" else 400)
    for _ in range(40):
        rows, cols, ld, offs = pins.random_case(rng, kind)
        buf = rng.integers(0, 256, size=max(rows * ld, 1), dtype=np.uint8)
        A = np.lib.stride_tricks.as_strided(buf, shape=(rows, cols), strides=(ld, 1))
        want = orc.rearrange(kind, A, offs)
        for threads in (1, 2, 3, 8):
            assert np.array_equal(orc.rearrange(kind, A, offs, threads=threads), want), (rows, cols, ld, offs)
    w = workloads.make("m_groups_skinny" if kind == "M" else "k_groups")
    assert np.array_equal(orc.rearrange(kind, w.scales, w.offs, threads=8), orc.rearrange(kind, w.scales, w.offs))
