"""Pins of the MXFP8 dim0-cast oracle (no GPU).

The oracle's E4M3 table and rounding are checked against torch's float8_e4m3fn
(a library implementation of the same format), its scale rule against the
closed form for powers of two, whole blocks against hand-worked values, any
result against properties every correct one has (the scale range and the
half-step error bound), and its blocked scales against the layout decoded from
the tile geometry. Deliberately broken copies must fail these pins.
"""

import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


def test_e4m3_table_matches_torch(orc):
    assert pins.check_e4m3_table(orc) == []


def test_e4m3_rounding_matches_torch(orc):
    assert pins.check_e4m3_encode(orc, np.random.default_rng(40)) == []


def test_scale_closed_form(orc):
    assert pins.check_scale_closed_form(orc) == []


def test_hand_worked_blocks(orc):
    assert pins.check_golden_blocks(orc) == []


def test_round_trip_properties(orc):
    assert pins.check_round_trip(orc, np.random.default_rng(41)) == []


def test_nonfinite_blocks(orc):
    assert pins.check_nonfinite(orc) == []


def test_blocked_scales_layout(orc):
    assert pins.check_blocked_scales(orc, np.random.default_rng(42)) == []


def test_strided_input_equals_packed(orc):
    rng = np.random.default_rng(43)
    base = pins.random_bf16_rows(rng, 50, 160)
    view = base[:, :96]                     # row stride 160 elements
    q1, s1 = orc.quantize_dim0(view)
    q2, s2 = orc.quantize_dim0(np.ascontiguousarray(view))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_dim1_is_dim0_of_the_transpose(orc):
    assert pins.check_dim1_transpose(orc, np.random.default_rng(45)) == []


def test_dim1_blocked_scales_layout(orc):
    assert pins.check_dim1_blocked(orc, np.random.default_rng(46)) == []


def test_dim1_3d_equals_dim1_of_the_stacked_experts(orc):
    assert pins.check_dim1_3d(orc, np.random.default_rng(48)) == []


DIM1_3D_MUTANTS = {
    "expert stride ignored": ("rc = oracle_quantize_dim1(x + e * expert_stride, K, N, ld, q + e * N * K",
                              "rc = oracle_quantize_dim1(x + 0 * expert_stride, K, N, ld, q + e * N * K"),
    "codes of an expert K bytes apart": ("K, N, ld, q + e * N * K, scales + e * per);",
                                         "K, N, ld, q + e * K, scales + e * per);"),
    "every expert gets expert 0's scales": ("oracle_3d(scales, E, N, K / 32, per, K / 32, blocked)",
                                            "oracle_3d(scales, E, N, K / 32, 0, K / 32, blocked)"),
}


@pytest.mark.parametrize("name", sorted(DIM1_3D_MUTANTS))
def test_dim1_3d_planted_mistake_is_caught(name):
    old, new = DIM1_3D_MUTANTS[name]
    fails = pins.with_mutant(old, new, lambda mut: pins.check_dim1_3d(mut, np.random.default_rng(48)))
    assert fails, "planted mistake '%s' passed every pin" % name


def test_scales_only_functions_agree(orc):
    rng = np.random.default_rng(47)
    x = pins.random_bf16_rows(rng, 96, 192)
    assert np.array_equal(orc.scales_dim0(x), orc.quantize_dim0(x)[1])
    assert np.array_equal(orc.scales_dim1(x), orc.quantize_dim1(x)[1])
    x[5, 7] = 0x7F80
    assert np.array_equal(orc.scales_dim1(x), orc.quantize_dim1(x)[1])


def test_dim1_rejects_bad_offsets(orc):
    x = np.zeros((64, 8), np.uint16)
    for offs in ([65], [40, 32], [-32, 64]):
        with pytest.raises(ValueError):
            orc.quantize_dim1_K_groups(x, offs)


def test_rejects_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.quantize_dim0(np.zeros((4, 48), np.uint16))     # K not a multiple of 32
    q, s = orc.quantize_dim0(np.zeros((0, 64), np.uint16))
    assert q.shape == (0, 64) and s.shape == (0, 2)


def test_workload_invariants(orc):
    import workloads

    w = workloads.make("quant_m_groups_small")
    q, blocked = orc.quantize_dim0_M_groups(w.x, w.offs)
    assert q.shape == (w.rows, w.K)
    assert blocked.size == orc.out_bytes("M", w.rows, w.K // 32, w.num_groups)
    assert not (q == 0x7F).any() and not (q == 0xFF).any()   # finite inputs give finite codes


MUTANTS = {
    "scale exponent 7": ("int s = (e - 1) - 8;", "int s = (e - 1) - 7;"),
    "floor(log2) off by one": ("int s = (e - 1) - 8;", "int s = e - 8;"),
    "E8M0 bias 126": ("return s + 127;", "return s + 126;"),
    "ties away from zero": ("if (err < best_err || (err == best_err && (c & 1) == 0)) {",
                            "if (err <= best_err) {"),
    "truncation instead of rounding": ("double err = fabs(a - value[c]);",
                                       "double err = value[c] <= a ? a - value[c] : 1e300;"),
    "sign dropped": ("return (uint8_t)(best | (signbit(y) ? 0x80 : 0));", "return (uint8_t)best;"),
    "signed maximum instead of magnitude": ("else if (fabs(v) > amax) amax = fabs(v);", "else if (v > amax) amax = v;"),
    "non-finite blocks quantised as finite": ("if (isnan(v) || isinf(v)) finite = 0;\n                else if",
                                              "if (isnan(v) || isinf(v)) continue;\n                else if"),
    "dim1 block along the feature dimension": ("x[(32 * b + k) * ld + n]", "x[(32 * b) * ld + n + k]"),
    "dim1 row stride taken as N": ("x[(32 * b + k) * ld + n]", "x[(32 * b + k) * N + n]"),
    "dim1 token offsets not divided by 32": ("scale_offs[g] = offs[g] / 32;", "scale_offs[g] = offs[g];"),
    "dim1 code rows 32 bytes apart": ("uint8_t *qb = qT + n * T + 32 * b;", "uint8_t *qb = qT + n * 32 + 32 * b;"),
    "subnormal exponent field": ("double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);",
                                 "double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -7);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]

    def all_pins(mut):
        rng = np.random.default_rng(44)
        fails = pins.check_e4m3_table(mut) + pins.check_e4m3_encode(mut, rng) + pins.check_scale_closed_form(mut)
        fails += pins.check_golden_blocks(mut) + pins.check_nonfinite(mut)
        try:
            fails += pins.check_round_trip(mut, rng)
        except (ValueError, IndexError) as e:
            fails.append(repr(e))
        fails += pins.check_dim1_transpose(mut, rng) + pins.check_dim1_blocked(mut, rng)
        return fails

    assert pins.with_mutant(old, new, all_pins), "mutant '%s' passed every pin" % name
