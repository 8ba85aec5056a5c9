"""Pins of the per-group row padding oracle (no GPU).

Padding puts each group's rows where the M-groups scale layout puts that
group's scale rows (measured from the pinned scale oracle on index-coded
inputs); unpadding inverts it; hand-worked placements; planted mistakes fail.
"""

import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


def test_pad_rows_follow_the_m_groups_layout(orc):
    assert pins.check_pad_placement(orc, np.random.default_rng(70)) == []


def test_unpad_inverts_pad(orc):
    assert pins.check_unpad_round_trip(orc, np.random.default_rng(71)) == []


def test_hand_worked_placement(orc):
    A = np.arange(1, 19, dtype=np.uint8).reshape(6, 3)
    P = orc.pad_M_groups(A, [2, 2, 6])
    assert P.shape == (6 + 3 * 128, 3)
    assert np.array_equal(P[0:2], A[0:2])            # group 0 at row 0
    assert np.array_equal(P[128:132], A[2:6])        # group 1 empty; group 2 at 128 = round_up(2, 128)
    assert not P[2:128].any() and not P[132:].any()
    A2 = np.full((300, 2), 7, np.uint8)
    P2 = orc.pad_M_groups(A2, [129, 300])             # 129 rows pad to 256
    assert (P2[:129] == 7).all() and not P2[129:256].any() and (P2[256:427] == 7).all() and not P2[427:].any()


def test_strided_input(orc):
    rng = np.random.default_rng(72)
    base = rng.integers(1, 256, size=(50, 12), dtype=np.uint8)
    assert np.array_equal(orc.pad_M_groups(base[:, :5], [20, 50]),
                          orc.pad_M_groups(np.ascontiguousarray(base[:, :5]), [20, 50]))


def test_rejects_invalid(orc):
    A = np.ones((10, 4), np.uint8)
    for offs in ([5, 3], [11], [-1, 10]):
        with pytest.raises(ValueError):
            orc.pad_M_groups(A, offs)


MUTANTS = {
    "pad groups to 64 rows": ("        out_row += round_up(size, 128);\n        start = offs[g];\n    }\n    return ORACLE_OK;\n}\n\nint oracle_unpad",
                              "        out_row += round_up(size, 64);\n        start = offs[g];\n    }\n    return ORACLE_OK;\n}\n\nint oracle_unpad"),
    "pad output row stride ld": ("padded[(out_row + i) * cols + j] = data[(start + i) * ld + j];",
                                 "padded[(out_row + i) * cols + j] = data[(start + i) * cols + j];"),
    "unpad reads unpadded rows": ("data[(start + i) * ld + j] = padded[(in_row + i) * cols + j];",
                                  "data[(start + i) * ld + j] = padded[(start + i) * cols + j];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]

    def all_pins(mut):
        fails = pins.check_pad_placement(mut, np.random.default_rng(73))
        fails += pins.check_unpad_round_trip(mut, np.random.default_rng(74))
        # strided input distinguishes the row stride
        base = np.random.default_rng(75).integers(1, 256, size=(40, 9), dtype=np.uint8)
        if not np.array_equal(mut.pad_M_groups(base[:, :4], [40]), oracle.pad_M_groups(np.ascontiguousarray(base[:, :4]), [40])):
            fails.append("strided input differs")
        return fails

    assert pins.with_mutant(old, new, all_pins), "mutant '%s' passed every pin" % name
