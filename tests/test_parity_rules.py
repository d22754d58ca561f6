"""The parity bar's own rules, checked on the CPU with planted GPU results.

`assert_pack_matches` lets a tie-ambiguous scale differ from the oracle's rounding, but
only to the quotient's other rounding neighbour. These tests hand it results built from
the oracle with one entry changed and check that each wrong one is refused.
"""
import numpy as np
import pytest

from oracle import rb_oracle as O
from tests.gpu_util import assert_pack_matches

# Row 0's first quotient is the mean of its magnitudes, (4 + 2^-9) / 4 = 1 + 2^-11: exactly
# halfway between the fp16 values 1 and 1 + 2^-10, so ties-to-even gives 1 and the other
# neighbour is 1 + 2^-10. Its residuals differ in sign and size between the two choices.
# Rows 1 and 2 have ordinary quotients.
W = np.array([[1.0 - 2.0 ** -8, -1.0 - 2.0 ** -8 - 2.0 ** -9, 1.0, 1.0],
              [0.3, -0.7, 0.2, 0.9],
              [-1.5, 0.25, 0.5, -0.125]], dtype=np.float32)


def _oracle(k, forced=None):
    r = O.binarize(W, k, scale_fmt="f16", forced_g=forced)
    return r["planes"].copy(), r["g"].copy()


def test_ambiguous_case_is_flagged():
    r = O.binarize(W, 2, scale_fmt="f16")
    assert r["ambiguous"][0, 0, 0] and not r["ambiguous"][0, 1:, 0].any()
    assert r["g"][0, 0, 0] == 1.0 and r["quot"][0, 0, 0] == 1.0 + 2.0 ** -11


@pytest.mark.parametrize("k", [1, 2])
def test_oracle_result_passes(k):
    p, g = _oracle(k)
    assert_pack_matches(W, k, None, "f16", 0, p, g)


def test_other_neighbour_with_its_own_later_planes_passes():
    # the GPU rounds row 0's first scale up; its second plane then follows from that choice
    p, g = _oracle(2, forced={(0, 0, 0): 1.0 + 2.0 ** -10})
    assert g[0, 0, 0] == 1.0 + 2.0 ** -10
    assert_pack_matches(W, 2, None, "f16", 0, p, g)


@pytest.mark.parametrize("wrong", [1.0 + 2.0 ** -9,      # two steps up
                                   1.0 - 2.0 ** -11,     # the neighbour on the far side
                                   1.0 + 3 * 2.0 ** -10])
@pytest.mark.parametrize("k", [1, 2])
def test_wrong_ambiguous_scale_is_refused(k, wrong):
    # for k = 1 this is the last plane, whose scale no later plane's bits depend on
    p, g = _oracle(k, forced={(0, 0, 0): wrong})
    with pytest.raises(AssertionError, match="not a rounding neighbour"):
        assert_pack_matches(W, k, None, "f16", 0, p, g)


def test_wrong_unambiguous_scale_is_refused():
    p, g = _oracle(2)
    g[1, 2, 0] = float(np.nextafter(np.float16(g[1, 2, 0]), np.float16(np.inf)))
    with pytest.raises(AssertionError, match="scale mismatch"):
        assert_pack_matches(W, 2, None, "f16", 0, p, g)


def test_flipped_bit_is_refused():
    p, g = _oracle(2)
    p[1, 1, 0] ^= 1 << 3
    with pytest.raises(AssertionError, match="bits"):
        assert_pack_matches(W, 2, None, "f16", 0, p, g)


def test_later_plane_following_the_oracle_choice_is_refused():
    # first scale rounded up, but the second plane's scale and bits left as the oracle's
    # down-rounding gives them: not what the GPU's own choice implies
    p, g = _oracle(2)
    p_up, g_up = _oracle(2, forced={(0, 0, 0): 1.0 + 2.0 ** -10})
    assert not np.array_equal(g[1, 0], g_up[1, 0])
    g[0, 0, 0] = g_up[0, 0, 0]
    with pytest.raises(AssertionError):
        assert_pack_matches(W, 2, None, "f16", 0, p, g)
