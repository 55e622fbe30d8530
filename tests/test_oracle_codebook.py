"""Pins of the oracle's dynamic-exponent codebooks.

Page: "8-bit Optimizers via Block-wise Quantization" -- abstract (dynamic quantization,
precise for large and small magnitudes; 2^8 = 256 values) and the citing-papers quote
from the k-bit inference scaling-laws paper (one sign bit, then a run of zero bits
giving a base-10 exponent).

The pages print no codebook values, so the exact values are "parity unpinned"
against the deployed system; what is pinned here are the structural facts the
description fixes: 256 distinct sorted values, exact 0 and 1, sign symmetry of the
signed map, one decade of magnitude per exponent, each decade holding 2^(free bits)
equally spaced bin midpoints.
"""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def maps(oref):
    return oref.dynamic_map(True), oref.dynamic_map(False)


def test_sorted_distinct_256(maps):
    for q in maps:
        assert q.dtype == np.float32 and q.shape == (256,)
        assert np.all(np.diff(q) > 0), "codebook must be strictly increasing"
        assert len(np.unique(q)) == 256


def test_exact_zero_and_one(maps):
    qs, qu = maps
    assert qs[127] == 0.0 and qs[255] == 1.0
    assert qu[0] == 0.0 and qu[255] == 1.0
    assert np.all(np.abs(qs) <= 1.0) and np.all(qu >= 0.0) and np.all(qu <= 1.0)


def test_signed_map_is_sign_symmetric(maps):
    qs, _ = maps
    for j in range(1, 128):
        assert qs[127 - j] == -qs[127 + j]


def _decade_members(q, E):
    lo, hi = 0.1 * 10.0 ** (-E), 10.0 ** (-E)
    v = q.astype(np.float64)
    return np.sort(v[(v > lo * (1 - 1e-7)) & (v < hi * (1 - 1e-7))])


@pytest.mark.parametrize("signed,free_bits", [(True, 6), (False, 7)])
def test_decade_structure(maps, signed, free_bits):
    """E leading zero bits select decade 10^-E; the bits after the indicator bit
    (6-E for the signed map, 7-E for the unsigned one) split it linearly."""
    q = maps[0] if signed else maps[1]
    pos = q[q > 0]
    total = 0
    for E in range(0, 7):
        members = _decade_members(pos, E)
        k = free_bits - E
        assert len(members) == 2 ** k, (E, len(members))
        total += len(members)
        lo, hi = 0.1 * 10.0 ** (-E), 10.0 ** (-E)
        step = (hi - lo) / 2 ** k
        # equally spaced bins, each value in the middle of its bin
        # values are fp32-rounded: allow two fp32 ulps of the decade's top
        tol = 2 * float(np.spacing(np.float32(hi)))
        if len(members) > 1:
            np.testing.assert_allclose(np.diff(members), step, rtol=0, atol=tol)
        np.testing.assert_allclose(members[0] - lo, step / 2, rtol=0, atol=tol)
        np.testing.assert_allclose(hi - members[-1], step / 2, rtol=0, atol=tol)
    # every value other than 0 and 1 belongs to one of the seven decades
    assert total == len(pos) - 1


def test_dynamic_range(maps):
    qs, qu = maps
    # smallest magnitudes sit in the 1e-6 decade: the "small magnitude" end of the range
    assert 1e-7 < qs[128] < 1e-6 and 1e-7 < qu[1] < 1e-6
    # largest bin spacing is in the top decade: 0.9/64 (signed) and 0.9/128 (unsigned)
    assert abs(np.diff(qs.astype(np.float64)).max() - 0.9 / 64) < 1e-7
    assert abs(np.diff(qu.astype(np.float64)).max() - 0.9 / 128) < 1e-7
