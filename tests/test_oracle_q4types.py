"""Pins for the oracle's FP4 and Int4 level tables (the 4-bit types the pages
compare NF4 with) and for the codec built on them.

Each test checks the oracle against something other than itself: a published
value table, a closed form or invariant, brute force in exact rational
arithmetic, or the ordering of reconstruction errors the pages state.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4
from oracle.bf16 import bf16_bits_to_fp64

# Non-negative values of the 4-bit float E2M1 as listed in the OCP
# Microscaling Formats specification's FP4 table (codes 0b000 .. 0b111).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _exact_nearest(x, levels):
    """argmin |x - L_i| in exact rationals, ties to the lower index."""
    xf = Fraction(float(x))
    best, best_d = None, None
    for i, l in enumerate(levels):
        d = abs(xf - Fraction(float(l)))
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def _key(f):
    b = int(np.float32(f).view(np.uint32))
    return b if b < 0x80000000 else -(b & 0x7FFFFFFF)


def _from_keys(keys):
    keys = np.asarray(keys, dtype=np.int64)
    bits = np.where(keys >= 0, keys, (-keys) | 0x80000000).astype(np.uint32)
    return bits.view(np.float32)


# ------------------------------------------------------------------- tables

def test_fp4_magnitudes_match_the_published_e2m1_table():
    assert nf4.fp4_magnitudes().tolist() == E2M1_TABLE


def test_fp4_levels():
    lv = nf4.fp4_levels()
    assert lv.dtype == np.float32 and lv.shape == (16,)
    want = [-v / 6.0 for v in reversed(E2M1_TABLE[1:])] + [0.0, 0.0] + [v / 6.0 for v in E2M1_TABLE[1:]]
    # each level is the fp32 value nearest to the rational v / 6
    for got, w in zip(lv.tolist(), want):
        assert got == float(np.float32(w))
    assert lv[0] == -1.0 and lv[15] == 1.0
    assert np.all(np.diff(lv.astype(np.float64)) >= 0)
    assert [i for i in range(15) if lv[i] == lv[i + 1]] == [7], "only the two zeros are equal"
    assert not np.signbit(lv[7]) and not np.signbit(lv[8])
    assert np.array_equal(lv, -lv[::-1]), "symmetric"


def test_int4_levels_are_sevenths():
    lv = nf4.int4_levels()
    assert lv.dtype == np.float32 and lv.shape == (16,)
    for k, got in zip(range(-8, 8), lv.tolist()):
        exact = Fraction(k, 7)
        assert abs(Fraction(got) - exact) <= abs(exact) * Fraction(1, 2 ** 24)
    assert lv[1] == -1.0 and lv[8] == 0.0 and lv[15] == 1.0
    gaps = np.diff(lv.astype(np.float64))
    assert np.allclose(gaps, 1.0 / 7.0, rtol=0, atol=2e-7), "evenly spaced"


def test_zero_codes():
    for qt in nf4.QTYPES:
        assert nf4.q4_levels(qt)[nf4.q4_zero_code(qt)] == 0.0


# -------------------------------------------------------------- code rule

@pytest.mark.parametrize("qtype", ["fp4", "int4"])
def test_threshold_rule_is_exact_nearest_near_every_boundary(qtype):
    levels = nf4.q4_levels(qtype)
    tau = nf4.midpoint_thresholds(levels)
    lv64 = levels.astype(np.float64)
    for i in range(15):
        if levels[i] == levels[i + 1]:
            continue
        mid = (float(levels[i]) + float(levels[i + 1])) / 2
        k = _key(np.float32(mid))
        xs = _from_keys(np.arange(k - 2000, k + 2001))
        xs = xs[np.abs(xs) <= 1.0]
        got = nf4.nearest_code(xs, tau)
        d = np.abs(xs.astype(np.float64)[:, None] - lv64[None, :])
        want = np.argmin(d, axis=1)   # first (lower) index on ties; differences exact here
        assert np.array_equal(got, want), (qtype, i)


@pytest.mark.parametrize("qtype", ["fp4", "int4"])
def test_codes_of_levels_zero_and_ends(qtype):
    lv = nf4.q4_levels(qtype)
    tau = nf4.midpoint_thresholds(lv)
    reach = np.array([i for i in range(16) if abs(float(lv[i])) <= 1.0 and (i == 0 or lv[i] != lv[i - 1])])
    assert np.array_equal(nf4.nearest_code(lv[reach], tau), reach)
    z = nf4.q4_zero_code(qtype)
    assert nf4.nearest_code(np.float32([0.0, -0.0]), tau).tolist() == [z, z]
    assert nf4.nearest_code(np.float32([-1.0, 1.0]), tau).tolist() == [int(reach[0]), 15]


@pytest.mark.parametrize("qtype", ["nf4", "fp4", "int4"])
def test_quantize_matches_brute_force_on_a_small_tensor(qtype):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(64 * 5 + 17) * 0.02).astype(np.float32)
    w[64:128] = 0.0                                  # a zero block
    w[128:192] = nf4.q4_levels(qtype)[rng.integers(0, 16, 64)] * np.float32(0.05)
    qd = nf4.quantize(w, qtype)
    assert qd["qtype"] == qtype
    lv = nf4.q4_levels(qtype)
    for b in range(6):
        blk = w[64 * b:64 * b + 64]
        c = np.float32(np.max(np.abs(blk)))
        for j, x in enumerate(blk):
            want = nf4.q4_zero_code(qtype) if c == 0 else _exact_nearest(np.float32(x / c), lv)
            assert qd["codes"][64 * b + j] == want, (b, j)
    # the zero block dequantizes to exact zeros
    deq = bf16_bits_to_fp64(nf4.dequantize_q(qd))
    assert np.all(deq[64:128] == 0.0)


# -------------------------------------------------- the pages' comparison

def test_nf4_reconstruction_error_below_fp4_and_int4():
    # The pages: NF4 beats FP4 and Int4 on quantization precision for
    # zero-centred normally distributed weights.
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(1 << 17) * 0.02).astype(np.float32)
    mse = {}
    for qt in nf4.QTYPES:
        deq = bf16_bits_to_fp64(nf4.dequantize_q(nf4.quantize(w, qt)))
        mse[qt] = float(np.mean((deq - w.astype(np.float64)) ** 2))
    assert mse["nf4"] < 0.85 * mse["fp4"]
    assert mse["nf4"] < 0.85 * mse["int4"]
