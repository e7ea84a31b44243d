"""Pins for the oracle's tables: NF4 levels and thresholds, the 8-bit constant
table T8 and its thresholds, and the storage accounting.

Each test checks the oracle against something other than itself: an
independent library routine, a closed form, an invariant, or brute force in
exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import nf4

DELTA = 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
P_TOP = 1.0 - DELTA


# ----------------------------------------------------------------- NF4 levels

def test_nf4_levels_match_second_inverse_normal_routine():
    # Same construction evaluated with scipy's ndtri instead of the stdlib
    # NormalDist.inv_cdf: the fp32 bit patterns must agree.
    pos = scipy.special.ndtri(np.linspace(P_TOP, 0.5, 9)[:8])
    neg = -scipy.special.ndtri(np.linspace(P_TOP, 0.5, 8)[:7])
    v = np.sort(np.concatenate([pos, neg, [0.0]]))
    v = (v / np.max(np.abs(v))).astype(np.float32)
    assert np.array_equal(v.view(np.uint32), nf4.nf4_levels().view(np.uint32))


def test_nf4_levels_invariants():
    lv = nf4.nf4_levels()
    assert lv.dtype == np.float32 and lv.shape == (16,)
    assert np.all(np.diff(lv) > 0), "strictly increasing"
    assert lv[0] == -1.0 and lv[15] == 1.0
    assert lv[7] == 0.0 and not np.signbit(lv[7]), "code 7 is an exact +0"
    assert np.sum(lv < 0) == 7 and np.sum(lv > 0) == 8, "asymmetric: 7 negative, 8 positive"


def test_nf4_levels_are_equal_probability_quantiles():
    # Invert with the normal CDF (a different routine from the one that built
    # the table): the positive levels must sit at 8 equally spaced
    # probabilities from 1/2 to P_TOP, the negative at 7.
    lv = nf4.nf4_levels_fp64()
    top = scipy.stats.norm.ppf(P_TOP)
    p_pos = scipy.stats.norm.cdf(lv[7:] * top)       # 0 and the 8 positive
    p_neg = scipy.stats.norm.cdf(-lv[:8][::-1] * top)  # 0 and the 7 negative, mirrored
    assert np.allclose(p_pos, 0.5 + (P_TOP - 0.5) * np.arange(9) / 8, atol=1e-12)
    assert np.allclose(p_neg, 0.5 + (P_TOP - 0.5) * np.arange(8) / 7, atol=1e-12)


def test_nf4_more_resolution_near_zero():
    # The levels follow the Gaussian: spacing grows away from zero on each side.
    lv = nf4.nf4_levels().astype(np.float64)
    pos_gaps = np.diff(lv[7:])
    neg_gaps = np.diff(lv[:8])[::-1]
    assert np.all(np.diff(pos_gaps) > 0)
    assert np.all(np.diff(neg_gaps) > 0)


# ------------------------------------------------------------ threshold rule

def _exact_nearest(x, levels):
    """argmin |x - L_i| in exact rationals, ties to the lower index."""
    xf = Fraction(float(x))
    best, best_d = None, None
    for i, l in enumerate(levels):
        d = abs(xf - Fraction(float(l)))
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def _vector_nearest(x, levels):
    """Vectorised exact nearest for fp32 x, levels in [-1, 1]: the fp64
    differences of two fp32 numbers of magnitude >= 2^-30 apart from zero are
    exact, and near a decision boundary both are far from zero."""
    x = np.asarray(x, np.float32).astype(np.float64)
    d = np.abs(x[:, None] - levels.astype(np.float64)[None, :])
    return np.argmin(d, axis=1)   # argmin returns the first (lower) index on ties


def _key(f):
    """Monotone integer key of a fp32 value (negatives mirrored)."""
    b = int(np.float32(f).view(np.uint32))
    return b if b < 0x80000000 else -(b & 0x7FFFFFFF)


def _from_keys(keys):
    keys = np.asarray(keys, dtype=np.int64)
    bits = np.where(keys >= 0, keys, (-keys) | 0x80000000).astype(np.uint32)
    return bits.view(np.float32)


def _window(center, half_width):
    """All fp32 values within half_width representable steps of center."""
    k = _key(np.float32(center))
    return _from_keys(np.arange(k - half_width, k + half_width + 1))


@pytest.mark.parametrize("table", ["nf4", "t8"])
def test_threshold_rule_is_exact_nearest_near_every_boundary(table):
    levels = nf4.nf4_levels() if table == "nf4" else nf4.t8_levels()
    tau = nf4.midpoint_thresholds(levels)
    width = 3000 if table == "nf4" else 300
    for i in range(len(levels) - 1):
        mid = (float(levels[i]) + float(levels[i + 1])) / 2
        xs = _window(mid, width)
        xs = xs[np.abs(xs) <= 1.0]
        got = nf4.nearest_code(xs, tau)
        want = _vector_nearest(xs, levels)   # T8: -0 and +0 tie, 127 wins
        assert np.array_equal(got, want), (table, i)


def test_nf4_threshold_rule_strided_sweep_of_all_fp32_in_unit_interval():
    # Every 499th fp32 bit pattern in [0, 1] and in [-1, -0].
    top = int(np.float32(1.0).view(np.int32))
    pos = np.arange(0, top + 1, 499, dtype=np.int64).astype(np.int32).view(np.float32)
    xs = np.concatenate([pos, -pos, np.float32([1.0, -1.0])])
    lv = nf4.nf4_levels()
    got = nf4.nearest_code(xs, nf4.nf4_thresholds())
    want = _vector_nearest(xs, lv)
    assert np.array_equal(got, want)


def test_nf4_exact_ties_go_to_lower_code():
    lv = nf4.nf4_levels()
    tau = nf4.nf4_thresholds()
    ties = []
    for i in range(15):
        mid = Fraction(float(lv[i])) + Fraction(float(lv[i + 1]))
        mid /= 2
        f = np.float32(float(mid))
        if Fraction(float(f)) == mid:
            ties.append((i, f))
            assert nf4.nearest_code([f], tau)[0] == i
            assert _exact_nearest(f, lv) == i
    # Four midpoints happen to be representable in fp32.
    assert [i for i, _ in ties] == [2, 6, 7, 14]


def test_nf4_naive_fp32_midpoint_rule_cases():
    # Inputs where comparing against the round-to-nearest fp32 midpoint would
    # give the wrong code; the oracle must give the exact nearest level.
    lv = nf4.nf4_levels()
    tau = nf4.nf4_thresholds()
    naive = ((lv[:-1].astype(np.float64) + lv[1:].astype(np.float64)) / 2).astype(np.float32)
    cases = []
    for i in range(15):
        x = naive[i]
        exact = _exact_nearest(x, lv)
        if int(np.searchsorted(naive, np.float32(x), side="left")) != exact:
            cases.append((x.view(np.uint32), exact))
            assert nf4.nearest_code([x], tau)[0] == exact
    assert len(cases) == 6
    hexes = sorted("%08x" % int(h) for h, _ in cases)
    assert hexes == sorted(["bf591cd8", "beadea74", "3df64860", "3e9582d2", "3ec753f6", "3f006d02"])


def test_nf4_code_of_levels_and_zeros():
    lv = nf4.nf4_levels()
    tau = nf4.nf4_thresholds()
    assert np.array_equal(nf4.nearest_code(lv, tau), np.arange(16))
    assert nf4.nearest_code(np.float32([0.0, -0.0]), tau).tolist() == [7, 7]


# ------------------------------------------------------------------------ T8

def test_t8_magnitudes_match_torch_float8_e4m3fn():
    # torch's float8_e4m3fn has the same bias-7 exponent and 3-bit mantissa;
    # it spends byte 0x7f on NaN, which the T8 reading uses for 480.
    m = nf4.t8_magnitudes()
    b = torch.arange(127, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(m[:127], ref)
    assert m[127] == 480.0 and m[126] == 448.0


def test_t8_table_invariants():
    t = nf4.t8_levels()
    assert t.dtype == np.float32 and t.shape == (256,)
    assert t[0] == -1.0 and t[255] == 1.0
    assert t[127] == 0.0 and np.signbit(t[127]) and t[128] == 0.0 and not np.signbit(t[128])
    # symmetric about the median, bit for bit apart from the sign
    assert np.array_equal(t[::-1].view(np.uint32) ^ np.uint32(0x80000000), t.view(np.uint32))
    assert np.all(np.diff(t[:128]) > 0) and np.all(np.diff(t[128:]) > 0)
    # entries are the fp32 quotient of the magnitude by 480
    for k in range(128):
        assert t[128 + k] == np.float32(np.float32(nf4.t8_magnitudes()[k]) / np.float32(480.0))


def test_t8_codes_of_special_values():
    tau = nf4.t8_thresholds()
    assert nf4.nearest_code(np.float32([0.0, -0.0, 1.0, -1.0]), tau).tolist() == [127, 127, 255, 0]
    t = nf4.t8_levels()
    codes = nf4.nearest_code(t, tau)
    expected = np.arange(256)
    expected[128] = 127   # +0 ties with -0, lower index
    assert np.array_equal(codes, expected)


def test_t8_threshold_strided_sweep():
    top = int(np.float32(1.0).view(np.int32))
    pos = np.arange(0, top + 1, 997, dtype=np.int64).astype(np.int32).view(np.float32)
    xs = np.concatenate([pos, -pos])
    lv = nf4.t8_levels()
    got = nf4.nearest_code(xs, nf4.t8_thresholds())
    want = _vector_nearest(xs, lv)
    assert np.array_equal(got, want)


# ---------------------------------------------------------- storage accounting

def test_double_quant_saves_about_0_37_bits_per_param():
    # Pages: DQ saves ~0.37 bits/param, roughly 3 GB on a 65B model
    # (automatone.win "QLoRA paper explained", How it works / Double
    # Quantization; creativeworksofknowledge.com "QLoRA: Fine-Tune 70B on One
    # GPU", The three innovations / 2).
    n = 64 * 256 * 4096
    bits = nf4.storage_bits_per_param(n)
    const_bits = bits - 4.0
    assert abs(const_bits - (8 / 64 + 32 / (64 * 256))) < 1e-6
    saving = 32 / 64 - const_bits
    assert abs(saving - 0.373) < 1e-3
    assert abs(65e9 * saving / 8 / 1e9 - 3.03) < 0.01
    # ~36 GB for 70B in the QLoRA column of the memory table (weights only)
    assert abs(70e9 * bits / 8 / 1e9 - 36.1) < 0.1
    # block size 64 is the one that gives ~0.37: 32 and 128 do not
    for b1, ok in ((32, False), (64, True), (128, False)):
        s = 32 / b1 - (8 / b1 + 32 / (b1 * 256))
        assert (abs(s - 0.37) < 0.01) == ok
