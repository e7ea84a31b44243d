"""Pins for the oracle's LoRA dropout: the Philox4x32-10 generator against its
authors' known-answer vectors, the keep rate, the bit packing, the reduction
to the dropout-free layer at p = 0, and the backward against finite
differences of the forward for a fixed mask."""

import numpy as np
import pytest

from oracle import dropout as od
from oracle import linear as olin
from oracle.bf16 import round_fp32_to_bf16_bits


# Known-answer vectors published with the Random123 library for
# Philox4x32 with 10 rounds: (counter words, key words, output words).
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = od.philox4x32_10(np.array([ctr], dtype=np.uint32), key)[0]
    assert tuple(int(x) for x in got) == want


def test_keep_rate_and_threshold():
    M, K, p = 512, 2048, 0.05
    keep = od.keep_mask(M, K, p, seed=1234)
    q = 1.0 - od.threshold(p) / 2.0 ** 32
    n = M * K
    assert abs(keep.mean() - q) < 5 * np.sqrt(q * (1 - q) / n)
    assert od.threshold(0.0) == 0 and od.keep_mask(4, 64, 0.0, 7).all()
    assert od.threshold(0.5) == 2 ** 31
    # different seeds give different masks; the same seed the same mask
    assert not np.array_equal(keep, od.keep_mask(M, K, p, seed=1235))
    assert np.array_equal(keep, od.keep_mask(M, K, p, seed=1234))


def test_mask_uses_word_e_mod_4_of_block_e_div_4():
    # element 4 b + w is word w of Philox(counter = (b, 0, 0, 0)), b < 2^32,
    # and the high counter word carries b >> 32 for a 64-bit counter.
    seed = (7 << 32) | 5
    keep = od.keep_mask(3, 8, 0.5, seed).reshape(-1)
    words = od.philox4x32_10(np.array([[b, 0, 0, 0] for b in range(6)], np.uint32), (5, 7))
    assert np.array_equal(keep, words.reshape(-1) >= 2 ** 31)


def test_row_subset_matches_the_full_mask():
    full = od.keep_mask(40, 96, 0.2, 77)
    rows = np.array([0, 7, 39])
    assert np.array_equal(od.keep_mask_rows(rows, 96, 0.2, 77), full[rows])
    # rows that start inside a counter block (K % 4 != 0)
    full = od.keep_mask(9, 70, 0.4, 79)
    rows = np.array([1, 2, 5, 8])
    assert np.array_equal(od.keep_mask_rows(rows, 70, 0.4, 79), full[rows])
    # element by element against the word layout
    seed = 79
    words = od.philox4x32_10(np.array([[b, 0, 0, 0] for b in range(158)], np.uint32), (seed, 0)).reshape(-1)
    assert np.array_equal(full.reshape(-1), words[:630] >= od.threshold(0.4))


def test_bits_round_trip():
    rng = np.random.default_rng(3)
    keep = rng.random((5, 70)) < 0.9
    bits = od.pack_bits(keep)
    assert bits.shape == (5, 3) and bits.dtype == np.uint32
    assert np.array_equal(od.unpack_bits(bits, 70), keep)
    assert int(bits[0, 0]) == sum(int(keep[0, k]) << k for k in range(32))


def _inputs(rng, M, N, K, r):
    bf = lambda a: round_fp32_to_bf16_bits(a.astype(np.float32))
    return (bf(rng.standard_normal((M, K))), rng.standard_normal((N, K)) * 0.02, bf(rng.standard_normal((r, K)) * 0.1),
            bf(rng.standard_normal((N, r)) * 0.1), bf(rng.standard_normal((M, N))))


def test_p0_reduces_to_the_dropout_free_layer():
    rng = np.random.default_rng(9)
    X, Wt, A, B, dY = _inputs(rng, 12, 16, 64, 4)
    keep = od.keep_mask(12, 64, 0.0, 1)
    Y, T = od.linear_fwd(X, Wt, A, B, 2.0, 0.0, keep)
    Y0, T0 = olin.linear_fwd(X, Wt, A, B, 2.0)
    assert np.allclose(Y, Y0, rtol=0, atol=1e-12) and np.allclose(T, 2.0 * T0, rtol=0, atol=1e-12)
    dX, dA, dB, _ = od.linear_bwd(dY, X, Wt, A, B, 2.0, 0.0, keep)
    dX0, dA0, dB0 = olin.linear_bwd(dY, X, Wt, A, B, 2.0)
    for a, b in ((dX, dX0), (dA, dA0), (dB, dB0)):
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_backward_matches_finite_differences_for_a_fixed_mask():
    # L = <dY, Y> is linear in X, A and B for a fixed mask: central
    # differences are exact up to fp64 rounding.
    rng = np.random.default_rng(21)
    M, N, K, r, p = 6, 8, 64, 3, 0.3
    X, Wt, A, B, dY = _inputs(rng, M, N, K, r)
    keep = od.keep_mask(M, K, p, 99)
    assert 0 < keep.sum() < M * K
    Xf, Af, Bf = (olin._f64(t) for t in (X, A, B))
    loss = lambda Xv, Av, Bv: float(np.sum(olin._f64(dY) * od.linear_fwd(Xv, Wt, Av, Bv, 0.5, p, keep)[0]))
    dX, dA, dB, _ = od.linear_bwd(dY, X, Wt, A, B, 0.5, p, keep)
    h = 1e-3
    for name, base, grad, idx in (("X", Xf, dX, (2, 17)), ("A", Af, dA, (1, 40)), ("B", Bf, dB, (5, 2))):
        for _ in range(1):
            plus, minus = base.copy(), base.copy()
            plus[idx] += h
            minus[idx] -= h
            args = {"X": (Xf, Af, Bf), "A": (Xf, Af, Bf), "B": (Xf, Af, Bf)}[name]
            ap = [plus if n == name else a for n, a in zip("XAB", args)]
            am = [minus if n == name else a for n, a in zip("XAB", args)]
            fd = (loss(*ap) - loss(*am)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-9 * max(1.0, abs(fd)), (name, fd, grad[idx])
    # a dropped element of X gets no LoRA gradient: dX there is the base term only
    m, k = np.argwhere(~keep)[0]
    base_only = (olin._f64(dY) @ olin._f64(Wt))[m, k]
    assert abs(dX[m, k] - base_only) <= 1e-12


@pytest.mark.parametrize("p", [0.05, 0.3])
def test_inverted_dropout_keeps_the_branch_unbiased(p):
    """Inverted dropout is defined so that the scaled, dropped input has the
    expected value of the undropped one: E[s_eff X_d] = s X.  Measured through
    the oracle layer itself: X = 1, A = 1 (r = 1) and W = 0 give T[m] =
    s_eff * (number of kept elements of row m); over 2^22 Philox draws the
    mean of T / K must be s within 5 standard errors of the keep rate.  A
    scale of s (1 - p), s (1 + p), s / (1 + p) or plain s misses it by 0.25 %
    or more, far beyond the bound (about 0.06 % at p = 0.05)."""
    M, K, s = 1024, 4096, 0.25
    one = round_fp32_to_bf16_bits(np.ones((M, K), np.float32))
    A = round_fp32_to_bf16_bits(np.ones((1, K), np.float32))
    B = round_fp32_to_bf16_bits(np.zeros((8, 1), np.float32))
    Wt = np.zeros((8, K))
    keep = od.keep_mask(M, K, p, seed=4321)
    _, T = od.linear_fwd(one, Wt, A, B, s, p, keep)
    ratio = float(np.mean(T)) / K / s
    sigma = np.sqrt(p * (1 - p) / (M * K)) / (1 - p)
    assert abs(ratio - 1.0) <= 5 * sigma + 1e-6, (ratio, sigma)
    # the factor is the fp32 rounding of the exact quotient (within half an ulp)
    from fractions import Fraction
    se = od.effective_scale(s, p)
    exact = Fraction(float(np.float32(s))) / (1 - Fraction(float(p)))
    assert abs(Fraction(float(se)) - exact) <= Fraction(float(np.spacing(se))) / 2
