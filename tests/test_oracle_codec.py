"""Pins for the oracle's codec: quantize, mean tree, double quantization,
packing, decode and bf16 rounding.

Brute force here is written independently of the oracle's vectorised code:
per-element Python loops, exact rational distances, and library routines
(math.fsum, torch's bf16 cast) that the oracle does not use.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nearest_ties_low(x, levels):
    xf = Fraction(float(x))
    best, best_d = 0, None
    for i, l in enumerate(levels):
        d = abs(xf - Fraction(float(l)))
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def _brute_quantize(w):
    """Element-by-element restatement with exact-rational nearest levels."""
    flat = [np.float32(v) for v in np.asarray(w, np.float32).reshape(-1)]
    n = len(flat)
    lv = nf4.nf4_levels()
    nb = (n + 63) // 64
    absmax, codes = [], []
    for b in range(nb):
        blk = flat[64 * b: 64 * b + 64]
        c = max(abs(v) for v in blk)
        absmax.append(np.float32(c))
        for v in blk:
            if c == 0:
                codes.append(7)
            else:
                codes.append(_nearest_ties_low(np.float32(v) / np.float32(c), lv))
    total = math.fsum(float(c) for c in absmax)  # used only for a bound below
    return absmax, codes, total


def _tensor(n, seed, scale=0.02):
    g = np.random.default_rng(seed)
    return (g.standard_normal(n) * scale).astype(np.float32)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 200, 513])
def test_level1_codes_match_brute_force(n):
    w = _tensor(n, n)
    if n > 10:
        w[3] = 0.0
        w[5] = -0.0
    q = nf4.quantize(w)
    absmax, codes, _ = _brute_quantize(w)
    assert np.array_equal(q["absmax"], np.array(absmax, np.float32))
    assert q["codes"].tolist() == codes
    assert len(q["packed"]) == (n + 1) // 2


def test_level2_codes_match_brute_force():
    # 3 groups (2 full, 1 partial) of first-level constants.
    w = _tensor(64 * 600, 7)
    w[64 * 10: 64 * 11] = 0.0                   # one all-zero block
    q = nf4.quantize(w)
    c = q["absmax"]
    mean = q["mean"]
    t8 = nf4.t8_levels()
    for g in range(3):
        d = [np.float32(v - mean) for v in c[256 * g: 256 * g + 256]]
        c2 = max(abs(v) for v in d)
        assert q["c2"][g] == c2
        for j, v in enumerate(d):
            want = 127 if c2 == 0 else _nearest_ties_low(np.float32(v) / np.float32(c2), t8)
            assert q["code8"][256 * g + j] == want


def test_packing_order():
    codes = np.array([1, 2, 3], np.uint8)
    assert nf4.pack_nibbles(codes).tolist() == [0x21, 0x03]
    rng = np.random.default_rng(0)
    for n in (1, 2, 7, 64, 65):
        c = rng.integers(0, 16, n).astype(np.uint8)
        assert np.array_equal(nf4.unpack_nibbles(nf4.pack_nibbles(c), n), c)


def test_absmax_element_maps_to_an_end_code():
    w = _tensor(64 * 300 + 17, 3)
    q = nf4.quantize(w)
    codes = q["codes"]
    for b in range(len(q["absmax"])):
        blk = codes[64 * b: 64 * b + 64]
        assert (0 in blk) or (15 in blk)
    nb = len(q["code8"])
    for g in range(len(q["c2"])):
        grp = q["code8"][256 * g: min(nb, 256 * g + 256)]
        assert (0 in grp) or (255 in grp)


def test_all_zero_tensor():
    w = np.zeros(64 * 300, np.float32)
    w[::7] = -0.0
    q = nf4.quantize(w)
    assert np.all(q["codes"] == 7) and np.all(q["code8"] == 127)
    assert q["mean"] == 0.0 and np.all(q["c2"] == 0.0)
    wt = nf4.dequantize_q(q)
    assert np.all(wt == 0), "w_tilde is +0 bit for bit"


def test_constant_absmax_gives_zero_scale():
    # Every block has the same absmax: centred constants are all 0, c2 = 0.
    w = _tensor(64 * 256 * 2, 5)
    w = np.sign(w).astype(np.float32) * np.float32(0.03)
    q = nf4.quantize(w)
    assert np.all(q["c2"] == 0.0) and np.all(q["code8"] == 127)
    assert q["mean"] == np.float32(0.03)
    wt = bf16.bf16_bits_to_fp32(nf4.dequantize_q(q))
    assert np.array_equal(wt, bf16.bf16_bits_to_fp32(bf16.round_fp32_to_bf16_bits(w)))


def test_mean_tree_sum():
    rng = np.random.default_rng(11)
    for n in (1, 2, 3, 5, 64, 1000, 4097):
        v = rng.random(n) * 0.05
        tree = nf4.pairwise_tree_sum_fp64(v)
        exact = math.fsum(v)
        # pairwise summation error bound: ceil(log2 n) * eps * sum|v|
        bound = max(1, math.ceil(math.log2(n))) * 2.0 ** -53 * np.sum(np.abs(v)) * 1.01
        assert abs(tree - exact) <= bound
    # integers: exact in any order
    v = np.arange(1, 1001, dtype=np.float64)
    assert nf4.pairwise_tree_sum_fp64(v) == 500500.0
    # the tree pairs neighbours: with these values the sequential sum loses
    # the small terms but the pairwise tree keeps them.
    v = np.array([2.0 ** 53, 1.0, 1.0, 1.0])
    assert nf4.pairwise_tree_sum_fp64(v) == 2.0 ** 53 + 2.0   # (2^53+1) + (1+1)
    seq = 0.0
    for x in v:
        seq += x
    assert seq == 2.0 ** 53


def test_mean_definition():
    w = _tensor(64 * 1000 + 5, 9)
    q = nf4.quantize(w)
    nb = len(q["absmax"])
    assert q["mean"] == np.float32(nf4.pairwise_tree_sum_fp64(q["absmax"]) / nb)
    # within one fp32 ulp of the exactly rounded mean
    exact = math.fsum(q["absmax"].astype(np.float64)) / nb
    assert abs(float(q["mean"]) - exact) <= float(np.spacing(np.float32(exact)))


def test_decode_matches_elementwise_restatement():
    w = _tensor(64 * 700 + 33, 13)
    q = nf4.quantize(w)
    lv = nf4.nf4_levels()
    t8 = nf4.t8_levels()
    wt32 = nf4.dequantize_fp32(q["packed"], q["code8"], q["c2"], q["mean"], q["n"])
    rng = np.random.default_rng(1)
    for i in rng.integers(0, q["n"], 500):
        b = i // 64
        prod = np.float32(t8[q["code8"][b]]) * np.float32(q["c2"][b // 256])
        chat = np.float32(np.float32(prod) + np.float32(q["mean"]))
        want = np.float32(np.float32(lv[q["codes"][i]]) * chat)
        assert wt32[i] == want


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),   # subnormals
        np.float32([0.0, -0.0, 1.0, -1.0]),
    ])
    # exact ties in both parities
    u = rng.integers(0, 2 ** 31, 1000, dtype=np.uint64).astype(np.uint32) & np.uint32(0x7FFF0000)
    x = np.concatenate([x, (u | np.uint32(0x8000)).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.round_fp32_to_bf16_bits(x), ref)


def test_reconstruction_quality_sanity():
    # Not a parity criterion: NF4 on N(0, 0.02) blocks of 64 reconstructs to
    # ~9% relative Frobenius error and double quantization adds little
    # ("no measurable performance hit", automatone.win, How it works).
    w = _tensor(64 * 256 * 64, 21)
    q = nf4.quantize(w)
    wt = bf16.bf16_bits_to_fp64(nf4.dequantize_q(q))
    err = np.linalg.norm(wt - w) / np.linalg.norm(w)
    lv = nf4.nf4_levels().astype(np.float64)
    no_dq = lv[q["codes"]] * np.repeat(q["absmax"].astype(np.float64), 64)[: q["n"]]
    err0 = np.linalg.norm(no_dq - w) / np.linalg.norm(w)
    assert 0.05 < err0 < 0.13
    assert err < err0 * 1.01


def test_storage_sizes():
    assert nf4.nf4_sizes(1) == (1, 1, 1)
    assert nf4.nf4_sizes(64) == (32, 1, 1)
    assert nf4.nf4_sizes(65) == (33, 2, 1)
    assert nf4.nf4_sizes(64 * 256 + 1) == (8193, 257, 2)
    with pytest.raises(ValueError):
        nf4.nf4_sizes(0)
    with pytest.raises(ValueError):
        nf4.quantize(np.float32([1.0, np.nan]))


def test_golden_small_tensor():
    """Regression pin: a small tensor quantized by the oracle when it was
    pinned (tests/golden/make_golden.py writes it from oracle/ only)."""
    path = os.path.join(GOLDEN, "codec_small.npz")
    g = np.load(path)
    q = nf4.quantize(g["w"])
    assert np.array_equal(q["packed"], g["packed"])
    assert np.array_equal(q["code8"], g["code8"])
    assert np.array_equal(q["c2"], g["c2"])
    assert q["mean"] == g["mean"][0]
    assert np.array_equal(nf4.dequantize_q(q), g["wt"])


def test_decoded_constants_within_the_second_level_error_bound():
    """Nearest-level coding bounds the decode error: with d = fl32(c - mean)
    and k its 8-bit code, |d / c2 - T8[k]| is at most half the larger table gap
    next to k, so |c_hat - c| <= c2 * that half gap plus the four fp32
    roundings of d, d / c2, the product and the sum.  Checked for every block
    with exact rational arithmetic, on groups whose scales differ by up to 7x
    (a dropped mean, a sign slip or a group index taken modulo 256 breaks it
    by orders of magnitude)."""
    rng = np.random.default_rng(31)
    groups = 12
    sig = np.array([0.002, 0.05, 0.01, 0.12, 0.004, 0.03, 0.08, 0.002, 0.02, 0.06, 0.007, 0.1])
    w = (rng.standard_normal((groups, 256 * 64)) * sig[:, None]).astype(np.float32).reshape(-1)
    q = nf4.quantize(w)
    chat = nf4.decode_constants(q["code8"], q["c2"], q["mean"])
    t8 = nf4.t8_levels().astype(np.float64)
    gaps = np.diff(t8)
    half = np.zeros(256)
    half[0] = gaps[0] / 2
    half[255] = gaps[-1] / 2
    half[1:255] = np.maximum(gaps[:-1], gaps[1:]) / 2
    mean = float(q["mean"])
    for b in range(len(q["absmax"])):
        c = float(q["absmax"][b])
        c2 = float(q["c2"][b // 256])
        k = int(q["code8"][b])
        ulp = float(np.spacing(np.float32(max(abs(c), abs(mean), c2))))
        bound = Fraction(c2) * Fraction(half[k]) + 4 * Fraction(ulp)
        assert abs(Fraction(float(chat[b])) - Fraction(c)) <= bound, b
    # the scales really differ between groups
    assert q["c2"].max() > 4 * q["c2"].min()
