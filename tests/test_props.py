"""Property tests of the oracle's quantizer (hypothesis, CPU): invariants the
blockwise absmax code must keep for any finite input (creativeworksofknowledge.com,
"QLoRA: Fine-Tune 70B on One GPU", The three innovations / 1. NF4 and
2. Double quantization)."""

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st
from hypothesis.extra import numpy as hnp

from oracle import nf4

finite32 = st.floats(min_value=-2.0 ** 100, max_value=2.0 ** 100, allow_nan=False, allow_infinity=False, width=32)
blocks = hnp.arrays(np.float32, st.integers(1, 6).map(lambda n: (n, 64)), elements=finite32)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(blocks)
def test_codes_monotone_in_x_within_a_block(w):
    # The first-level code is a non-decreasing function of the weight inside
    # one block (one constant divides every weight of the block).
    codes = nf4.quantize(w)["codes"].reshape(w.shape)
    for b in range(w.shape[0]):
        order = np.argsort(w[b], kind="stable")
        assert np.all(np.diff(codes[b][order].astype(np.int16)) >= 0)


@settings(max_examples=200, deadline=None, derandomize=True)
@given(blocks)
def test_absmax_element_takes_an_end_code(w):
    # The element of largest magnitude divides to exactly +1 or -1, the two
    # end levels: every block with a nonzero constant holds code 0 or 15;
    # an all-zero block is all the zero code.
    ref = nf4.quantize(w)
    codes = ref["codes"].reshape(w.shape)
    for b in range(w.shape[0]):
        if ref["absmax"][b] > 0:
            assert (codes[b] == 0).any() or (codes[b] == 15).any()
        else:
            assert (codes[b] == nf4.q4_zero_code("nf4")).all()


@settings(max_examples=100, deadline=None, derandomize=True)
@given(blocks, st.integers(-20, 20))
def test_codes_invariant_under_power_of_two_scaling(w, e):
    # Scaling a whole tensor by 2^e (staying in the normal range) scales each
    # block constant by 2^e and leaves every quotient, hence every code,
    # unchanged.
    amax = float(np.max(np.abs(w)))
    tiny = float(np.min(np.abs(w[w != 0]))) if np.any(w != 0) else 1.0
    if amax * 2.0 ** e > 1e37 or tiny * 2.0 ** e < 1e-37 or tiny < 1e-37:
        return
    scaled = (w * np.float32(2.0 ** e)).astype(np.float32)
    assert np.array_equal(nf4.quantize(w)["codes"], nf4.quantize(scaled)["codes"])


@settings(max_examples=100, deadline=None, derandomize=True)
@given(hnp.arrays(np.float32, st.integers(1, 700), elements=finite32))
def test_constant_codes_bound_the_centred_constants(w):
    # Second level: the decoded constant code times the group scale stays
    # within half the widest gap of the 8-bit table from the centred
    # constant, and a group whose centred constants are all zero has scale 0.
    ref = nf4.quantize(w)
    t8 = nf4.t8_levels().astype(np.float64)
    half_gap = float(np.max(np.diff(t8))) / 2
    centred = ref["absmax"].astype(np.float64) - np.float64(ref["mean"])
    for b in range(len(ref["code8"])):
        c2 = float(ref["c2"][b // 256])
        err = abs(t8[ref["code8"][b]] * c2 - np.float64(np.float32(centred[b])))
        assert err <= half_gap * c2 * (1 + 1e-6) + 1e-30
