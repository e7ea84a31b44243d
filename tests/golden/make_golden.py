"""Writes tests/golden/codec_small.npz from the oracle only.

The tensor mixes Gaussian blocks, an all-zero block, a block of equal
magnitudes, exact level multiples and a partial tail block (n = 64*300 + 37),
so the stored codes exercise every branch of the codec.
Run:  python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import nf4  # noqa: E402


def make_tensor():
    rng = np.random.Generator(np.random.PCG64(20230523))
    n = 64 * 300 + 37
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w[64 * 5: 64 * 6] = 0.0
    w[64 * 7: 64 * 8] = np.float32(0.011) * np.sign(w[64 * 7: 64 * 8])
    lv = nf4.nf4_levels()
    w[64 * 9: 64 * 9 + 16] = lv * np.float32(0.05)
    w[64 * 11 + 3] = np.float32(-0.5)     # one large outlier block
    return w


def main():
    w = make_tensor()
    q = nf4.quantize(w)
    out = os.path.join(HERE, "codec_small.npz")
    np.savez(out, w=w, packed=q["packed"], code8=q["code8"], c2=q["c2"],
             mean=np.float32([q["mean"]]), wt=nf4.dequantize_q(q))
    print("wrote", out)


if __name__ == "__main__":
    main()
