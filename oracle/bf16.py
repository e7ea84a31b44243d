"""bf16 helpers for the oracle (test infrastructure only).

The pages fix bf16 as the compute type: "dequantize each layer's weights back
to a compute dtype (BFloat16) on the fly" (automatone.win, "QLoRA paper
explained", How it works) and "one storage data type (usually NF4) and one
computation data type (16-bit BrainFloat)" (aiwiki.com.my, "QLoRA", Key
Concepts and Technology).  The rounding mode is not stated; the reading taken
is IEEE round-to-nearest-even on the fp32 bit pattern, with subnormals kept.
"""

import numpy as np


def round_fp32_to_bf16_bits(x):
    """fp32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    The upper 16 bits of the fp32 pattern are kept; the lower 16 bits decide
    the rounding: above half -> up, below -> down, exactly half -> towards the
    even upper half.  Non-finite inputs are outside the contract.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == np.uint64(1)))
    out = upper + round_up.astype(np.uint64)
    return out.astype(np.uint16)


def bf16_bits_to_fp64(b):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_bits_to_fp32(b):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
