"""NF4 + double-quantization codec, plain NumPy (test infrastructure only).

What the pages fix, and the readings taken where they are silent:

* NF4 levels.  NF4 "sets its levels at the quantiles of a standard normal
  distribution" and is optimal "for zero-centered normally distributed
  weights" (automatone.win, "QLoRA paper explained", How it works / 4-bit
  NormalFloat; creativeworksofknowledge.com, "QLoRA: Fine-Tune 70B on One
  GPU", The three innovations / 1. NF4).  Reading: 16 levels with an exact
  zero, 8 positive quantiles and 7 negative ones, normalised to [-1, 1].  The
  outermost probability is 1 - delta with delta = (1/30 + 1/32) / 2 (the mean
  of the half-bin offsets for 15 and 16 equal-probability bins), because the
  quantile at probability 1 is infinite.  Levels are built in fp64 and rounded
  once to fp32.

* Blockwise absmax.  "Block-wise quantization produces a scaling constant per
  block" (automatone.win, How it works / Double Quantization).  Reading: blocks
  of 64 consecutive elements of the row-major flattened tensor, constant =
  max |w| over the block; the last block may be partial.

* Code rule.  Reading: x = fl32(w / c) (IEEE fp32 division); code = index of
  the nearest level, ties to the lower index.  Implemented as the number of
  fp32 thresholds strictly below x, where threshold i is the exact midpoint of
  levels i and i+1 rounded toward minus infinity to fp32 (this reproduces
  real-arithmetic nearest-with-ties-low for every fp32 x).  A block whose
  constant is 0 gets code 7 (the exact zero level) everywhere.

* Packing.  Reading: byte j holds element 2j in its low nibble and element
  2j+1 in its high nibble; for an odd element count the last high nibble is 0.

* Double quantization.  The constants "are themselves quantized (FP32 ->
  FP8)" (creativeworksofknowledge.com, The three innovations / 2. Double
  quantization), "saving about 0.37 bits per parameter" (automatone.win, How
  it works / Double Quantization).  Reading: one fp32 mean per tensor is
  subtracted (fp64 pairwise-tree sum in a fixed order, divided by the block
  count, rounded to fp32); the centred constants are grouped by 256, each group
  keeps c2 = max |c - mean| in fp32 and an 8-bit code into the table T8 below,
  with the same nearest/ties-low rule.  A group with c2 = 0 gets code 127.

* T8.  Reading: an E4M3-shaped 8-bit code (4 exponent bits with bias 7, 3
  mantissa bits, subnormals at exponent 0, no infinities or NaNs, so the
  largest magnitude is 480), as an ascending signed table
  [-m127 .. -m0, +m0 .. +m127] with every entry fl32(+-m / 480).

* Decode.  c_hat = fl32(fl32(T8[code8] * c2) + mean), two separate fp32
  roundings (no fused multiply-add); w_tilde = bf16_rne(fl32(NF4[q] * c_hat)).

* The other 4-bit data types.  The pages compare NF4 with plain 4-bit
  integers, whose 16 levels are evenly spaced, and 4-bit floats, whose levels
  follow the exponent (automatone.win, "QLoRA paper explained", How it works /
  4-bit NormalFloat; Results table, FP4 vs NF4).  Everything except the level
  table is shared (blocks, code rule, packing, double quantization, decode).
  Readings:
    fp4   the 4-bit float E2M1 (1 sign bit, 2 exponent bits with bias 1,
          1 mantissa bit, subnormals at exponent 0; magnitudes 0, 0.5, 1, 1.5,
          2, 3, 4, 6), divided by its largest magnitude 6 in fp32 so that the
          block's absmax maps to 6.  Ascending table [-v7 .. -v1, 0, 0, v1 ..
          v7]: the two zeros are codes 7 and 8; code 8 is never produced.
    int4  symmetric absmax integers: level k = fl32(k / 7) for the 16
          two's-complement values k = -8 .. 7, so that the absmax maps to 7;
          code 0 (-8/7) lies outside [-1, 1] and is never produced.
  A block whose constant is 0 gets the code of the zero level (7, 7, 8).
"""

import math
from statistics import NormalDist

import numpy as np

from .bf16 import round_fp32_to_bf16_bits

BLOCK = 64          # elements per first-level absmax block
GROUP = 256         # first-level constants per second-level group
ZERO_CODE = 7       # NF4 code of the exact zero level
QTYPES = ("nf4", "fp4", "int4")   # 4-bit data types; the index is the stored type id
ZERO_CODE8 = 127    # T8 code of -0 (where exact zero maps, ties to low)


# --------------------------------------------------------------------------
# Tables
# --------------------------------------------------------------------------

def nf4_levels_fp64():
    """The 16 NF4 levels in fp64 before the final fp32 rounding."""
    nd = NormalDist(0.0, 1.0)
    delta = 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    p_top = 1.0 - delta
    # 8 positive quantiles: 9 equally spaced probabilities from p_top down to
    # 1/2, the last (probability 1/2, quantile 0) dropped.
    pos = [nd.inv_cdf(float(p)) for p in np.linspace(p_top, 0.5, 9)[:8]]
    # 7 negative quantiles, mirrored: 8 points from p_top down to 1/2, last dropped.
    neg = [-nd.inv_cdf(float(p)) for p in np.linspace(p_top, 0.5, 8)[:7]]
    v = np.sort(np.array(pos + neg + [0.0], dtype=np.float64))
    return v / np.max(np.abs(v))


def nf4_levels():
    """16 NF4 levels as fp32, ascending; code 7 is the exact zero."""
    return nf4_levels_fp64().astype(np.float32)


def _round_down_fp32(m):
    """Round fp64 values toward minus infinity to fp32."""
    m = np.asarray(m, dtype=np.float64)
    f = m.astype(np.float32)
    too_big = f.astype(np.float64) > m
    f[too_big] = np.nextafter(f[too_big], np.float32(-np.inf))
    return f


def midpoint_thresholds(levels_fp32):
    """Decision thresholds of nearest-level rounding with ties to the lower index.

    code(x) = number of thresholds strictly below x.  Threshold i is the exact
    fp64 midpoint of levels i and i+1 rounded toward minus infinity to fp32.
    Where two neighbouring levels are equal in value (T8's -0 and +0) the
    upper one is never the lower-index nearest, so threshold i takes the value
    of threshold i+1 and code i+1 is skipped.
    """
    lv = np.asarray(levels_fp32, dtype=np.float32).astype(np.float64)
    mid = (lv[:-1] + lv[1:]) / 2.0   # exact: sum of two fp32 fits in fp64, /2 exact
    tau = _round_down_fp32(mid)
    for i in range(len(tau) - 2, -1, -1):
        if lv[i] == lv[i + 1]:
            tau[i] = tau[i + 1]
    return tau


def nf4_thresholds():
    return midpoint_thresholds(nf4_levels())


def fp4_magnitudes():
    """The 8 non-negative E2M1 values by code 2 e + m: exponent field e (bias
    1, subnormal at e = 0), mantissa bit m."""
    out = []
    for e in range(4):
        for m in range(2):
            out.append(m / 2.0 if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1))
    return np.array(out, dtype=np.float64)


def fp4_levels():
    """16 ascending FP4 levels (E2M1 / 6 in fp32); codes 7 and 8 are both zero."""
    v = fp4_magnitudes().astype(np.float32) / np.float32(6.0)   # IEEE fp32 division
    pos = v[1:]
    return np.concatenate([-pos[::-1], np.zeros(2, np.float32), pos]).astype(np.float32)


def int4_levels():
    """16 ascending Int4 levels fl32(k / 7), k = -8 .. 7; code 8 is zero."""
    k = np.arange(-8, 8).astype(np.float32)
    return (k / np.float32(7.0)).astype(np.float32)


def q4_levels(qtype="nf4"):
    """Level table of a 4-bit data type ("nf4", "fp4" or "int4")."""
    if qtype == "nf4":
        return nf4_levels()
    if qtype == "fp4":
        return fp4_levels()
    if qtype == "int4":
        return int4_levels()
    raise ValueError("unknown 4-bit type %r" % (qtype,))


def q4_zero_code(qtype="nf4"):
    """Code written for every element of a block whose constant is 0."""
    return {"nf4": ZERO_CODE, "fp4": 7, "int4": 8}[qtype]


def t8_magnitudes():
    """The 128 non-negative magnitudes of the E4M3-shaped code, index k = 8*e + f."""
    out = []
    for e in range(16):
        for f in range(8):
            if e == 0:
                out.append(math.ldexp(f / 8.0, -6))
            else:
                out.append(math.ldexp(1.0 + f / 8.0, e - 7))
    return np.array(out, dtype=np.float64)


def t8_levels():
    """256-entry ascending signed 8-bit constant table, fp32, range [-1, 1]."""
    m = t8_magnitudes().astype(np.float32)          # exactly representable
    pos = m / np.float32(480.0)                     # IEEE fp32 division
    neg = -pos[::-1]
    return np.concatenate([neg, pos]).astype(np.float32)


def t8_thresholds():
    return midpoint_thresholds(t8_levels())


# --------------------------------------------------------------------------
# Helpers
# --------------------------------------------------------------------------

def nf4_sizes(n):
    """(packed bytes, first-level blocks, second-level groups) for n elements."""
    if n < 1:
        raise ValueError("n must be >= 1")
    nb = (n + BLOCK - 1) // BLOCK
    return (n + 1) // 2, nb, (nb + GROUP - 1) // GROUP


def pack_nibbles(q):
    """codes uint8[n] -> uint8[ceil(n/2)]: element 2j low nibble, 2j+1 high nibble."""
    q = np.asarray(q, dtype=np.uint8)
    if len(q) % 2:
        q = np.concatenate([q, np.zeros(1, np.uint8)])
    return (q[0::2] | (q[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed, n):
    packed = np.asarray(packed, dtype=np.uint8)
    q = np.empty(2 * len(packed), np.uint8)
    q[0::2] = packed & np.uint8(0x0F)
    q[1::2] = packed >> np.uint8(4)
    return q[:n]


def nearest_code(x, thresholds):
    """Number of thresholds strictly below x (nearest level, ties to the lower index)."""
    return np.searchsorted(thresholds, np.asarray(x, np.float32), side="left").astype(np.uint8)


def pairwise_tree_sum_fp64(values):
    """fp64 sum in a fixed pairwise order: zero-pad to a power of two, then
    repeatedly add neighbours (a[0::2] + a[1::2]) until one value remains."""
    a = np.asarray(values, dtype=np.float64)
    n = len(a)
    p = 1
    while p < n:
        p *= 2
    a = np.concatenate([a, np.zeros(p - n)])
    while len(a) > 1:
        a = a[0::2] + a[1::2]
    return float(a[0])


def _block_view(flat, block, fill):
    n = len(flat)
    nb = (n + block - 1) // block
    padded = np.full(nb * block, fill, dtype=flat.dtype)
    padded[:n] = flat
    return padded.reshape(nb, block)


# --------------------------------------------------------------------------
# Quantize / dequantize
# --------------------------------------------------------------------------

def quantize(w, qtype="nf4"):
    """Quantize a fp32 tensor (any shape, flattened row-major) to NF4 + DQ
    (or to the FP4 / Int4 level table, same format otherwise).

    Returns a dict with
      packed  uint8[ceil(n/2)]   NF4 codes, two per byte
      code8   uint8[nb]          8-bit codes of the block constants
      c2      float32[nb2]       per-256-group scale of the centred constants
      mean    float32            per-tensor mean of the block constants
      absmax  float32[nb]        the first-level constants (input to the second
                                 level; not part of the stored format)
      codes   uint8[n]           unpacked NF4 codes (convenience)
      n       int
      qtype   str                "nf4", "fp4" or "int4"
    """
    flat = np.ascontiguousarray(np.asarray(w, dtype=np.float32)).reshape(-1)
    n = len(flat)
    if n < 1:
        raise ValueError("quantize: empty tensor")
    if not np.all(np.isfinite(flat)):
        raise ValueError("quantize: non-finite input")
    _, nb, nb2 = nf4_sizes(n)

    # Level 1: per-block absmax, normalise, nearest NF4 level.
    blocks = _block_view(flat, BLOCK, np.float32(0.0))
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)          # fp32 IEEE division
    codes = nearest_code(x, midpoint_thresholds(q4_levels(qtype)))
    codes[absmax == 0, :] = q4_zero_code(qtype)
    codes = codes.reshape(-1)[:n]
    packed = pack_nibbles(codes)

    # Level 2: mean, centre, per-group scale, nearest T8 code.
    mean = np.float32(pairwise_tree_sum_fp64(absmax) / nb)
    centred = (absmax - mean).astype(np.float32)
    groups = _block_view(centred, GROUP, np.float32(0.0))
    c2 = np.max(np.abs(groups), axis=1).astype(np.float32)
    safe2 = np.where(c2 > 0, c2, np.float32(1.0)).astype(np.float32)
    x2 = (groups / safe2[:, None]).astype(np.float32)
    code8 = nearest_code(x2, t8_thresholds())
    code8[c2 == 0, :] = ZERO_CODE8
    code8 = code8.reshape(-1)[:nb]

    return dict(packed=packed, code8=code8, c2=c2, mean=mean, absmax=absmax,
                codes=codes, n=n, qtype=qtype)


def decode_constants(code8, c2, mean):
    """c_hat[b] = fl32(fl32(T8[code8[b]] * c2[b // 256]) + mean), no FMA."""
    code8 = np.asarray(code8, dtype=np.uint8)
    t8 = t8_levels()
    scale = np.asarray(c2, dtype=np.float32)[np.arange(len(code8)) // GROUP]
    prod = (t8[code8] * scale).astype(np.float32)
    return (prod + np.float32(mean)).astype(np.float32)


def dequantize_fp32(packed, code8, c2, mean, n, qtype="nf4"):
    """fl32(NF4[q] * c_hat) for every element, before the bf16 rounding."""
    q = unpack_nibbles(packed, n)
    c_hat = decode_constants(code8, c2, mean)
    lv = q4_levels(qtype)
    return (lv[q] * c_hat[np.arange(n) // BLOCK]).astype(np.float32)


def dequantize(packed, code8, c2, mean, n, qtype="nf4"):
    """Dequantized weights as uint16 bf16 bit patterns, shape [n]."""
    return round_fp32_to_bf16_bits(dequantize_fp32(packed, code8, c2, mean, n, qtype))


def dequantize_q(qd):
    """dequantize() applied to the dict returned by quantize()."""
    return dequantize(qd["packed"], qd["code8"], qd["c2"], qd["mean"], qd["n"], qd.get("qtype", "nf4"))


def storage_bits_per_param(n):
    """Stored bits per parameter: 4-bit codes + 8-bit constant codes + fp32 c2 + fp32 mean."""
    packed, nb, nb2 = nf4_sizes(n)
    return (8.0 * packed + 8.0 * nb + 32.0 * nb2 + 32.0) / n
