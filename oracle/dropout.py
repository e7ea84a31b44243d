"""LoRA dropout on the adapter input, plain NumPy (test infrastructure only).

The pages' adapter configuration drops the LoRA branch's input with
probability 0.05 (creativeworksofknowledge.com, "QLoRA: Fine-Tune 70B on One
GPU", Code: ``lora_dropout=0.05``).  The pages give no mask generator or
scaling; readings taken:

* Mask.  Counter-based, so that the forward and backward passes (and any
  implementation) reproduce it from a seed: Philox4x32-10 (Salmon, Moraes,
  Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).
  Element e = m * K + k of X [M, K] uses word e % 4 of
  Philox4x32-10(counter = (e // 4) as a 64-bit value in words 0 (low) and 1
  (high), words 2 and 3 zero; key = (seed low 32 bits, seed high 32 bits)).
  It is kept iff that word >= t with t = floor(p * 2^32) (p as given, in
  fp64), so p = 0 keeps everything.

* Scaling.  Inverted dropout: kept elements are scaled by 1 / (1 - p).  The
  factor is folded into the LoRA scale once, s_eff = fl32(s / (1 - p)) (fp64
  quotient rounded to fp32), and the dropped input X_d = X * keep is exact in
  bf16 (elements are kept or zeroed).

* The layer (dropout on the branch input only; the base path sees X):
      T  = s_eff X_d A^T                Y  = X w_tilde^T + T B^T
      G  = s_eff dY B                   dX = dY w_tilde + (G A) * keep
      dA = G^T X_d                      dB = dY^T T
  all products in fp64 from the exact bf16 input values.

* Storage of the mask: bit (k % 32) of uint32 word [m][k // 32].
"""

import numpy as np

from .linear import _f64

PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key increments (Weyl sequence)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counters, key):
    """Philox4x32-10 of each row of counters (uint32 [n, 4]) under key (k0, k1)."""
    c = [np.asarray(counters, dtype=np.uint64)[:, i].copy() for i in range(4)]
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W[0])) & MASK32
            k1 = (k1 + np.uint64(PHILOX_W[1])) & MASK32
        p0 = c[0] * m0          # < 2^64: exact in uint64
        p1 = c[2] * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack(c, axis=1).astype(np.uint32)


def threshold(p):
    """Keep threshold t = floor(p * 2^32) for 0 <= p < 1."""
    p = float(p)
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p * 4294967296.0))


def effective_scale(scale, p):
    """s_eff = fl32(s / (1 - p)), quotient in fp64."""
    return np.float32(float(np.float32(scale)) / (1.0 - float(p)))


def _keep_range(e0, n, p, seed):
    """Keep flags of the n consecutive elements e0 .. e0 + n - 1: Philox is
    evaluated once per counter block b = e // 4 that the range touches, and
    element e takes word e % 4 of its block (4 b + w is word w of block b)."""
    e0, n = int(e0), int(n)
    b0, b1 = e0 // 4, (e0 + n - 1) // 4 + 1
    blocks = np.arange(b0, b1, dtype=np.uint64)
    ctr = np.zeros((len(blocks), 4), np.uint32)
    ctr[:, 0] = (blocks & MASK32).astype(np.uint32)
    ctr[:, 1] = (blocks >> np.uint64(32)).astype(np.uint32)
    seed = int(seed)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(-1)
    w = words[e0 - 4 * b0: e0 - 4 * b0 + n]
    return w.astype(np.uint64) >= np.uint64(threshold(p))


def keep_mask(M, K, p, seed):
    """bool [M, K]: which elements of the LoRA input survive."""
    return _keep_range(0, M * K, p, seed).reshape(M, K)


def keep_mask_rows(rows, K, p, seed):
    """The rows `rows` of keep_mask(M, K, p, seed), for any M > max(rows)."""
    rows = [int(r) for r in np.asarray(rows).reshape(-1)]
    return np.stack([_keep_range(r * K, K, p, seed) for r in rows]).reshape(len(rows), K)


def pack_bits(keep):
    """bool [M, K] -> uint32 [M, ceil(K / 32)], bit k % 32 of word k // 32."""
    keep = np.asarray(keep, dtype=bool)
    M, K = keep.shape
    words = (K + 31) // 32
    padded = np.zeros((M, words * 32), dtype=np.uint64)
    padded[:, :K] = keep
    shifts = np.arange(32, dtype=np.uint64)
    return (padded.reshape(M, words, 32) << shifts).sum(axis=2).astype(np.uint32)


def unpack_bits(bits, K):
    bits = np.asarray(bits, dtype=np.uint32)
    shifts = np.arange(32, dtype=np.uint32)
    return ((bits[:, :, None] >> shifts) & 1).reshape(bits.shape[0], -1)[:, :K].astype(bool)


def drop(X, keep):
    """X_d as bf16 bit patterns: X where kept, +0 elsewhere."""
    return np.where(keep, np.asarray(X, dtype=np.uint16), np.uint16(0)).astype(np.uint16)


def linear_fwd(X, Wt, A, B, scale, p, keep):
    """(Y, T) of the layer with dropout on the LoRA input; T includes s_eff."""
    se = float(effective_scale(scale, p))
    Xd = _f64(X) * keep
    T = se * (Xd @ _f64(A).T)
    Y = _f64(X) @ _f64(Wt).T + T @ _f64(B).T
    return Y, T


def linear_bwd(dY, X, Wt, A, B, scale, p, keep):
    """(dX, dA, dB, G) of the layer with dropout on the LoRA input."""
    se = float(effective_scale(scale, p))
    Xd = _f64(X) * keep
    G = se * (_f64(dY) @ _f64(B))
    dX = _f64(dY) @ _f64(Wt) + (G @ _f64(A)) * keep
    dA = G.T @ Xd
    dB = _f64(dY).T @ (se * (Xd @ _f64(A).T))
    return dX, dA, dB, G
