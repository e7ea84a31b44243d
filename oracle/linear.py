"""Forward and backward of the QLoRA linear layer in fp64 (test infrastructure only).

The layer keeps a frozen base weight W in NF4 and adds a trainable low-rank
pair A [r, K], B [N, r] (automatone.win, "QLoRA paper explained", The problem:
LoRA "trains a pair of small low-rank matrices per layer"; creativeworksof
knowledge.com, "QLoRA: Fine-Tune 70B on One GPU", Code: ``r``, ``lora_alpha``,
``bias="none"``).  The base weight is used as its dequantized bf16 copy
w_tilde (automatone.win, How it works: dequantize to BFloat16 on the fly and
run the math).  Gradients flow through the frozen base into X and into the
adapters only, never into W (automatone.win, How it works; aiwiki.com.my,
"QLoRA", Key Concepts and Technology).

Reading taken for the LoRA branch: scale s = alpha / r applied to the
up-projection, no bias, no dropout:

    T  = X A^T                      [M, r]
    Y  = X w_tilde^T + s T B^T      [M, N]
    G  = dY B                       [M, r]
    dX = dY w_tilde + s G A         [M, K]
    dA = s G^T X                    [r, K]
    dB = s dY^T T                   [N, r]

Every product is the plain mathematical one, evaluated in fp64 from the exact
values of the bf16 inputs with no intermediate rounding.  Inputs are uint16
arrays of bf16 bit patterns; ``scale`` is the fp32 value the caller passes.
"""

import numpy as np

from .bf16 import bf16_bits_to_fp64


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_fp64(a)
    return a.astype(np.float64)


def lora_down(X, A):
    """T = X A^T in fp64."""
    return _f64(X) @ _f64(A).T


def lora_grad_in(dY, B):
    """G = dY B in fp64 (the adapter-side gradient before the scale)."""
    return _f64(dY) @ _f64(B)


def linear_fwd(X, Wt, A, B, scale):
    """Returns (Y, T) in fp64."""
    X, Wt, A, B = _f64(X), _f64(Wt), _f64(A), _f64(B)
    s = float(np.float32(scale))
    T = X @ A.T
    Y = X @ Wt.T + s * (T @ B.T)
    return Y, T


def linear_bwd(dY, X, Wt, A, B, scale):
    """Returns (dX, dA, dB) in fp64."""
    dY, X, Wt, A, B = _f64(dY), _f64(X), _f64(Wt), _f64(A), _f64(B)
    s = float(np.float32(scale))
    T = X @ A.T
    G = lora_grad_in(dY, B)
    dX = dY @ Wt + s * (G @ A)
    dA = s * (G.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB


# ---- sampled forms for full-size checks: same definitions, fewer outputs ----

def linear_fwd_rows(X, Wt, A, B, scale, rows):
    """Rows ``rows`` of Y, computed only from those rows of X."""
    Xr = _f64(np.asarray(X)[rows])
    Wt, A, B = _f64(Wt), _f64(A), _f64(B)
    s = float(np.float32(scale))
    return Xr @ Wt.T + s * ((Xr @ A.T) @ B.T)


def linear_dx_rows(dY, Wt, A, B, scale, rows):
    """Rows ``rows`` of dX, computed only from those rows of dY."""
    dYr = _f64(np.asarray(dY)[rows])
    Wt, A, B = _f64(Wt), _f64(A), _f64(B)
    s = float(np.float32(scale))
    return dYr @ Wt + s * ((dYr @ B) @ A)


def linear_dA_cols(dY, X, B, scale, cols):
    """Columns ``cols`` of dA = s (dY B)^T X."""
    G = _f64(dY) @ _f64(B)
    s = float(np.float32(scale))
    return s * (G.T @ _f64(np.asarray(X)[:, cols]))


def linear_dB_rows(dY, X, A, scale, rows):
    """Rows ``rows`` of dB = s dY^T (X A^T)."""
    T = _f64(X) @ _f64(A).T
    s = float(np.float32(scale))
    return s * (_f64(np.asarray(dY)[:, rows]).T @ T)
