"""Pins for the oracle's linear layer: brute-force loops, finite differences,
adjoint identities and layout special cases."""

import numpy as np
import pytest

from oracle import bf16, linear


def _bf16(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    return bf16.round_fp32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _loops_fwd(X, Wt, A, B, s):
    M, K = len(X), len(X[0])
    N, r = len(B), len(B[0])
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        T = [sum(X[m][k] * A[j][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            base = sum(X[m][k] * Wt[n][k] for k in range(K))
            lora = sum(T[j] * B[n][j] for j in range(r))
            Y[m][n] = base + s * lora
    return np.array(Y)


def _loops_bwd(dY, X, Wt, A, B, s):
    M, K = len(X), len(X[0])
    N, r = len(B), len(B[0])
    G = [[sum(dY[m][n] * B[n][j] for n in range(N)) for j in range(r)] for m in range(M)]
    T = [[sum(X[m][k] * A[j][k] for k in range(K)) for j in range(r)] for m in range(M)]
    dX = [[sum(dY[m][n] * Wt[n][k] for n in range(N)) + s * sum(G[m][j] * A[j][k] for j in range(r))
           for k in range(K)] for m in range(M)]
    dA = [[s * sum(G[m][j] * X[m][k] for m in range(M)) for k in range(K)] for j in range(r)]
    dB = [[s * sum(dY[m][n] * T[m][j] for m in range(M)) for j in range(r)] for n in range(N)]
    return np.array(dX), np.array(dA), np.array(dB)


@pytest.mark.parametrize("M,N,K,r", [(3, 5, 7, 2), (4, 6, 9, 3), (1, 2, 64, 1)])
def test_brute_force_loops(M, N, K, r):
    X, Wt, A, B, dY = (_bf16((M, K), 1), _bf16((N, K), 2, 0.02), _bf16((r, K), 3, 0.1),
                       _bf16((N, r), 4, 0.1), _bf16((M, N), 5))
    s = 0.75
    f = bf16.bf16_bits_to_fp64
    Y, T = linear.linear_fwd(X, Wt, A, B, s)
    assert np.allclose(Y, _loops_fwd(f(X).tolist(), f(Wt).tolist(), f(A).tolist(), f(B).tolist(), s),
                       rtol=1e-12, atol=1e-14)
    dX, dA, dB = linear.linear_bwd(dY, X, Wt, A, B, s)
    rX, rA, rB = _loops_bwd(f(dY).tolist(), f(X).tolist(), f(Wt).tolist(), f(A).tolist(),
                            f(B).tolist(), s)
    for got, want in ((dX, rX), (dA, rA), (dB, rB)):
        assert got.shape == want.shape
        assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def test_finite_differences_16x16_layer():
    # L(X, A, B) = <dY, Y>; Y is linear in X, in A (B fixed) and in B (A fixed),
    # so central differences are exact up to fp64 rounding.
    rng = np.random.default_rng(7)
    M, N, K, r = 4, 16, 16, 4
    X = rng.standard_normal((M, K))
    Wt = rng.standard_normal((N, K)) * 0.02
    A = rng.standard_normal((r, K)) * 0.1
    B = rng.standard_normal((N, r)) * 0.1
    dY = rng.standard_normal((M, N))
    s = 2.0
    h = 2.0 ** -10

    def L(X_, A_, B_):
        return float(np.sum(dY * linear.linear_fwd(X_, Wt, A_, B_, s)[0]))

    dX, dA, dB = linear.linear_bwd(dY, X, Wt, A, B, s)
    for name, P, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        num = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args_p = {"X": (Pp, A, B), "A": (X, Pp, B), "B": (X, A, Pp)}[name]
            args_m = {"X": (Pm, A, B), "A": (X, Pm, B), "B": (X, A, Pm)}[name]
            num[idx] = (L(*args_p) - L(*args_m)) / (2 * h)
        assert np.allclose(num, grad, rtol=1e-9, atol=1e-9), name


def test_adjoint_identities():
    rng = np.random.default_rng(8)
    M, N, K, r = 32, 48, 64, 8
    X = rng.standard_normal((M, K))
    Wt = rng.standard_normal((N, K)) * 0.02
    A = rng.standard_normal((r, K)) * 0.01
    B = rng.standard_normal((N, r)) * 0.01
    dY = rng.standard_normal((M, N))
    s = 0.25
    Y, _ = linear.linear_fwd(X, Wt, A, B, s)
    dX, dA, dB = linear.linear_bwd(dY, X, Wt, A, B, s)
    lora = Y - X @ Wt.T
    assert np.isclose(np.sum(dY * Y), np.sum(dX * X), rtol=1e-12)
    assert np.isclose(np.sum(dY * lora), np.sum(dA * A), rtol=1e-10)
    assert np.isclose(np.sum(dY * lora), np.sum(dB * B), rtol=1e-10)


def test_identity_input_exposes_layout():
    # X = I_K: Y = w_tilde^T + s A^T B^T, which fixes which index is which.
    rng = np.random.default_rng(9)
    N, K, r = 6, 5, 2
    Wt = rng.standard_normal((N, K))
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    Y, T = linear.linear_fwd(np.eye(K), Wt, A, B, 0.5)
    assert np.allclose(Y, Wt.T + 0.5 * A.T @ B.T)
    assert np.allclose(T, A.T)


def test_sampled_forms_agree_with_full():
    rng = np.random.default_rng(10)
    M, N, K, r = 20, 12, 64, 4
    X, Wt, A, B, dY = (_bf16((M, K), 11), _bf16((N, K), 12, 0.02), _bf16((r, K), 13, 0.01),
                       _bf16((N, r), 14, 0.01), _bf16((M, N), 15))
    s = 2.0
    Y, _ = linear.linear_fwd(X, Wt, A, B, s)
    dX, dA, dB = linear.linear_bwd(dY, X, Wt, A, B, s)
    rows = np.array([0, 7, 19])
    assert np.allclose(linear.linear_fwd_rows(X, Wt, A, B, s, rows), Y[rows], rtol=1e-13)
    assert np.allclose(linear.linear_dx_rows(dY, Wt, A, B, s, rows), dX[rows], rtol=1e-13)
    cols = np.array([1, 63])
    assert np.allclose(linear.linear_dA_cols(dY, X, B, s, cols), dA[:, cols], rtol=1e-13)
    nrows = np.array([0, 11])
    assert np.allclose(linear.linear_dB_rows(dY, X, A, s, nrows), dB[nrows], rtol=1e-13)
