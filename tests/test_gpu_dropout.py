"""GPU parity of LoRA dropout with the oracle: the keep mask and the dropped
input bit for bit (the mask is a counter-based Philox4x32-10 stream, so both
sides draw the same bits from the seed), and the layer's forward and backward
with dropout within the matmul tolerance."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import dropout as od
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import DEV, as_f64, assert_close, bf16_bits, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

P05 = float(np.float32(0.05))   # the probability as the library receives it (fp32)


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("M,K,p,seed", [
    (37, 1088, P05, 123),
    (5, 64, 0.5, (1 << 40) + 99),   # a seed with a non-zero high key word
    (16, 256, 0.0, 7),              # p = 0 keeps everything
])
def test_mask_and_dropped_input_bit_exact(M, K, p, seed):
    print("mask case", (M, K, p, seed), flush=True)
    X = workloads.activation_bf16((M, K), 5000 + M)
    Xd, keep = q.dropout_mask(to_dev_bf16(X), p, seed)
    Xd2 = q.dropout_apply(to_dev_bf16(X), keep)
    torch.cuda.synchronize()
    ref_keep = od.keep_mask(M, K, p, seed)
    assert np.array_equal(_bits(keep), od.pack_bits(ref_keep))
    assert np.array_equal(bf16_bits(Xd), od.drop(X, ref_keep))
    assert np.array_equal(bf16_bits(Xd2), od.drop(X, ref_keep))


def test_mask_full_size_sampled_rows():
    """The 7B activation shape (8192 x 11008): sampled rows of the mask (the
    counter passes 2^24 blocks, so the high counter word is exercised at
    larger shapes)."""
    M, K, seed = 8192, 11008, 2024
    X = workloads.device_normal((M, K), 1.0, 5100, DEV, torch.bfloat16)
    _, keep = q.dropout_mask(X, P05, seed)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 8191])
    ref = od.keep_mask_rows(rows, K, P05, seed)
    assert np.array_equal(_bits(keep)[rows], od.pack_bits(ref))
    rate = float(np.unpackbits(_bits(keep).view(np.uint8)).mean())
    assert abs(rate - (1 - od.threshold(P05) / 2.0 ** 32)) < 1e-3


def _layer(M, N, K, r, p, seed, s):
    W = workloads.weight((N, K), 5200 + K)
    X = workloads.activation_bf16((M, K), 5300 + M)
    A = workloads.lora_bf16((r, K), 5400)
    B = workloads.lora_bf16((N, r), 5500)
    dY = workloads.activation_bf16((M, N), 5600)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Xd_, Ad, Bd, dYd = (to_dev_bf16(t) for t in (X, A, B, dY))
    Y, T, keep = q.linear_fwd_dropout(Xd_, w, Ad, Bd, s, p, seed)
    dX, dA, dB = q.linear_bwd_dropout(dYd, Xd_, T, w, Ad, Bd, s, p, keep)
    torch.cuda.synchronize()
    wt = nf4.dequantize_q(nf4.quantize(W)).reshape(N, K)
    return (W, X, A, B, dY, wt), (w, Xd_, Ad, Bd, dYd), (Y, T, keep, dX, dA, dB)


@pytest.mark.parametrize("M,N,K,r", [(300, 520, 1088, 16), (16, 256, 1024, 64), (1024, 1024, 4096, 64)])
def test_layer_with_dropout(M, N, K, r):
    print("dropout layer case", (M, N, K, r), flush=True)
    s, seed = 16.0 / r, 31337
    (W, X, A, B, dY, wt), _, (Y, T, keep, dX, dA, dB) = _layer(M, N, K, r, P05, seed, s)
    ref_keep = od.keep_mask(M, K, P05, seed)
    assert np.array_equal(_bits(keep), od.pack_bits(ref_keep))
    Yr, Tr = od.linear_fwd(X, wt, A, B, s, P05, ref_keep)
    dXr, dAr, dBr, _ = od.linear_bwd(dY, X, wt, A, B, s, P05, ref_keep)
    assert_close(as_f64(T), Tr, "T")
    assert_close(as_f64(Y), Yr, "Y")
    assert_close(as_f64(dX), dXr, "dX")
    assert_close(as_f64(dA), dAr, "dA")
    assert_close(as_f64(dB), dBr, "dB")


def test_p0_matches_the_dropout_free_layer():
    """p = 0: T, Y, dA and dB bit-identical to the plain layer (same kernels
    and scale); dX within the tolerance (the LoRA term is added first)."""
    M, N, K, r, s = 300, 520, 1088, 16, 1.0
    _, (w, X, A, B, dY), (Y, T, keep, dX, dA, dB) = _layer(M, N, K, r, 0.0, 1, s)
    Y0, T0 = q.linear_fwd(X, w, A, B, s)
    dX0, dA0, dB0 = q.linear_bwd(dY, X, T0, w, A, B, s)
    torch.cuda.synchronize()
    eq = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert eq(T, T0) and eq(Y, Y0) and eq(dA, dA0) and eq(dB, dB0)
    assert_close(as_f64(dX), as_f64(dX0), "dX vs plain")
    assert int(np.unpackbits(_bits(keep).view(np.uint8)).min()) == 1
