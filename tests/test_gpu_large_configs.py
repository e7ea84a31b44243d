"""GPU parity at the larger layer configs: a LLaMA-33B-shaped layer at 8192
tokens and a LLaMA-65B-shaped model (80 layers quantized on the device, one
layer at 16384 tokens).  Full-size products are checked on sampled rows and
columns that the fp64 oracle computes one by one (same tolerance as the other
matmul tests); the codec is checked bit-exactly on whole tensors."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import DEV, as_f64, assert_close, bf16_bits, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _sampled_layer_check(cfg, li, tokens=None, seed=0):
    d = workloads.linear_inputs(cfg, li, tokens)
    M, N, K = d["M"], d["N"], d["K"]
    print("full-size case", cfg.name, cfg.linears[li].name, (M, N, K), flush=True)
    w = q.NF4Weight.quantize(to_dev_f32(d["W"]))
    Xd, Ad, Bd, dYd = (to_dev_bf16(d[k]) for k in ("X", "A", "B", "dY"))
    Y, T = q.linear_fwd(Xd, w, Ad, Bd, d["scale"])
    dX, dA, dB = q.linear_bwd(dYd, Xd, T, w, Ad, Bd, d["scale"])
    torch.cuda.synchronize()
    ref = nf4.quantize(d["W"])
    assert np.array_equal(w.packed.cpu().numpy(), ref["packed"]), "packed"
    assert np.array_equal(w.code8.cpu().numpy(), ref["code8"]), "code8"
    wt = nf4.dequantize_q(ref).reshape(N, K)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.integers(0, M, 24), [0, M - 1]]))
    assert_close(as_f64(Y)[rows], olin.linear_fwd_rows(d["X"], wt, d["A"], d["B"], d["scale"], rows), "Y rows")
    assert_close(as_f64(dX)[rows], olin.linear_dx_rows(d["dY"], wt, d["A"], d["B"], d["scale"], rows), "dX rows")
    cols = np.unique(np.concatenate([rng.integers(0, K, 48), [0, K - 1]]))
    assert_close(as_f64(dA)[:, cols], olin.linear_dA_cols(d["dY"], d["X"], d["B"], d["scale"], cols), "dA cols")
    nrows = np.unique(np.concatenate([rng.integers(0, N, 48), [0, N - 1]]))
    assert_close(as_f64(dB)[nrows], olin.linear_dB_rows(d["dY"], d["X"], d["A"], d["scale"], nrows), "dB rows")
    del w, Y, T, dX, dA, dB, Xd, Ad, Bd, dYd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("li", [0, 4, 6])
def test_llama33b_full_size_sampled(li):
    """33B layer (hidden 6656, FFN 17920) at 8192 tokens, r = 64."""
    _sampled_layer_check(workloads.CONFIGS[3], li, seed=li)


@pytest.mark.parametrize("li", [0, 4, 6])
def test_llama65b_layer_m16384_sampled(li):
    """One 65B layer (hidden 8192, FFN 22016) at 16384 tokens, r = 64."""
    _sampled_layer_check(workloads.CONFIGS[4], li, seed=100 + li)


def _stored_bytes(n):
    """Bytes the layout stores for an n-parameter tensor: packed codes, 8-bit
    constant codes, second-level scales and the mean."""
    nb = -(-n // 64)
    return -(-n // 2) + nb + 4 * (-(-nb // 256)) + 4


def test_llama65b_quantize_80_layers():
    """All 80 layers of the 65B model generated and quantized on the device.
    Checks the stored size of every tensor (4 + 8/64 + 32/16384 bits per
    parameter plus the mean), and bit-exact codes, constants, scales and mean
    of whole tensors in layers 0 and 79 and two layers in between."""
    cfg = workloads.CONFIGS[4]
    checked = {(0, "q_proj"), (79, "down_proj"), (23, "k_proj"), (51, "up_proj")}
    params = 0
    stored = 0
    for layer in range(cfg.layers):
        for lin, W in workloads.device_layer_weights(cfg, layer, DEV):
            w = q.NF4Weight.quantize(W)
            n = W.numel()
            got = w.packed.numel() + w.code8.numel() + 4 * w.c2.numel() + 4 * w.mean.numel()
            assert got == _stored_bytes(n), (layer, lin.name, got)
            params += n
            stored += got
            if (layer, lin.name) in checked:
                print("codec case 65B layer", layer, lin.name, tuple(W.shape), flush=True)
                ref = nf4.quantize(W.cpu().numpy())
                assert np.array_equal(w.packed.cpu().numpy(), ref["packed"]), "packed"
                assert np.array_equal(w.code8.cpu().numpy(), ref["code8"]), "code8"
                assert np.array_equal(w.c2.cpu().numpy().view(np.uint32), ref["c2"].view(np.uint32)), "c2"
                mean = np.float32(w.mean.cpu().numpy()[0])
                assert mean.view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), "mean"
            del w, W
        torch.cuda.synchronize()
    assert params == cfg.layers * sum(l.out_features * l.in_features for l in cfg.linears)
    bits = 8.0 * stored / params
    print("65B: %d params, %d bytes stored, %.6f bits/param" % (params, stored, bits), flush=True)
    assert 4.126953 <= bits <= 4.126954


@pytest.mark.parametrize("kernel", ["fwd", "dx"])
def test_fused_matmul_repeat_bit_identical(kernel):
    """Sixteen repeated calls of a fused NF4 matmul at the 65B gate_proj shape
    (M = 16384, N = 22016, K = 8192, r = 64) give bit-identical outputs.  The
    kernels reuse their LDS stages every step, so an unfinished DMA or
    expansion write at a step boundary shows up as an occasional tile that
    differs from one call to the next."""
    M, N, K, r = 16384, 22016, 8192, 64
    print("repeat case", kernel, (M, N, K, r), flush=True)
    w = q.NF4Weight.quantize(workloads.device_normal((N, K), 0.02, 11, DEV))
    if kernel == "fwd":
        L = workloads.device_normal((M, K), 1.0, 12, DEV, torch.bfloat16)
        R = workloads.device_normal((N, r), 0.01, 14, DEV, torch.bfloat16)
        call = lambda out: q.nf4_matmul_fwd(L, w, Ln, R, out=out)
    else:
        L = workloads.device_normal((M, N), 1.0, 12, DEV, torch.bfloat16)
        R = workloads.device_normal((r, K), 0.01, 14, DEV, torch.bfloat16)
        call = lambda out: q.nf4_matmul_dx(L, w, Ln, R, out=out)
    Ln = workloads.device_normal((M, r), 1.0, 13, DEV, torch.bfloat16)
    ref = call(None)
    assert not bool(torch.isnan(ref).any())
    out = torch.empty_like(ref)
    for i in range(16):
        out.fill_(float("nan"))
        call(out)
        diff = (out != ref).nonzero()
        if diff.numel():
            tiles = sorted({(int(a) // 256, int(b) // 256) for a, b in diff[:4096].cpu().numpy()})
            raise AssertionError("call %d: %d elements differ, tiles %s" % (i + 1, diff.shape[0], tiles[:8]))
    del w, L, R, Ln, ref, out
    torch.cuda.empty_cache()
