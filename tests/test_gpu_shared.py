"""GPU parity of the shared-input LoRA products (linears that read the same X,
like q / k / v or gate / up): T = s X A_i^T and dA = G_i^T X for every
member in one launch must be bit-identical to the per-linear calls, and
match the oracle; the grouped forward fuses them for descriptors that carry
the same X."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import as_f64, assert_close, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _eq(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M,K,rs", [
    (300, 1088, (64, 100, 8)),      # ragged rows, a rank past one chunk, an odd rank
    (8192, 4096, (64, 64, 64)),     # the 7B q / k / v shape
    (8192, 4096, (64, 64)),         # the 7B gate / up shape
    (40, 256, (16,)),               # a single member
])
def test_lora_down_shared(M, K, rs):
    print("shared down case", (M, K, rs), flush=True)
    X = workloads.activation_bf16((M, K), 4000 + M)
    As = [workloads.lora_bf16((r, K), 4100 + i) for i, r in enumerate(rs)]
    scales = [16.0 / r for r in rs]
    Xd = to_dev_bf16(X)
    Ad = [to_dev_bf16(A) for A in As]
    Ts = q.lora_down_shared(Xd, Ad, scales)
    singles = [q.lora_down(Xd, A, s) for A, s in zip(Ad, scales)]
    torch.cuda.synchronize()
    for T, T1 in zip(Ts, singles):
        assert _eq(T, T1)
    rows = np.arange(0, M, max(1, M // 64))
    for T, A, s in zip(Ts, As, scales):
        ref = np.float32(s) * olin.lora_down(X[rows], A)
        assert_close(as_f64(T)[rows], ref, "T")


@pytest.mark.parametrize("M,K,rs", [
    (300, 1088, (64, 100, 8)),      # one M-split
    (4096, 1088, (64, 20)),         # several M-splits (fp32 partials), an unpadded and a padded G
    (8192, 4096, (64, 64, 64)),     # the 7B q / k / v shape
    (8192, 11008, (64, 64)),        # 7B gate / up read X [8192, 4096]; here a wider X
])
def test_lora_dA_shared(M, K, rs):
    print("shared dA case", (M, K, rs), flush=True)
    X = workloads.activation_bf16((M, K), 4200 + M)
    Gs = [workloads.lora_bf16((M, r), 4300 + i) for i, r in enumerate(rs)]
    Xd = to_dev_bf16(X)
    Gd = [to_dev_bf16(G) for G in Gs]
    dAs = q.lora_dA_shared(Xd, Gd)
    dY = torch.zeros(M, 8, dtype=torch.bfloat16, device=Xd.device)
    singles = [q.lora_grads(Xd, dY, G, G, need_dB=False)[0] for G in Gd]
    torch.cuda.synchronize()
    for dA, dA1 in zip(dAs, singles):
        assert _eq(dA, dA1)
    cols = np.arange(0, K, max(1, K // 48))
    for dA, G in zip(dAs, Gs):
        # G^T X through the oracle's dA = s (dY B)^T X with dY = G, B = I, s = 1
        ref = olin.linear_dA_cols(G, X, np.eye(G.shape[1]), 1.0, cols)
        assert_close(as_f64(dA)[:, cols], ref, "dA")


@pytest.mark.parametrize("M", [100, 1024])
def test_group_forward_fuses_shared_inputs(M):
    """q, k, v share one X and gate, up another; o has its own: the grouped
    forward gives bit-identical Y and T to single calls."""
    print("group shared case M", M, flush=True)
    Xa = to_dev_bf16(workloads.activation_bf16((M, 1024), 4400 + M))
    Xb = to_dev_bf16(workloads.activation_bf16((M, 512), 4500 + M))
    Xc = to_dev_bf16(workloads.activation_bf16((M, 1024), 4600 + M))
    spec = [(Xa, 1024, 1024, 64), (Xa, 256, 1024, 64), (Xa, 256, 1024, 16),
            (Xb, 768, 512, 32), (Xb, 768, 512, 32), (Xc, 512, 1024, 64)]
    items, refs = [], []
    for i, (Xd, N, K, r) in enumerate(spec):
        W = workloads.weight((N, K), 4700 + i)
        A = workloads.lora_bf16((r, K), 4800 + i)
        B = workloads.lora_bf16((N, r), 4900 + i)
        w = q.NF4Weight.quantize(to_dev_f32(W))
        items.append((Xd, w, to_dev_bf16(A), to_dev_bf16(B), 16.0 / r))
        refs.append((W, A, B, 16.0 / r))
    outs = q.linear_fwd_group(items)
    singles = [q.linear_fwd(*it) for it in items]
    torch.cuda.synchronize()
    for (Y, T), (Y1, T1) in zip(outs, singles):
        assert _eq(Y, Y1) and _eq(T, T1)
    # one member against the oracle
    X = items[1][0].view(torch.int16).cpu().numpy().view(np.uint16)
    W, A, B, s = refs[1]
    Yr, _ = olin.linear_fwd(X, nf4.dequantize_q(nf4.quantize(W)).reshape(W.shape), A, B, s)
    assert_close(as_f64(outs[1][0]), Yr, "group Y")
