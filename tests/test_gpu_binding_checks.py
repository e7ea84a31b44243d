"""The Python binding rejects, before any launch, caller workspaces that are
too small and caller-supplied outputs or inputs of the wrong shape or dtype,
so that no mismatched buffer reaches a kernel as a raw pointer."""

import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from tests.gpu_util import to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

M, N, K, R, S = 96, 256, 512, 16, 2.0


@pytest.fixture(scope="module")
def layer():
    W = workloads.weight((N, K), 1800)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    X = to_dev_bf16(workloads.activation_bf16((M, K), 1801))
    A = to_dev_bf16(workloads.lora_bf16((R, K), 1802))
    B = to_dev_bf16(workloads.lora_bf16((N, R), 1803))
    dY = to_dev_bf16(workloads.activation_bf16((M, N), 1804))
    return w, X, A, B, dY


def _small(nbytes):
    return torch.empty(max(nbytes - 16, 0), dtype=torch.uint8, device="cuda:0")


def test_undersized_workspaces_raise(layer):
    w, X, A, B, dY = layer
    L = q.lib()
    _, T = q.linear_fwd(X, w, A, B, S)
    G = q.lora_grad_in(dY, B, S)
    with pytest.raises(ValueError, match="needed"):
        q.linear_bwd(dY, X, T, w, A, B, S, workspace=_small(L.qlora_linear_workspace_bytes(M, N, K, R, 1)))
    with pytest.raises(ValueError, match="needed"):
        q.lora_grads(X, dY, G, T, workspace=_small(L.qlora_lora_grads_workspace_bytes(M, N, K, R)))
    with pytest.raises(ValueError, match="needed"):
        q.linear_fwd_dropout(X, w, A, B, S, 0.1, 3,
                             workspace=_small(L.qlora_linear_dropout_workspace_bytes(M, N, K, R, 0)))
    _, T2, keep = q.linear_fwd_dropout(X, w, A, B, S, 0.1, 3)
    with pytest.raises(ValueError, match="needed"):
        q.linear_bwd_dropout(dY, X, T2, w, A, B, S, 0.1, keep,
                             workspace=_small(L.qlora_linear_dropout_workspace_bytes(M, N, K, R, 1)))
    with pytest.raises(ValueError, match="needed"):
        q.lora_grad_in(dY, B, S, workspace=_small(L.qlora_lora_grad_in_workspace_bytes(N, R)))
    torch.cuda.synchronize()


def test_mismatched_tensors_raise(layer):
    w, X, A, B, dY = layer
    _, T = q.linear_fwd(X, w, A, B, S)
    G = q.lora_grad_in(dY, B, S)
    bf = torch.bfloat16
    bad_T = torch.empty(M, R + 8, dtype=bf, device="cuda:0")
    with pytest.raises(ValueError):
        q.lora_grads(X, dY, G, bad_T)
    with pytest.raises(ValueError):
        q.lora_grads(X, dY[:M // 2].contiguous(), G, T)
    with pytest.raises(TypeError):
        q.lora_grads(X.float(), dY, G, T)
    with pytest.raises(ValueError):
        q.lora_down(X, A, S, out=torch.empty(M - 1, R, dtype=bf, device="cuda:0"))
    with pytest.raises(ValueError):
        q.nf4_matmul_fwd(X, w, T, B, out=torch.empty(M, N - 8, dtype=bf, device="cuda:0"))
    with pytest.raises(ValueError):
        q.nf4_matmul_dx(dY, w, G, A, out=torch.empty(M, K, dtype=bf, device="cuda:0").t())
    with pytest.raises(ValueError):
        q.lora_grad_in(dY, B, S, out=torch.empty(M, R - 1, dtype=bf, device="cuda:0"))
    with pytest.raises(ValueError):
        q.linear_bwd(dY, X, T, w, A, B, S, dA_out=torch.empty(R, K - 64, dtype=bf, device="cuda:0"))
    Xd, keep = q.dropout_mask(X, 0.1, 5)
    with pytest.raises(ValueError):
        q.nf4_matmul_dx_dropout(dY, w, G, A, keep, out=torch.empty(M, K + 64, dtype=bf, device="cuda:0"))
    with pytest.raises(ValueError):
        q.dropout_mask(X, 0.1, 5, keep_out=torch.empty(M, K // 64, dtype=torch.int32, device="cuda:0"))
    with pytest.raises(ValueError):
        q.linear_fwd_dropout(X, w, A, B, S, 0.1, 5, T_out=torch.empty(M, 2 * R, dtype=bf, device="cuda:0"))
    torch.cuda.synchronize()
