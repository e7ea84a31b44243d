"""Every output combination of the composite backward passes, with and
without LoRA dropout: T given or NULL (recomputed from X, or from X_d with
dropout), and each non-empty subset of dX / dA / dB requested.  Requested
outputs are compared with the oracle; outputs, workspaces and the untouched
buffers of unrequested outputs sit between guard bands, and the unrequested
ones must keep their fill.  Also the M = 0 contract: nothing is written."""

import itertools

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import dropout as od
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import Guarded, as_f64, assert_close, guarded_like, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

M, N, K, R, S = 300, 512, 768, 32, 0.5
SUBSETS = [c for n in (1, 2, 3) for c in itertools.combinations(("dX", "dA", "dB"), n)]


def _host(seed):
    W = workloads.weight((N, K), seed)
    X = workloads.activation_bf16((M, K), seed + 1)
    A = workloads.lora_bf16((R, K), seed + 2)
    B = workloads.lora_bf16((N, R), seed + 3)
    dY = workloads.activation_bf16((M, N), seed + 4)
    return W, X, A, B, dY


def _outputs(tag):
    shapes = {"dX": (M, K), "dA": (R, K), "dB": (N, R)}
    return {k: guarded_like(shp, seed=hash((tag, k)) % 1000) for k, shp in shapes.items()}


@pytest.mark.parametrize("t_given", [True, False])
def test_linear_bwd_every_output_subset(t_given):
    W, X, A, B, dY = _host(1500)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Xd, Ad, Bd, dYd = (to_dev_bf16(t) for t in (X, A, B, dY))
    _, T = q.linear_fwd(Xd, w, Ad, Bd, S)
    wt = nf4.dequantize_q(nf4.quantize(W)).reshape(N, K)
    ref = dict(zip(("dX", "dA", "dB"), olin.linear_bwd(dY, X, wt, A, B, S)))
    for sub in SUBSETS:
        print("bwd subset", sub, "T given" if t_given else "T NULL", flush=True)
        outs = _outputs(sub)
        gws = Guarded(q.lib().qlora_linear_workspace_bytes(M, N, K, R, 1), seed=77, fill=0)
        q.linear_bwd(dYd, Xd, T if t_given else None, w, Ad, Bd, S, need_dX="dX" in sub, need_dA="dA" in sub,
                     need_dB="dB" in sub, workspace=gws.payload, dX_out=outs["dX"][1], dA_out=outs["dA"][1],
                     dB_out=outs["dB"][1])
        torch.cuda.synchronize()
        assert gws.intact(), "workspace guard"
        for k, (g, t) in outs.items():
            assert g.intact(), "%s guard (%s)" % (k, sub)
            if k in sub:
                assert_close(as_f64(t), ref[k], "%s %s" % (k, sub))
            else:
                assert torch.all(g.payload == 0xFF), "%s written although not requested (%s)" % (k, sub)


@pytest.mark.parametrize("t_given", [True, False])
def test_linear_bwd_dropout_every_output_subset(t_given):
    p, seed = 0.1, 0xABCDEF
    W, X, A, B, dY = _host(1600)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Xd, Ad, Bd, dYd = (to_dev_bf16(t) for t in (X, A, B, dY))
    _, T, keep = q.linear_fwd_dropout(Xd, w, Ad, Bd, S, p, seed)
    kr = od.keep_mask(M, K, p, seed)
    torch.cuda.synchronize()
    assert np.array_equal(keep.cpu().numpy().view(np.uint32), od.pack_bits(kr))
    wt = nf4.dequantize_q(nf4.quantize(W)).reshape(N, K)
    dXr, dAr, dBr, _ = od.linear_bwd(dY, X, wt, A, B, S, p, kr)
    ref = {"dX": dXr, "dA": dAr, "dB": dBr}
    for sub in SUBSETS:
        print("dropout bwd subset", sub, "T given" if t_given else "T NULL", flush=True)
        outs = _outputs(("drop",) + sub)
        gws = Guarded(q.lib().qlora_linear_dropout_workspace_bytes(M, N, K, R, 1), seed=78, fill=0)
        q.linear_bwd_dropout(dYd, Xd, T if t_given else None, w, Ad, Bd, S, p, keep, need_dX="dX" in sub,
                             need_dA="dA" in sub, need_dB="dB" in sub, workspace=gws.payload,
                             dX_out=outs["dX"][1], dA_out=outs["dA"][1], dB_out=outs["dB"][1])
        torch.cuda.synchronize()
        assert gws.intact(), "workspace guard"
        for k, (g, t) in outs.items():
            assert g.intact(), "%s guard (%s)" % (k, sub)
            if k in sub:
                assert_close(as_f64(t), ref[k], "dropout %s %s" % (k, sub))
            else:
                assert torch.all(g.payload == 0xFF), "%s written although not requested (%s)" % (k, sub)


def test_zero_tokens_write_nothing():
    """M = 0: every entry point that takes a token count returns OK and leaves
    its outputs (here dA, dB and the workspace) exactly as they were."""
    W, _, A, B, _ = _host(1700)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Ad, Bd = to_dev_bf16(A), to_dev_bf16(B)
    X0 = torch.empty(0, K, dtype=torch.bfloat16, device="cuda:0")
    dY0 = torch.empty(0, N, dtype=torch.bfloat16, device="cuda:0")
    G0 = torch.empty(0, R, dtype=torch.bfloat16, device="cuda:0")
    outs = _outputs("m0")
    gws = Guarded(max(q.lib().qlora_linear_workspace_bytes(0, N, K, R, 1),
                      q.lib().qlora_lora_grads_workspace_bytes(0, N, K, R)), seed=79, fill=0x5A)
    q.linear_bwd(dY0, X0, None, w, Ad, Bd, S, workspace=gws.payload, dX_out=outs["dX"][1][:0],
                 dA_out=outs["dA"][1], dB_out=outs["dB"][1])
    q.lora_grads(X0, dY0, G0, G0, workspace=gws.payload, dA_out=outs["dA"][1], dB_out=outs["dB"][1])
    Y0, T0 = q.linear_fwd(X0, w, Ad, Bd, S)
    torch.cuda.synchronize()
    assert Y0.shape == (0, N) and T0.shape == (0, R)
    assert gws.intact() and torch.all(gws.payload == 0x5A)
    for k, (g, _) in outs.items():
        assert g.intact() and torch.all(g.payload == 0xFF), k
