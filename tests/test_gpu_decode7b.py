"""The decode-regime forward at the LLaMA-7B layer shapes, exactly as the
benchmark calls it: one grouped call over the seven linears (q, k, v, o,
gate, up, down; each with its own X, T_out and Y) and one call per linear,
at M = 1, 16 and 64 tokens, r = 64, alpha = 16.  Every element of every Y
and T is compared with the fp64 oracle, a repeated grouped call must give the
same bits, and the outputs and the workspace sit between guard bands."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import Guarded, as_f64, assert_close, guarded_like, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

CFG = workloads.CONFIGS[2]


@pytest.fixture(scope="module")
def weights():
    """Device NF4 weights of the 7 linears and the oracle's dequantized copies."""
    out = []
    for li, lin in enumerate(CFG.linears):
        W = workloads.linear_inputs(CFG, li, tokens=1)["W"]
        out.append((q.NF4Weight.quantize(to_dev_f32(W)), nf4.dequantize_q(nf4.quantize(W)).reshape(W.shape)))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M", [1, 16, 64])
def test_llama7b_decode_group_and_single(weights, M):
    print("decode 7B case M", M, flush=True)
    s, r = CFG.scale, CFG.rank
    host, items, guards = [], [], []
    for li, lin in enumerate(CFG.linears):
        d = workloads.linear_inputs(CFG, li, tokens=M)
        X, A, B = (to_dev_bf16(d[k]) for k in ("X", "A", "B"))
        gY, Y = guarded_like((M, d["N"]), seed=10 * li + 1)
        gT, T = guarded_like((M, r), seed=10 * li + 2)
        guards += [(gY, lin.name + " Y"), (gT, lin.name + " T")]
        items.append((X, weights[li][0], A, B, s, T, Y))
        host.append(d)
    from bit_nf4_quantized_absmax_amd._capi import LinearDescStruct
    import ctypes
    sts = [it[1].struct() for it in items]
    descs = (LinearDescStruct * 7)(*[LinearDescStruct(it[0].data_ptr(), ctypes.pointer(st), it[2].data_ptr(),
                                                      it[3].data_ptr(), r, s, it[6].data_ptr(), it[5].data_ptr())
                                     for it, st in zip(items, sts)])
    gws = Guarded(q.lib().qlora_linear_group_workspace_bytes(7, descs, M), seed=99, fill=0)
    q.linear_fwd_group(items, workspace=gws.payload)
    first = [(Y.clone(), T.clone()) for (_, _, _, _, _, T, Y) in items]
    q.linear_fwd_group(items, workspace=gws.payload)
    torch.cuda.synchronize()
    for g, name in guards + [(gws, "group workspace")]:
        assert g.intact(), "M=%d: guard band of %s overwritten" % (M, name)
    for (Y1, T1), it, lin in zip(first, items, CFG.linears):
        assert torch.equal(Y1.view(torch.int16), it[6].view(torch.int16)), lin.name + ": repeat Y"
        assert torch.equal(T1.view(torch.int16), it[5].view(torch.int16)), lin.name + ": repeat T"
    # the per-linear calls, each with its own guarded workspace
    singles = []
    for li, it in enumerate(items):
        X, w, A, B = it[:4]
        N, K = w.rows, w.cols
        gy, Ys = guarded_like((M, N), seed=200 + li)
        gt, Ts = guarded_like((M, r), seed=300 + li)
        gw = Guarded(q.lib().qlora_linear_workspace_bytes(M, N, K, r, 0), seed=400 + li, fill=0)
        q.linear_fwd(X, w, A, B, s, T_out=Ts, out=Ys, workspace=gw.payload)
        singles.append((Ys, Ts, (gy, gt, gw)))
    torch.cuda.synchronize()
    for li, (d, lin) in enumerate(zip(host, CFG.linears)):
        for g in singles[li][2]:
            assert g.intact(), "M=%d %s: single-call guard band overwritten" % (M, lin.name)
        Yr, Tr = olin.linear_fwd(d["X"], weights[li][1], d["A"], d["B"], s)
        Tr = float(np.float32(s)) * Tr
        assert_close(as_f64(items[li][6]), Yr, "M=%d %s group Y" % (M, lin.name))
        assert_close(as_f64(items[li][5]), Tr, "M=%d %s group T" % (M, lin.name))
        assert_close(as_f64(singles[li][0]), Yr, "M=%d %s single Y" % (M, lin.name))
        assert_close(as_f64(singles[li][1]), Tr, "M=%d %s single T" % (M, lin.name))
