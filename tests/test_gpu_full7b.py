"""Full-output GPU parity at the LLaMA-7B layer shapes (8192 tokens, r = 64,
alpha = 16), every linear of the layer, in the launch configuration the
benchmark times: T = s X A^T (lora_down), Y (nf4_matmul_fwd), G = s dY B
(lora_grad_in), dX (nf4_matmul_dx), dA and dB (lora_grads).  Every element
of T, Y, G, dX, dA and dB is compared with the fp64 oracle (relative
Frobenius error <= 5e-3 and |err| <= 2e-2 max|ref|), the dequantized weight
bit for bit, and every output and workspace sits between guard bands that
must stay intact.  The masked dX kernel of LoRA dropout is checked the same
way at the three distinct 7B shapes."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import dropout as od
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import Guarded, as_f64, assert_close, bf16_bits, guarded_like, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

CFG = workloads.CONFIGS[1]



@pytest.mark.parametrize("li", range(7))
def test_llama7b_linear_full_outputs(li):
    lin = CFG.linears[li]
    d = workloads.linear_inputs(CFG, li)
    M, N, K, r, s = d["M"], d["N"], d["K"], d["r"], CFG.scale
    print("full 7B case", lin.name, (M, N, K, r), flush=True)
    w = q.NF4Weight.quantize(to_dev_f32(d["W"]))
    X, A, B, dY = (to_dev_bf16(d[k]) for k in ("X", "A", "B", "dY"))
    gT, T = guarded_like((M, r), seed=1)
    gY, Y = guarded_like((M, N), seed=2)
    gG, G = guarded_like((M, r), seed=3)
    gdX, dX = guarded_like((M, K), seed=4)
    gdA, dA = guarded_like((r, K), seed=5)
    gdB, dB = guarded_like((N, r), seed=6)
    gws = Guarded(q.lib().qlora_lora_grads_workspace_bytes(M, N, K, r), seed=7, fill=0)
    ggw = Guarded(q.lib().qlora_lora_grad_in_workspace_bytes(N, r), seed=8, fill=0)
    q.lora_down(X, A, s, out=T)
    q.nf4_matmul_fwd(X, w, T, B, out=Y)
    q.lora_grad_in(dY, B, s, out=G, workspace=ggw.payload)
    q.nf4_matmul_dx(dY, w, G, A, out=dX)
    q.lora_grads(X, dY, G, T, workspace=gws.payload, dA_out=dA, dB_out=dB)
    torch.cuda.synchronize()
    for g, name in ((gT, "T"), (gY, "Y"), (gG, "G"), (gdX, "dX"), (gdA, "dA"), (gdB, "dB"), (gws, "ws"),
                    (ggw, "grad_in ws")):
        assert g.intact(), lin.name + ": guard band of " + name + " overwritten"

    ref = nf4.quantize(d["W"])
    wt = nf4.dequantize_q(ref).reshape(N, K)
    assert np.array_equal(bf16_bits(w.dequantize()), wt), lin.name + ": dequantized weight"
    Yr, Tr = olin.linear_fwd(d["X"], wt, d["A"], d["B"], s)
    sf = float(np.float32(s))
    assert_close(as_f64(T), sf * Tr, lin.name + " T")
    del Tr
    assert_close(as_f64(Y), Yr, lin.name + " Y")
    del Yr
    assert_close(as_f64(G), sf * olin.lora_grad_in(d["dY"], d["B"]), lin.name + " G")
    dXr, dAr, dBr = olin.linear_bwd(d["dY"], d["X"], wt, d["A"], d["B"], s)
    assert_close(as_f64(dX), dXr, lin.name + " dX")
    assert_close(as_f64(dA), dAr, lin.name + " dA")
    assert_close(as_f64(dB), dBr, lin.name + " dB")
    del w, X, A, B, dY, T, Y, G, dX, dA, dB
    torch.cuda.empty_cache()


_MASKS = {}


def _oracle_keep(M, K, p, seed):
    key = (M, K, p, seed)
    if key not in _MASKS:
        _MASKS.clear()
        _MASKS[key] = od.keep_mask(M, K, p, seed)
    return _MASKS[key]


@pytest.mark.parametrize("li", [0, 4, 6])
def test_llama7b_masked_dx_full_outputs(li):
    """The dropout variant of the dX matmul (LoRA term gated by the keep
    mask) at the 7B shapes and 8192 tokens, p = 0.05: the mask bit-exact and
    every element of dX against the oracle."""
    lin = CFG.linears[li]
    d = workloads.linear_inputs(CFG, li)
    M, N, K, r, s, p = d["M"], d["N"], d["K"], d["r"], CFG.scale, 0.05
    seed = 0x5EED0000 + K
    print("masked dX case", lin.name, (M, N, K, r), flush=True)
    w = q.NF4Weight.quantize(to_dev_f32(d["W"]))
    X, A, B, dY = (to_dev_bf16(d[k]) for k in ("X", "A", "B", "dY"))
    Xd, keep = q.dropout_mask(X, p, seed)
    se = float(od.effective_scale(s, p))
    G = q.lora_grad_in(dY, B, se)
    gdX, dX = guarded_like((M, K), seed=9)
    q.nf4_matmul_dx_dropout(dY, w, G, A, keep, out=dX)
    torch.cuda.synchronize()
    assert gdX.intact(), lin.name + ": guard band of dX overwritten"
    kr = _oracle_keep(M, K, p, seed)
    assert np.array_equal(keep.cpu().numpy().view(np.uint32), od.pack_bits(kr)), lin.name + ": keep mask"
    wt = nf4.dequantize_q(nf4.quantize(d["W"])).reshape(N, K)
    dXr, _, _, _ = od.linear_bwd(d["dY"], d["X"], wt, d["A"], d["B"], s, p, kr)
    assert_close(as_f64(dX), dXr, lin.name + " masked dX")
    del w, X, A, B, dY, Xd, keep, G, dX
    torch.cuda.empty_cache()
