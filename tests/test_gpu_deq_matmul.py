"""GPU checks of the matmuls from a dequantized weight (qlora_deq_matmul_fwd,
_fwd_group, _dx): given the bf16 weight the dequantizer writes, their outputs
are bit-identical to the fused dequant matmuls on the NF4 weight (same weight
values, same contraction order), and they match the fp64 oracle (relative
Frobenius error <= 5e-3, elementwise |err| <= 2e-2 max|ref|)."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import DEV, Guarded, as_f64, assert_close, bf16_bits, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _dev(M, N, K, r, qtype, seed):
    g = torch.Generator(DEV).manual_seed(seed)
    bf = torch.bfloat16
    W = torch.randn(N, K, device=DEV, generator=g) * 0.02
    w = q.NF4Weight.quantize(W, qtype)
    return dict(w=w, Wd=w.dequantize(), X=torch.randn(M, K, device=DEV, generator=g).to(bf),
                dY=torch.randn(M, N, device=DEV, generator=g).to(bf),
                T=(torch.randn(M, r, device=DEV, generator=g) * 0.1).to(bf),
                G=(torch.randn(M, r, device=DEV, generator=g) * 0.1).to(bf),
                A=(torch.randn(r, K, device=DEV, generator=g) * 0.01).to(bf),
                B=(torch.randn(N, r, device=DEV, generator=g) * 0.01).to(bf))


def _same(a, b, name):
    assert torch.isfinite(a.float()).all(), name + ": not finite"
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


# M >= 65 (the fused kernels' tile route): ragged row tiles, N and K that
# leave partial column tiles, r not a multiple of 8 and r over 64 (two LoRA
# steps), the three 4-bit tables.  r = 64 with an even number of 64-deep
# contraction steps runs the LoRA step inside the DMA pipeline (two steps is
# the shortest such loop); r = 64 with an odd count stages it after the loop.
CASES = [(300, 1024, 512, 64, "nf4"), (257, 576, 1088, 12, "fp4"), (513, 1344, 704, 96, "int4"),
         (65, 64, 64, 128, "nf4"), (1000, 2048, 4096, 8, "nf4"), (300, 704, 576, 64, "nf4"),
         (130, 128, 128, 64, "fp4")]


@pytest.mark.parametrize("M,N,K,r,qtype", CASES)
def test_deq_matmul_bit_identical_to_fused(M, N, K, r, qtype):
    print("deq matmul case", (M, N, K, r, qtype), flush=True)
    d = _dev(M, N, K, r, qtype, 7 + M)
    Y = q.deq_matmul_fwd(d["X"], d["Wd"], d["T"], d["B"])
    dX = q.deq_matmul_dx(d["dY"], d["Wd"], d["G"], d["A"])
    Yf = q.nf4_matmul_fwd(d["X"], d["w"], d["T"], d["B"])
    dXf = q.nf4_matmul_dx(d["dY"], d["w"], d["G"], d["A"])
    torch.cuda.synchronize()
    _same(Y, Yf, "Y")
    _same(dX, dXf, "dX")


def test_deq_matmul_group_llama7b_gate_up_and_dx():
    cfg = workloads.CONFIGS[1]
    lins = [l for l in cfg.linears if l.name in ("gate_proj", "up_proj")]
    print("deq matmul group case gate/up", cfg.tokens, flush=True)
    ds = [_dev(cfg.tokens, l.out_features, l.in_features, cfg.rank, "nf4", 60 + i) for i, l in enumerate(lins)]
    grp = q.deq_matmul_fwd_group([dict(X=d["X"], Wd=d["Wd"], T=d["T"], B=d["B"]) for d in ds])
    fused = q.nf4_matmul_fwd_group([dict(X=d["X"], w=d["w"], T=d["T"], B=d["B"]) for d in ds])
    dxs = [q.deq_matmul_dx(d["dY"], d["Wd"], d["G"], d["A"]) for d in ds]
    dxf = [q.nf4_matmul_dx(d["dY"], d["w"], d["G"], d["A"]) for d in ds]
    torch.cuda.synchronize()
    for i in range(2):
        _same(grp[i], fused[i], "Y member %d" % i)
        _same(dxs[i], dxf[i], "dX member %d" % i)


def test_deq_matmul_llama7b_down_dx():
    # down_proj: N = 4096 output rows, K = 11008: 43 column tiles of dX, a
    # partial last one
    cfg = workloads.CONFIGS[1]
    lin = [l for l in cfg.linears if l.name == "down_proj"][0]
    print("deq matmul case down_proj", cfg.tokens, flush=True)
    d = _dev(cfg.tokens, lin.out_features, lin.in_features, cfg.rank, "nf4", 70)
    dX = q.deq_matmul_dx(d["dY"], d["Wd"], d["G"], d["A"])
    Y = q.deq_matmul_fwd(d["X"], d["Wd"], d["T"], d["B"])
    dXf = q.nf4_matmul_dx(d["dY"], d["w"], d["G"], d["A"])
    Yf = q.nf4_matmul_fwd(d["X"], d["w"], d["T"], d["B"])
    torch.cuda.synchronize()
    _same(dX, dXf, "dX")
    _same(Y, Yf, "Y")


@pytest.mark.parametrize("M", [16, 300])
def test_deq_matmul_matches_oracle(M):
    # the oracle's linear layer on the oracle's dequantized weight; M = 16
    # runs the tile route too (the fused forward would take the decode route)
    N, K, r, scale = 512, 768, 16, 2.0
    print("deq matmul oracle case", (M, N, K, r), flush=True)
    seed = 900 + M
    W = workloads.weight((N, K), seed)
    X = workloads.activation_bf16((M, K), seed + 1)
    A = workloads.lora_bf16((r, K), seed + 2)
    B = workloads.lora_bf16((N, r), seed + 3)
    dY = workloads.activation_bf16((M, N), seed + 4)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Wd = w.dequantize()
    wt = nf4.dequantize_q(nf4.quantize(W)).reshape(W.shape)
    assert np.array_equal(bf16_bits(Wd), wt), "dequantized weight"
    Xd, Ad, Bd, dYd = (to_dev_bf16(t) for t in (X, A, B, dY))
    T = q.lora_down(Xd, Ad, scale)
    G = q.lora_grad_in(dYd, Bd, scale)
    Y = q.deq_matmul_fwd(Xd, Wd, T, Bd)
    dX = q.deq_matmul_dx(dYd, Wd, G, Ad)
    torch.cuda.synchronize()
    Yr, _ = olin.linear_fwd(X, wt, A, B, scale)
    dXr, _, _ = olin.linear_bwd(dY, X, wt, A, B, scale)
    assert_close(as_f64(Y), Yr, "Y")
    assert_close(as_f64(dX), dXr, "dX")


def test_deq_matmul_writes_only_its_output_and_m0_is_a_no_op():
    M, N, K, r = 130, 320, 256, 24
    print("deq matmul guard case", (M, N, K, r), flush=True)
    d = _dev(M, N, K, r, "nf4", 5)
    gy = Guarded(M * N * 2)
    gx = Guarded(M * K * 2)
    Y = gy.tensor((M, N))
    dX = gx.tensor((M, K))
    q.deq_matmul_fwd(d["X"], d["Wd"], d["T"], d["B"], out=Y)
    q.deq_matmul_dx(d["dY"], d["Wd"], d["G"], d["A"], out=dX)
    torch.cuda.synchronize()
    assert gy.intact() and gx.intact()
    assert torch.isfinite(Y.float()).all() and torch.isfinite(dX.float()).all()
    e = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    e2 = torch.empty(0, r, dtype=torch.bfloat16, device=DEV)
    Y0 = q.deq_matmul_fwd(e, d["Wd"], e2, d["B"])
    assert Y0.shape == (0, N)


def test_deq_matmul_dx_rejects_n_not_multiple_of_64():
    d = _dev(128, 72, 128, 8, "nf4", 3)
    with pytest.raises(q.QLoRAError):
        q.deq_matmul_dx(d["dY"], d["Wd"], d["G"], d["A"])
    Y = q.deq_matmul_fwd(d["X"], d["Wd"], d["T"], d["B"])   # the forward takes N % 8 == 0
    Yf = q.nf4_matmul_fwd(d["X"], d["w"], d["T"], d["B"])
    torch.cuda.synchronize()
    _same(Y, Yf, "Y (N = 72)")


@pytest.mark.parametrize("cfg_index,names", [(3, ("gate_proj", "down_proj")), (4, ("up_proj", "down_proj"))])
def test_deq_matmul_larger_layers_bit_identical(cfg_index, names):
    # the 33B (M = 8192) and 65B (M = 16384) shapes that the bench's layer
    # figures run through this path: forward and dX, as the fused kernels
    cfg = workloads.CONFIGS[cfg_index]
    for i, lin in enumerate(l for l in cfg.linears if l.name in names):
        print("deq matmul case", cfg.name, lin.name, cfg.tokens, flush=True)
        d = _dev(cfg.tokens, lin.out_features, lin.in_features, cfg.rank, "nf4", 80 + 10 * cfg_index + i)
        Y = q.deq_matmul_fwd(d["X"], d["Wd"], d["T"], d["B"])
        Yf = q.nf4_matmul_fwd(d["X"], d["w"], d["T"], d["B"])
        torch.cuda.synchronize()
        _same(Y, Yf, "Y " + lin.name)
        del Y, Yf
        dX = q.deq_matmul_dx(d["dY"], d["Wd"], d["G"], d["A"])
        dXf = q.nf4_matmul_dx(d["dY"], d["w"], d["G"], d["A"])
        torch.cuda.synchronize()
        _same(dX, dXf, "dX " + lin.name)
        del d, dX, dXf
        torch.cuda.empty_cache()
