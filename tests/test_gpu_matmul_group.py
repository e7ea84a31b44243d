"""GPU checks of qlora_nf4_matmul_fwd_group: forward products that share M in
one launch over their concatenated tile grids are bit-identical to one
qlora_nf4_matmul_fwd call each (whose results the other GPU tests compare
with the oracle)."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _member(M, N, K, r, qtype, seed):
    g = torch.Generator(DEV).manual_seed(seed)
    bf = torch.bfloat16
    W = torch.randn(N, K, device=DEV, generator=g) * 0.02
    return dict(X=torch.randn(M, K, device=DEV, generator=g).to(bf), w=q.NF4Weight.quantize(W, qtype),
                T=(torch.randn(M, r, device=DEV, generator=g) * 0.1).to(bf),
                B=(torch.randn(N, r, device=DEV, generator=g) * 0.01).to(bf))


def _check(members, name):
    print("matmul group case", name, [(m["X"].shape[0], m["w"].rows, m["w"].cols, m["B"].shape[1], m["w"].qtype)
                                      for m in members], flush=True)
    grp = q.nf4_matmul_fwd_group(members)
    singles = [q.nf4_matmul_fwd(m["X"], m["w"], m["T"], m["B"]) for m in members]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(grp, singles)):
        assert torch.isfinite(a.float()).all(), "%s member %d not finite" % (name, i)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "%s member %d" % (name, i)


def test_matmul_fwd_group_llama7b_gate_up():
    cfg = workloads.CONFIGS[1]
    lins = [l for l in cfg.linears if l.name in ("gate_proj", "up_proj")]
    assert len(lins) == 2
    _check([_member(cfg.tokens, l.out_features, l.in_features, cfg.rank, "nf4", 50 + i) for i, l in enumerate(lins)],
           "gate_up")


def test_matmul_fwd_group_mixed():
    # ragged M (several row tiles, a partial one), mixed N / K, r = 12 (not a
    # multiple of 8) and r = 96 (two LoRA steps), the three 4-bit tables
    members = [_member(300, 520, 1024, 64, "nf4", 1), _member(300, 1000, 640, 12, "fp4", 2),
               _member(300, 264, 2048, 96, "int4", 3), _member(300, 8, 64, 8, "nf4", 4)]
    _check(members, "mixed")


def test_matmul_fwd_group_decode_regime():
    # M <= 64: members take the decode-regime route one call each
    members = [_member(16, 4096, 4096, 64, "nf4", 11), _member(16, 1024, 4096, 64, "nf4", 12)]
    _check(members, "decode")
