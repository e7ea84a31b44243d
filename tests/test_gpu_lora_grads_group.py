"""GPU checks of qlora_lora_grads_group: dA and dB of several linears in one
contraction launch (plus one partial-sum launch) are bit-identical to one
qlora_lora_grads call per linear, whose results the other GPU tests compare
with the oracle."""

import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _member(M, N, K, r, seed, need_dA=True, need_dB=True):
    g = torch.Generator(DEV).manual_seed(seed)
    bf = torch.bfloat16
    return dict(X=torch.randn(M, K, device=DEV, generator=g).to(bf),
                dY=torch.randn(M, N, device=DEV, generator=g).to(bf),
                G=(torch.randn(M, r, device=DEV, generator=g) * 0.1).to(bf),
                T=(torch.randn(M, r, device=DEV, generator=g) * 0.1).to(bf),
                need_dA=need_dA, need_dB=need_dB)


def _check(members, name):
    print("lora grads group case", name, [(m["X"].shape[0], m["dY"].shape[1], m["X"].shape[1], m["G"].shape[1])
                                          for m in members], flush=True)
    for m in members:
        if m["X"].shape[0] == 0:   # M = 0: the outputs must be left as they were
            m["dA_out"] = torch.full((m["G"].shape[1], m["X"].shape[1]), 7, dtype=torch.int16, device=DEV).view(
                torch.bfloat16)
            m["dB_out"] = torch.full((m["dY"].shape[1], m["G"].shape[1]), 7, dtype=torch.int16, device=DEV).view(
                torch.bfloat16)
    grp = q.lora_grads_group(members)
    singles = [q.lora_grads(m["X"], m["dY"], m["G"], m["T"], need_dA=m["need_dA"], need_dB=m["need_dB"])
               for m in members]
    torch.cuda.synchronize()
    for i, ((ga, gb), (sa, sb)) in enumerate(zip(grp, singles)):
        if members[i]["X"].shape[0] == 0:
            assert bool((ga.view(torch.int16) == 7).all()) and bool((gb.view(torch.int16) == 7).all()), "M = 0 wrote"
            continue
        if ga is not None:
            assert torch.equal(ga.view(torch.int16), sa.view(torch.int16)), "%s member %d dA" % (name, i)
            assert torch.isfinite(ga.float()).all()
        if gb is not None:
            assert torch.equal(gb.view(torch.int16), sb.view(torch.int16)), "%s member %d dB" % (name, i)
            assert torch.isfinite(gb.float()).all()


def test_lora_grads_group_mixed_members():
    # ragged M, r not a multiple of 8 (padded operand), r = 96 (two column
    # chunks), members that need only dA or only dB, a member with M = 0
    members = [_member(1000, 256, 512, 64, 1), _member(777, 72, 136, 12, 2), _member(4096, 1024, 2048, 96, 3),
               _member(2048, 4096, 512, 8, 4, need_dB=False), _member(512, 264, 4096, 16, 5, need_dA=False),
               _member(0, 64, 64, 8, 6)]
    _check(members, "mixed")


def test_lora_grads_group_llama7b_layer():
    # the 7 linears of the 7B layer at 8192 tokens, r = 64: 14 products in one launch
    cfg = workloads.CONFIGS[1]
    members = [_member(cfg.tokens, lin.out_features, lin.in_features, cfg.rank, 100 + i)
               for i, lin in enumerate(cfg.linears)]
    _check(members, "llama7b")
