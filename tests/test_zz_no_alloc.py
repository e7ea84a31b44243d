"""qlora_linear_fwd_noalloc (the forward for callers that cannot allocate:
its scratch is the library's static per-GPU device array) against
qlora_linear_fwd with a caller workspace, through the C ABI: two calls in a
row on one stream, the second with a smaller input, then a large-M call whose
T lives in the scratch; Y and T must be bit-identical to the workspace entry
point's, and within the tolerance of the oracle.  A call that needs more
than the static scratch is rejected before launching anything."""

import ctypes

import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from bit_nf4_quantized_absmax_amd import _capi
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import DEV, as_f64, assert_close, guarded_like, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _case(M, N, K, r, seed):
    W = workloads.weight((N, K), seed)
    X = workloads.activation_bf16((M, K), seed + 1)
    A = workloads.lora_bf16((r, K), seed + 2)
    B = workloads.lora_bf16((N, r), seed + 3)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    return dict(W=W, X=X, A=A, B=B, w=w, st=w.struct(), Xd=to_dev_bf16(X), Ad=to_dev_bf16(A), Bd=to_dev_bf16(B),
                M=M, N=N, K=K, r=r, s=16.0 / r)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _noalloc(c, Y, T):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return q.lib().qlora_linear_fwd_noalloc(_ptr(c["Xd"]), c["M"], ctypes.byref(c["st"]), _ptr(c["Ad"]),
                                            _ptr(c["Bd"]), c["r"], c["s"], _ptr(Y), _ptr(T), stream)


def _with_workspace(c, Y, T):
    L = q.lib()
    nbytes = L.qlora_linear_workspace_bytes(c["M"], c["N"], c["K"], c["r"], 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.qlora_linear_fwd(_ptr(c["Xd"]), c["M"], ctypes.byref(c["st"]), _ptr(c["Ad"]), _ptr(c["Bd"]), c["r"],
                            c["s"], _ptr(Y), _ptr(T), _ptr(ws), nbytes, stream)
    return rc, ws


def test_noalloc_matches_workspace_entry_point():
    cases = [
        ("decode stream, M=64, 11008 x 4096", _case(64, 11008, 4096, 64, 2100), True),
        ("decode stream, M=5, 4096 x 4096 (smaller)", _case(5, 4096, 4096, 64, 2200), True),
        ("M=300, T in the scratch", _case(300, 512, 768, 32, 2300), False),
    ]
    outs = []
    for name, c, keep_t in cases:
        print("noalloc case", name, flush=True)
        gY, Y = guarded_like((c["M"], c["N"]), seed=len(outs))
        gT, T = guarded_like((c["M"], c["r"]), seed=10 + len(outs)) if keep_t else (None, None)
        assert _noalloc(c, Y, T) == _capi.QLORA_OK, name
        outs.append((name, c, gY, Y, gT, T))
    refs = []
    for name, c, _, _, _, T in outs:
        Y2 = torch.empty(c["M"], c["N"], dtype=torch.bfloat16, device=DEV)
        T2 = torch.empty(c["M"], c["r"], dtype=torch.bfloat16, device=DEV) if T is not None else None
        rc, ws = _with_workspace(c, Y2, T2)
        assert rc == _capi.QLORA_OK, name
        refs.append((Y2, T2, ws))
    torch.cuda.synchronize()
    for (name, c, gY, Y, gT, T), (Y2, T2, _) in zip(outs, refs):
        assert gY.intact() and (gT is None or gT.intact()), name + ": guard band"
        assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), name + ": Y differs from qlora_linear_fwd"
        if T is not None:
            assert torch.equal(T.view(torch.int16), T2.view(torch.int16)), name + ": T differs"
        wt = nf4.dequantize_q(nf4.quantize(c["W"])).reshape(c["N"], c["K"])
        Yr, _ = olin.linear_fwd(c["X"], wt, c["A"], c["B"], c["s"])
        assert_close(as_f64(Y), Yr, name + " Y vs oracle")


def test_noalloc_rejects_beyond_the_static_scratch():
    # T [70000, 128] bf16 = 17.1 MiB > 16 MiB, with no T_out to hold it
    M, N, K, r = 70000, 64, 64, 128
    c = _case(M, N, K, r, 2400)
    gY, Y = guarded_like((M, N), seed=30)
    assert _noalloc(c, Y, None) == _capi.QLORA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert gY.intact() and torch.all(gY.payload == 0xFF), "a rejected call wrote its output"
    assert "SCRATCH" in q.status_string(_capi.QLORA_ERR_SCRATCH_LIMIT)
    # with T_out the same call needs no scratch and runs
    gT, T = guarded_like((M, r), seed=31)
    assert _noalloc(c, Y, T) == _capi.QLORA_OK
    torch.cuda.synchronize()
    assert gY.intact() and gT.intact()
    assert not torch.isnan(Y.float()).any()
