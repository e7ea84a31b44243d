"""PyTorch-facing binding of libqlora_mi355x (argument marshalling only).

Torch provides device memory and streams; every step of the computation runs
in the HIP kernels behind the C ABI.  Tensors must be CUDA (HIP) tensors,
contiguous, with the dtypes named below; work is enqueued on the current
stream of the tensor's device.

Layer (automatone.win, "QLoRA paper explained", How it works; aiwiki.com.my,
"QLoRA", Key Concepts and Technology): frozen NF4 weight W [N, K] with double
-quantized constants, bf16 compute, LoRA pair A [r, K], B [N, r], scale
s = alpha / r:  Y = X deq(W)^T + s (X A^T) B^T.
"""

import ctypes
from dataclasses import dataclass

import torch

from ._capi import NF4WeightStruct, check, lib


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def nf4_sizes(n):
    pb, nb, nb2 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    check(lib().qlora_nf4_sizes(int(n), ctypes.byref(pb), ctypes.byref(nb), ctypes.byref(nb2)), "qlora_nf4_sizes")
    return pb.value, nb.value, nb2.value


Q4_TYPES = ("nf4", "fp4", "int4")   # 4-bit level tables; the index is qlora_q4_type


@dataclass
class NF4Weight:
    """A frozen weight [rows, cols] in NF4 with double-quantized constants.

    packed uint8 [ceil(n/2)], code8 uint8 [nb], c2 float32 [nb2], mean float32 [1].
    qtype names the 4-bit level table ("nf4", or "fp4" / "int4" for the
    comparison types; the rest of the format is the same).
    """
    packed: torch.Tensor
    code8: torch.Tensor
    c2: torch.Tensor
    mean: torch.Tensor
    rows: int
    cols: int
    qtype: str = "nf4"

    @property
    def shape(self):
        return (self.rows, self.cols)

    @property
    def device(self):
        return self.packed.device

    def struct(self):
        return NF4WeightStruct(self.packed.data_ptr(), self.code8.data_ptr(), self.c2.data_ptr(),
                               self.mean.data_ptr(), self.rows, self.cols, Q4_TYPES.index(self.qtype))

    @classmethod
    def empty(cls, rows, cols, device, qtype="nf4"):
        if qtype not in Q4_TYPES:
            raise ValueError("qtype must be one of %s" % (Q4_TYPES,))
        pb, nb, nb2 = nf4_sizes(rows * cols)
        return cls(torch.empty(pb, dtype=torch.uint8, device=device),
                   torch.empty(nb, dtype=torch.uint8, device=device),
                   torch.empty(nb2, dtype=torch.float32, device=device),
                   torch.empty(1, dtype=torch.float32, device=device), rows, cols, qtype)

    @classmethod
    def quantize(cls, W, qtype="nf4"):
        """Quantize a float32, bfloat16 or float16 [rows, cols] device tensor
        (qlora_quantize_nf4 / qlora_quantize_nf4_16) with the 4-bit level
        table `qtype` ("nf4", "fp4" or "int4")."""
        if W.dim() != 2:
            raise ValueError("W must be 2-D [out_features, in_features]")
        in16 = {torch.bfloat16: 1, torch.float16: 2}.get(W.dtype)
        if in16 is None:
            _need(W, torch.float32, "W")
        else:
            _need(W, W.dtype, "W")
        rows, cols = W.shape
        w = cls.empty(rows, cols, W.device, qtype)
        ws_bytes = lib().qlora_quantize_workspace_bytes(rows * cols)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=W.device)
        st = w.struct()
        if in16 is None:
            check(lib().qlora_quantize_nf4(_ptr(W), ctypes.byref(st), _ptr(ws), ws_bytes, _stream(W)),
                  "qlora_quantize_nf4")
        else:
            check(lib().qlora_quantize_nf4_16(_ptr(W), in16, ctypes.byref(st), _ptr(ws), ws_bytes, _stream(W)),
                  "qlora_quantize_nf4_16")
        return w

    def dequantize(self):
        """bf16 [rows, cols] copy of the weight (qlora_dequantize_nf4)."""
        out = torch.empty(self.rows, self.cols, dtype=torch.bfloat16, device=self.device)
        st = self.struct()
        check(lib().qlora_dequantize_nf4(ctypes.byref(st), _ptr(out), _stream(out)), "qlora_dequantize_nf4")
        return out

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in (self.packed, self.code8, self.c2, self.mean))


def _lin_checks(X, w, A, B, r_expect=None):
    N, K = w.rows, w.cols
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M, %d]" % K)
    _need(X, torch.bfloat16, "X")
    r = A.shape[0]
    _need(A, torch.bfloat16, "A", (r, K))
    _need(B, torch.bfloat16, "B", (N, r))
    return X.shape[0], N, K, r


def linear_fwd(X, w, A, B, scale, T_out=None, out=None, workspace=None):
    """Y = X deq(W)^T + scale (X A^T) B^T; returns (Y, T) with T = scale X A^T [M, r]."""
    M, N, K, r = _lin_checks(X, w, A, B)
    Y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", (M, N))
    T = T_out if T_out is not None else torch.empty(M, r, dtype=torch.bfloat16, device=X.device)
    _need(T, torch.bfloat16, "T", (M, r))
    ws_bytes = lib().qlora_linear_workspace_bytes(M, N, K, r, 0)
    ws = None
    if ws_bytes:
        ws = workspace if workspace is not None else torch.empty(ws_bytes, dtype=torch.uint8, device=X.device)
        if ws.numel() * ws.element_size() < ws_bytes:
            raise ValueError("workspace smaller than %d bytes" % ws_bytes)
    st = w.struct()
    check(lib().qlora_linear_fwd(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), _ptr(Y),
                                 _ptr(T), None if ws is None else _ptr(ws), ws_bytes, _stream(X)),
          "qlora_linear_fwd")
    return Y, T


def linear_fwd_group(linears, scale=None, workspace=None):
    """Forward of up to 8 independent linears sharing the token count M.

    `linears` is a sequence of (X, w, A, B, scale) or (X, w, A, B, scale, T_out,
    Y_out) tuples; returns the list of (Y, T).  Same results as calling
    linear_fwd on each; in the decode regime the group costs two launches."""
    from ._capi import LinearDescStruct
    if not 1 <= len(linears) <= 8:
        raise ValueError("a group holds 1 to 8 linears")
    M = None
    outs, descs, structs = [], [], []
    for item in linears:
        X, w, A, B, sc = item[:5]
        T_out = item[5] if len(item) > 5 else None
        Y_out = item[6] if len(item) > 6 else None
        m, N, K, r = _lin_checks(X, w, A, B)
        if M is None:
            M = m
        elif m != M:
            raise ValueError("all linears of a group share M")
        Y = Y_out if Y_out is not None else torch.empty(m, N, dtype=torch.bfloat16, device=X.device)
        _need(Y, torch.bfloat16, "Y", (m, N))
        T = T_out if T_out is not None else torch.empty(m, r, dtype=torch.bfloat16, device=X.device)
        _need(T, torch.bfloat16, "T", (m, r))
        st = w.struct()
        structs.append(st)
        descs.append(LinearDescStruct(X.data_ptr(), ctypes.pointer(st), A.data_ptr(), B.data_ptr(), r, float(sc),
                                      Y.data_ptr(), T.data_ptr()))
        outs.append((Y, T))
    arr = (LinearDescStruct * len(descs))(*descs)
    ws_bytes = lib().qlora_linear_group_workspace_bytes(len(descs), arr, M)
    ws = None
    if ws_bytes:
        ws = workspace if workspace is not None else torch.empty(ws_bytes, dtype=torch.uint8,
                                                                  device=linears[0][0].device)
        if ws.numel() * ws.element_size() < ws_bytes:
            raise ValueError("workspace smaller than %d bytes" % ws_bytes)
    check(lib().qlora_linear_fwd_group(len(descs), arr, M, None if ws is None else _ptr(ws), ws_bytes,
                                       _stream(linears[0][0])), "qlora_linear_fwd_group")
    return outs


def linear_bwd(dY, X, T, w, A, B, scale, need_dX=True, need_dA=True, need_dB=True, workspace=None):
    """Returns (dX, dA, dB) (None where not requested); T = scale X A^T as
    returned by linear_fwd, or None (recomputed)."""
    M, N, K, r = _lin_checks(X, w, A, B)
    _need(dY, torch.bfloat16, "dY", (M, N))
    if T is not None:
        _need(T, torch.bfloat16, "T", (M, r))
    dev = X.device
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev) if need_dX else None
    dA = torch.empty(r, K, dtype=torch.bfloat16, device=dev) if need_dA else None
    dB = torch.empty(N, r, dtype=torch.bfloat16, device=dev) if need_dB else None
    ws_bytes = lib().qlora_linear_workspace_bytes(M, N, K, r, 1)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    st = w.struct()
    check(lib().qlora_linear_bwd(_ptr(dY), _ptr(X), _ptr(T), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
                                 float(scale), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes, _stream(X)),
          "qlora_linear_bwd")
    return dX, dA, dB


# ---- the individual steps ------------------------------------------------------

def lora_down(X, A, scale, out=None):
    """T = scale X A^T."""
    M, K = X.shape
    r = A.shape[0]
    _need(X, torch.bfloat16, "X")
    _need(A, torch.bfloat16, "A", (r, K))
    T = out if out is not None else torch.empty(M, r, dtype=torch.bfloat16, device=X.device)
    check(lib().qlora_lora_down(_ptr(X), M, K, _ptr(A), r, float(scale), _ptr(T), _stream(X)), "qlora_lora_down")
    return T


def _arrays(ptrs, rs, scales=None):
    n = len(ptrs)
    return ((ctypes.c_void_p * n)(*ptrs), (ctypes.c_int32 * n)(*rs),
            None if scales is None else (ctypes.c_float * n)(*[float(s) for s in scales]))


def lora_down_shared(X, As, scales, outs=None):
    """[T_i = scale_i X A_i^T] for linears that share X (qlora_lora_down_shared):
    one launch, bit-identical to lora_down per linear."""
    M, K = X.shape
    _need(X, torch.bfloat16, "X")
    if not 1 <= len(As) <= 8 or len(scales) != len(As):
        raise ValueError("1 to 8 members, one scale each")
    Ts = []
    for i, A in enumerate(As):
        _need(A, torch.bfloat16, "A", (A.shape[0], K))
        T = outs[i] if outs is not None else torch.empty(M, A.shape[0], dtype=torch.bfloat16, device=X.device)
        _need(T, torch.bfloat16, "T", (M, A.shape[0]))
        Ts.append(T)
    pa, ra, sa = _arrays([A.data_ptr() for A in As], [A.shape[0] for A in As], scales)
    pt, _, _ = _arrays([T.data_ptr() for T in Ts], [1] * len(Ts))
    check(lib().qlora_lora_down_shared(_ptr(X), M, K, len(As), pa, ra, sa, pt, _stream(X)), "qlora_lora_down_shared")
    return Ts


def lora_dA_shared(X, Gs, outs=None, workspace=None):
    """[dA_i = G_i^T X] for linears that share X (qlora_lora_dA_shared; G_i
    carries the scale): one launch (+ the split sums), bit-identical to the dA
    of lora_grads per linear."""
    M, K = X.shape
    _need(X, torch.bfloat16, "X")
    if not 1 <= len(Gs) <= 8:
        raise ValueError("1 to 8 members")
    dAs = []
    for i, G in enumerate(Gs):
        _need(G, torch.bfloat16, "G", (M, G.shape[1]))
        dA = outs[i] if outs is not None else torch.empty(G.shape[1], K, dtype=torch.bfloat16, device=X.device)
        _need(dA, torch.bfloat16, "dA", (G.shape[1], K))
        dAs.append(dA)
    pg, ra, _ = _arrays([G.data_ptr() for G in Gs], [G.shape[1] for G in Gs])
    pd, _, _ = _arrays([dA.data_ptr() for dA in dAs], [1] * len(dAs))
    ws_bytes = lib().qlora_lora_dA_shared_workspace_bytes(M, K, len(Gs), ra)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=X.device)
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError("workspace smaller than %d bytes" % ws_bytes)
    check(lib().qlora_lora_dA_shared(_ptr(X), M, K, len(Gs), pg, ra, pd, _ptr(ws), ws_bytes, _stream(X)),
          "qlora_lora_dA_shared")
    return dAs


def dropout_mask(X, p, seed):
    """(X_d, keep): the LoRA input with dropout p (qlora_dropout_mask); keep is
    int32 [M, K / 32], bit k % 32 of word k / 32."""
    M, K = X.shape
    _need(X, torch.bfloat16, "X")
    Xd = torch.empty_like(X)
    keep = torch.empty(M, K // 32, dtype=torch.int32, device=X.device)
    check(lib().qlora_dropout_mask(_ptr(X), M, K, float(p), int(seed), _ptr(Xd), _ptr(keep), _stream(X)),
          "qlora_dropout_mask")
    return Xd, keep


def dropout_apply(X, keep):
    """X_d from X and a keep mask (qlora_dropout_apply)."""
    M, K = X.shape
    _need(X, torch.bfloat16, "X")
    _need(keep, torch.int32, "keep", (M, K // 32))
    Xd = torch.empty_like(X)
    check(lib().qlora_dropout_apply(_ptr(X), M, K, _ptr(keep), _ptr(Xd), _stream(X)), "qlora_dropout_apply")
    return Xd


def nf4_matmul_dx_dropout(dY, w, G, A, keep, out=None):
    """dX = dY deq(W) + (G A) * keep (G = s_eff dY B)."""
    M = dY.shape[0]
    r = A.shape[0]
    _need(dY, torch.bfloat16, "dY", (M, w.rows))
    _need(G, torch.bfloat16, "G", (M, r))
    _need(A, torch.bfloat16, "A", (r, w.cols))
    _need(keep, torch.int32, "keep", (M, w.cols // 32))
    dX = out if out is not None else torch.empty(M, w.cols, dtype=torch.bfloat16, device=dY.device)
    st = w.struct()
    check(lib().qlora_nf4_matmul_dx_dropout(_ptr(dY), M, ctypes.byref(st), _ptr(G), _ptr(A), r, _ptr(keep), _ptr(dX),
                                            _stream(dY)), "qlora_nf4_matmul_dx_dropout")
    return dX


def dropout_scale(scale, p):
    """s_eff = fl32(s / (1 - p)), the LoRA scale with inverted dropout."""
    import numpy as np
    return float(np.float32(float(np.float32(scale)) / (1.0 - float(np.float32(p)))))


def linear_fwd_dropout(X, w, A, B, scale, p, seed, T_out=None, out=None, workspace=None):
    """Forward with LoRA dropout: returns (Y, T, keep)."""
    M, N, K, r = _lin_checks(X, w, A, B)
    Y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    T = T_out if T_out is not None else torch.empty(M, r, dtype=torch.bfloat16, device=X.device)
    keep = torch.empty(M, K // 32, dtype=torch.int32, device=X.device)
    ws_bytes = lib().qlora_linear_dropout_workspace_bytes(M, N, K, r, 0)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=X.device)
    st = w.struct()
    check(lib().qlora_linear_fwd_dropout(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), float(p),
                                         int(seed), _ptr(Y), _ptr(T), _ptr(keep), _ptr(ws), ws_bytes, _stream(X)),
          "qlora_linear_fwd_dropout")
    return Y, T, keep


def linear_bwd_dropout(dY, X, T, w, A, B, scale, p, keep, need_dX=True, need_dA=True, need_dB=True,
                       workspace=None):
    """Backward with LoRA dropout given the forward's keep mask: (dX, dA, dB)."""
    M, N, K, r = _lin_checks(X, w, A, B)
    _need(dY, torch.bfloat16, "dY", (M, N))
    _need(keep, torch.int32, "keep", (M, K // 32))
    dev = X.device
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev) if need_dX else None
    dA = torch.empty(r, K, dtype=torch.bfloat16, device=dev) if need_dA else None
    dB = torch.empty(N, r, dtype=torch.bfloat16, device=dev) if need_dB else None
    ws_bytes = lib().qlora_linear_dropout_workspace_bytes(M, N, K, r, 1)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    st = w.struct()
    check(lib().qlora_linear_bwd_dropout(_ptr(dY), _ptr(X), _ptr(T), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
                                         float(scale), float(p), _ptr(keep), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                         ws_bytes, _stream(X)), "qlora_linear_bwd_dropout")
    return dX, dA, dB


def nf4_matmul_fwd(X, w, T, B, out=None):
    """Y = X deq(W)^T + T B^T (T = scale X A^T)."""
    M = X.shape[0]
    r = B.shape[1]
    _need(X, torch.bfloat16, "X", (M, w.cols))
    _need(T, torch.bfloat16, "T", (M, r))
    _need(B, torch.bfloat16, "B", (w.rows, r))
    Y = out if out is not None else torch.empty(M, w.rows, dtype=torch.bfloat16, device=X.device)
    st = w.struct()
    check(lib().qlora_nf4_matmul_fwd(_ptr(X), M, ctypes.byref(st), _ptr(T), _ptr(B), r, _ptr(Y), _stream(X)),
          "qlora_nf4_matmul_fwd")
    return Y


def lora_grad_in(dY, B, scale, out=None, workspace=None):
    """G = scale dY B."""
    M, N = dY.shape
    r = B.shape[1]
    _need(dY, torch.bfloat16, "dY")
    _need(B, torch.bfloat16, "B", (N, r))
    G = out if out is not None else torch.empty(M, r, dtype=torch.bfloat16, device=dY.device)
    ws_bytes = lib().qlora_lora_grad_in_workspace_bytes(N, r)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dY.device)
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError("workspace smaller than %d bytes" % ws_bytes)
    check(lib().qlora_lora_grad_in(_ptr(dY), M, N, _ptr(B), r, float(scale), _ptr(G), _ptr(ws), ws_bytes,
                                   _stream(dY)), "qlora_lora_grad_in")
    return G


def nf4_matmul_dx(dY, w, G, A, out=None):
    """dX = dY deq(W) + G A (G = scale dY B)."""
    M = dY.shape[0]
    r = A.shape[0]
    _need(dY, torch.bfloat16, "dY", (M, w.rows))
    _need(G, torch.bfloat16, "G", (M, r))
    _need(A, torch.bfloat16, "A", (r, w.cols))
    dX = out if out is not None else torch.empty(M, w.cols, dtype=torch.bfloat16, device=dY.device)
    st = w.struct()
    check(lib().qlora_nf4_matmul_dx(_ptr(dY), M, ctypes.byref(st), _ptr(G), _ptr(A), r, _ptr(dX), _stream(dY)),
          "qlora_nf4_matmul_dx")
    return dX


def lora_grads(X, dY, G, T, need_dA=True, need_dB=True, workspace=None):
    """dA = G^T X, dB = dY^T T (G and T carry the scale)."""
    M, K = X.shape
    N = dY.shape[1]
    r = G.shape[1]
    dev = X.device
    dA = torch.empty(r, K, dtype=torch.bfloat16, device=dev) if need_dA else None
    dB = torch.empty(N, r, dtype=torch.bfloat16, device=dev) if need_dB else None
    ws_bytes = lib().qlora_lora_grads_workspace_bytes(M, N, K, r)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    check(lib().qlora_lora_grads(_ptr(X), _ptr(dY), _ptr(G), _ptr(T), M, N, K, r, _ptr(dA), _ptr(dB), _ptr(ws),
                                 ws_bytes, _stream(X)), "qlora_lora_grads")
    return dA, dB


# ---- autograd ----------------------------------------------------------------

class QLoRALinearFn(torch.autograd.Function):
    """Y = X deq(W)^T + scale (X A^T) B^T with gradients for X, A and B only."""

    @staticmethod
    def forward(ctx, X, A, B, w, scale):
        Y, T = linear_fwd(X, w, A, B, scale)
        ctx.save_for_backward(X, A, B, T)
        ctx.w, ctx.scale = w, scale
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, A, B, T = ctx.saved_tensors
        dX, dA, dB = linear_bwd(dY.contiguous(), X, T, ctx.w, A, B, ctx.scale,
                                need_dX=ctx.needs_input_grad[0], need_dA=ctx.needs_input_grad[1],
                                need_dB=ctx.needs_input_grad[2])
        return dX, dA, dB, None, None


class QLoRALinear(torch.nn.Module):
    """A linear layer with a frozen NF4 base weight and a trainable LoRA pair.

    No bias and no dropout (the adapter configuration uses bias="none").
    """

    def __init__(self, weight_fp32, r, alpha, lora_A=None, lora_B=None):
        super().__init__()
        self.w = NF4Weight.quantize(weight_fp32.contiguous())
        N, K = self.w.shape
        dev = weight_fp32.device
        self.r = int(r)
        self.scale = float(torch.tensor(alpha, dtype=torch.float32) / torch.tensor(r, dtype=torch.float32))
        self.lora_A = torch.nn.Parameter(lora_A if lora_A is not None else
                                         torch.zeros(r, K, dtype=torch.bfloat16, device=dev))
        self.lora_B = torch.nn.Parameter(lora_B if lora_B is not None else
                                         torch.zeros(N, r, dtype=torch.bfloat16, device=dev))

    def forward(self, x):
        lead = x.shape[:-1]
        y = QLoRALinearFn.apply(x.reshape(-1, x.shape[-1]).contiguous(), self.lora_A, self.lora_B, self.w,
                                self.scale)
        return y.reshape(*lead, y.shape[-1])
