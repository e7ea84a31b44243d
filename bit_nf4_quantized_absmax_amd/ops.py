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

from ._capi import DeqMatmulFwdDescStruct, LoraGradsDescStruct, MatmulFwdDescStruct, NF4WeightStruct, check, lib


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


def _workspace(workspace, need, device):
    """(tensor or None, bytes passed to the C ABI): the caller's workspace, or
    a fresh one of `need` bytes.  The byte count handed to the library is the
    buffer's real size, so the C-side QLORA_ERR_WORKSPACE check guards it."""
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a tensor")
    have = workspace.numel() * workspace.element_size()
    if have < need:
        raise ValueError("workspace holds %d bytes, %d needed" % (have, need))
    if workspace.device.type != "cuda":
        raise ValueError("workspace must be on a GPU device")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace, have


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


def quantize_group(Ws, qtypes=None):
    """Quantize up to 8 device tensors [rows, cols] of one dtype (float32,
    bfloat16 or float16) in one call (qlora_quantize_nf4_group: two launches
    for the whole group).  qtypes: one 4-bit table name per tensor (default
    all "nf4").  Returns one NF4Weight per tensor, bit-identical to
    NF4Weight.quantize of each."""
    Ws = list(Ws)
    if not 1 <= len(Ws) <= 8:
        raise ValueError("a group holds 1 to 8 weights")
    qtypes = list(qtypes) if qtypes is not None else ["nf4"] * len(Ws)
    if len(qtypes) != len(Ws):
        raise ValueError("one qtype per weight")
    dtype = Ws[0].dtype
    in_type = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}.get(dtype)
    if in_type is None:
        raise ValueError("W must be float32, bfloat16 or float16")
    for i, W in enumerate(Ws):
        _need(W, dtype, "Ws[%d]" % i)
        if W.dim() != 2:
            raise ValueError("Ws[%d] must be 2-D [out_features, in_features]" % i)
    outs = [NF4Weight.empty(W.shape[0], W.shape[1], W.device, qt) for W, qt in zip(Ws, qtypes)]
    sts = (NF4WeightStruct * len(Ws))(*[w.struct() for w in outs])
    ws_bytes = lib().qlora_quantize_group_workspace_bytes(len(Ws), sts)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=Ws[0].device)
    ptrs = (ctypes.c_void_p * len(Ws))(*[_ptr(W) for W in Ws])
    check(lib().qlora_quantize_nf4_group(len(Ws), ptrs, in_type, sts, _ptr(ws), ws_bytes, _stream(Ws[0])),
          "qlora_quantize_nf4_group")
    return outs


def dequantize_group(weights, outs=None):
    """bf16 copies of up to 8 NF4Weights in one launch (qlora_dequantize_nf4_group),
    into `outs` (bf16 [rows, cols] each) when given."""
    weights = list(weights)
    if not 1 <= len(weights) <= 8:
        raise ValueError("a group holds 1 to 8 weights")
    if outs is None:
        outs = [torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device=w.device) for w in weights]
    else:
        outs = list(outs)
        if len(outs) != len(weights):
            raise ValueError("one output per weight")
        for i, (w, o) in enumerate(zip(weights, outs)):
            _need(o, torch.bfloat16, "outs[%d]" % i, (w.rows, w.cols))
    sts = (NF4WeightStruct * len(weights))(*[w.struct() for w in weights])
    ptrs = (ctypes.c_void_p * len(weights))(*[_ptr(o) for o in outs])
    check(lib().qlora_dequantize_nf4_group(len(weights), sts, ptrs, _stream(outs[0])), "qlora_dequantize_nf4_group")
    return outs


def nf4_matmul_fwd_group(members):
    """Y_i = X_i deq(W_i)^T + T_i B_i^T for up to 4 products sharing M in one
    launch (qlora_nf4_matmul_fwd_group).  members: sequence of dicts with X,
    w (NF4Weight), T, B and optional out.  Returns [Y, ...], bit-identical to
    nf4_matmul_fwd of each."""
    members = list(members)
    if not 1 <= len(members) <= 4:
        raise ValueError("a group holds 1 to 4 products")
    descs, outs, structs = [], [], []
    for i, mb in enumerate(members):
        X, w, T, B = mb["X"], mb["w"], mb["T"], mb["B"]
        M = _mat(X, "members[%d].X" % i)[0]
        r = _mat(B, "members[%d].B" % i)[1]
        _need(X, torch.bfloat16, "members[%d].X" % i, (M, w.cols))
        _need(T, torch.bfloat16, "members[%d].T" % i, (M, r))
        _need(B, torch.bfloat16, "members[%d].B" % i, (w.rows, r))
        Y = _out(mb.get("out"), (M, w.rows), X.device, "members[%d].out" % i)
        structs.append(w.struct())
        outs.append(Y)
        descs.append((X, M, T, B, r, Y))
    arr = (MatmulFwdDescStruct * len(descs))(*[
        MatmulFwdDescStruct(X.data_ptr(), M, ctypes.pointer(st), T.data_ptr(), B.data_ptr(), r, Y.data_ptr())
        for (X, M, T, B, r, Y), st in zip(descs, structs)])
    check(lib().qlora_nf4_matmul_fwd_group(len(descs), arr, _stream(members[0]["X"])), "qlora_nf4_matmul_fwd_group")
    return outs


def _mat(t, name, dtype=torch.bfloat16):
    """A 2-D contiguous device tensor of `dtype`; returns its shape."""
    _need(t, dtype, name)
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    return tuple(t.shape)


def _out(t, shape, device, name, dtype=torch.bfloat16):
    """The caller's output tensor (checked) or a fresh one."""
    if t is None:
        return torch.empty(*shape, dtype=dtype, device=device)
    _need(t, dtype, name, shape)
    return t


def _lin_checks(X, w, A, B):
    N, K = w.rows, w.cols
    _need(X, torch.bfloat16, "X")
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M, %d]" % K)
    _need(A, torch.bfloat16, "A")
    if A.dim() != 2:
        raise ValueError("A must be 2-D [r, K]")
    r = A.shape[0]
    _need(A, torch.bfloat16, "A", (r, K))
    _need(B, torch.bfloat16, "B", (N, r))
    return X.shape[0], N, K, r


def linear_fwd(X, w, A, B, scale, T_out=None, out=None, workspace=None):
    """Y = X deq(W)^T + scale (X A^T) B^T; returns (Y, T) with T = scale X A^T [M, r]."""
    M, N, K, r = _lin_checks(X, w, A, B)
    Y = _out(out, (M, N), X.device, "Y")
    T = _out(T_out, (M, r), X.device, "T")
    ws, ws_bytes = _workspace(workspace, lib().qlora_linear_workspace_bytes(M, N, K, r, 0), X.device)
    st = w.struct()
    check(lib().qlora_linear_fwd(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), _ptr(Y),
                                 _ptr(T), _ptr(ws), ws_bytes, _stream(X)), "qlora_linear_fwd")
    return Y, T


def linear_fwd_group(linears, workspace=None):
    """Forward of up to 8 independent linears sharing the token count M.

    `linears` is a sequence of (X, w, A, B, scale) or (X, w, A, B, scale, T_out,
    Y_out) tuples; returns the list of (Y, T).  Same results as calling
    linear_fwd on each (bit for bit except on the streaming decode route,
    within the tolerance there); in the decode regime the group costs the
    launches of one call."""
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
        Y = _out(Y_out, (m, N), X.device, "Y")
        T = _out(T_out, (m, r), X.device, "T")
        st = w.struct()
        structs.append(st)
        descs.append(LinearDescStruct(X.data_ptr(), ctypes.pointer(st), A.data_ptr(), B.data_ptr(), r, float(sc),
                                      Y.data_ptr(), T.data_ptr()))
        outs.append((Y, T))
    arr = (LinearDescStruct * len(descs))(*descs)
    dev = linears[0][0].device
    ws, ws_bytes = _workspace(workspace, lib().qlora_linear_group_workspace_bytes(len(descs), arr, M), dev)
    check(lib().qlora_linear_fwd_group(len(descs), arr, M, _ptr(ws), ws_bytes, _stream(linears[0][0])),
          "qlora_linear_fwd_group")
    return outs


def linear_bwd(dY, X, T, w, A, B, scale, need_dX=True, need_dA=True, need_dB=True, workspace=None,
               dX_out=None, dA_out=None, dB_out=None):
    """Returns (dX, dA, dB) (None where not requested); T = scale X A^T as
    returned by linear_fwd, or None (recomputed)."""
    M, N, K, r = _lin_checks(X, w, A, B)
    _need(dY, torch.bfloat16, "dY", (M, N))
    if T is not None:
        _need(T, torch.bfloat16, "T", (M, r))
    dev = X.device
    dX = _out(dX_out, (M, K), dev, "dX") if need_dX else None
    dA = _out(dA_out, (r, K), dev, "dA") if need_dA else None
    dB = _out(dB_out, (N, r), dev, "dB") if need_dB else None
    ws, ws_bytes = _workspace(workspace, lib().qlora_linear_workspace_bytes(M, N, K, r, 1), dev)
    st = w.struct()
    check(lib().qlora_linear_bwd(_ptr(dY), _ptr(X), _ptr(T), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
                                 float(scale), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes, _stream(X)),
          "qlora_linear_bwd")
    return dX, dA, dB


# ---- the individual steps ------------------------------------------------------

def lora_down(X, A, scale, out=None):
    """T = scale X A^T."""
    M, K = _mat(X, "X")
    r = _mat(A, "A")[0]
    _need(A, torch.bfloat16, "A", (r, K))
    T = _out(out, (M, r), X.device, "T")
    check(lib().qlora_lora_down(_ptr(X), M, K, _ptr(A), r, float(scale), _ptr(T), _stream(X)), "qlora_lora_down")
    return T


def _arrays(ptrs, rs, scales=None):
    n = len(ptrs)
    return ((ctypes.c_void_p * n)(*ptrs), (ctypes.c_int32 * n)(*rs),
            None if scales is None else (ctypes.c_float * n)(*[float(s) for s in scales]))


def lora_down_shared(X, As, scales, outs=None):
    """[T_i = scale_i X A_i^T] for linears that share X (qlora_lora_down_shared):
    one launch, bit-identical to lora_down per linear."""
    M, K = _mat(X, "X")
    if not 1 <= len(As) <= 8 or len(scales) != len(As):
        raise ValueError("1 to 8 members, one scale each")
    if outs is not None and len(outs) != len(As):
        raise ValueError("one output per member")
    Ts = []
    for i, A in enumerate(As):
        r = _mat(A, "A")[0]
        _need(A, torch.bfloat16, "A", (r, K))
        Ts.append(_out(None if outs is None else outs[i], (M, r), X.device, "T"))
    pa, ra, sa = _arrays([A.data_ptr() for A in As], [A.shape[0] for A in As], scales)
    pt, _, _ = _arrays([T.data_ptr() for T in Ts], [1] * len(Ts))
    check(lib().qlora_lora_down_shared(_ptr(X), M, K, len(As), pa, ra, sa, pt, _stream(X)), "qlora_lora_down_shared")
    return Ts


def lora_dA_shared(X, Gs, outs=None, workspace=None):
    """[dA_i = G_i^T X] for linears that share X (qlora_lora_dA_shared; G_i
    carries the scale): one launch (+ the split sums), bit-identical to the dA
    of lora_grads per linear."""
    M, K = _mat(X, "X")
    if not 1 <= len(Gs) <= 8:
        raise ValueError("1 to 8 members")
    if outs is not None and len(outs) != len(Gs):
        raise ValueError("one output per member")
    dAs = []
    for i, G in enumerate(Gs):
        r = _mat(G, "G")[1]
        _need(G, torch.bfloat16, "G", (M, r))
        dAs.append(_out(None if outs is None else outs[i], (r, K), X.device, "dA"))
    pg, ra, _ = _arrays([G.data_ptr() for G in Gs], [G.shape[1] for G in Gs])
    pd, _, _ = _arrays([dA.data_ptr() for dA in dAs], [1] * len(dAs))
    ws, ws_bytes = _workspace(workspace, lib().qlora_lora_dA_shared_workspace_bytes(M, K, len(Gs), ra), X.device)
    check(lib().qlora_lora_dA_shared(_ptr(X), M, K, len(Gs), pg, ra, pd, _ptr(ws), ws_bytes, _stream(X)),
          "qlora_lora_dA_shared")
    return dAs


def dropout_mask(X, p, seed, out=None, keep_out=None):
    """(X_d, keep): the LoRA input with dropout p (qlora_dropout_mask); keep is
    int32 [M, K / 32], bit k % 32 of word k / 32."""
    M, K = _mat(X, "X")
    Xd = _out(out, (M, K), X.device, "X_d")
    keep = _out(keep_out, (M, K // 32), X.device, "keep", torch.int32)
    check(lib().qlora_dropout_mask(_ptr(X), M, K, float(p), int(seed), _ptr(Xd), _ptr(keep), _stream(X)),
          "qlora_dropout_mask")
    return Xd, keep


def dropout_apply(X, keep, out=None):
    """X_d from X and a keep mask (qlora_dropout_apply)."""
    M, K = _mat(X, "X")
    _need(keep, torch.int32, "keep", (M, K // 32))
    Xd = _out(out, (M, K), X.device, "X_d")
    check(lib().qlora_dropout_apply(_ptr(X), M, K, _ptr(keep), _ptr(Xd), _stream(X)), "qlora_dropout_apply")
    return Xd


def nf4_matmul_dx_dropout(dY, w, G, A, keep, out=None):
    """dX = dY deq(W) + (G A) * keep (G = s_eff dY B)."""
    M = _mat(dY, "dY")[0]
    r = _mat(A, "A")[0]
    _need(dY, torch.bfloat16, "dY", (M, w.rows))
    _need(G, torch.bfloat16, "G", (M, r))
    _need(A, torch.bfloat16, "A", (r, w.cols))
    _need(keep, torch.int32, "keep", (M, w.cols // 32))
    dX = _out(out, (M, w.cols), dY.device, "dX")
    st = w.struct()
    check(lib().qlora_nf4_matmul_dx_dropout(_ptr(dY), M, ctypes.byref(st), _ptr(G), _ptr(A), r, _ptr(keep), _ptr(dX),
                                            _stream(dY)), "qlora_nf4_matmul_dx_dropout")
    return dX


def linear_fwd_dropout(X, w, A, B, scale, p, seed, T_out=None, out=None, keep_out=None, workspace=None):
    """Forward with LoRA dropout: returns (Y, T, keep)."""
    M, N, K, r = _lin_checks(X, w, A, B)
    Y = _out(out, (M, N), X.device, "Y")
    T = _out(T_out, (M, r), X.device, "T")
    keep = _out(keep_out, (M, K // 32), X.device, "keep", torch.int32)
    ws, ws_bytes = _workspace(workspace, lib().qlora_linear_dropout_workspace_bytes(M, N, K, r, 0), X.device)
    st = w.struct()
    check(lib().qlora_linear_fwd_dropout(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), float(p),
                                         int(seed), _ptr(Y), _ptr(T), _ptr(keep), _ptr(ws), ws_bytes, _stream(X)),
          "qlora_linear_fwd_dropout")
    return Y, T, keep


def linear_bwd_dropout(dY, X, T, w, A, B, scale, p, keep, need_dX=True, need_dA=True, need_dB=True,
                       workspace=None, dX_out=None, dA_out=None, dB_out=None):
    """Backward with LoRA dropout given the forward's keep mask: (dX, dA, dB);
    T as returned by linear_fwd_dropout, or None (recomputed)."""
    M, N, K, r = _lin_checks(X, w, A, B)
    _need(dY, torch.bfloat16, "dY", (M, N))
    _need(keep, torch.int32, "keep", (M, K // 32))
    if T is not None:
        _need(T, torch.bfloat16, "T", (M, r))
    dev = X.device
    dX = _out(dX_out, (M, K), dev, "dX") if need_dX else None
    dA = _out(dA_out, (r, K), dev, "dA") if need_dA else None
    dB = _out(dB_out, (N, r), dev, "dB") if need_dB else None
    ws, ws_bytes = _workspace(workspace, lib().qlora_linear_dropout_workspace_bytes(M, N, K, r, 1), dev)
    st = w.struct()
    check(lib().qlora_linear_bwd_dropout(_ptr(dY), _ptr(X), _ptr(T), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
                                         float(scale), float(p), _ptr(keep), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                         ws_bytes, _stream(X)), "qlora_linear_bwd_dropout")
    return dX, dA, dB


def nf4_matmul_fwd(X, w, T, B, out=None):
    """Y = X deq(W)^T + T B^T (T = scale X A^T)."""
    M = _mat(X, "X")[0]
    r = _mat(B, "B")[1]
    _need(X, torch.bfloat16, "X", (M, w.cols))
    _need(T, torch.bfloat16, "T", (M, r))
    _need(B, torch.bfloat16, "B", (w.rows, r))
    Y = _out(out, (M, w.rows), X.device, "Y")
    st = w.struct()
    check(lib().qlora_nf4_matmul_fwd(_ptr(X), M, ctypes.byref(st), _ptr(T), _ptr(B), r, _ptr(Y), _stream(X)),
          "qlora_nf4_matmul_fwd")
    return Y


def lora_grad_in(dY, B, scale, out=None, workspace=None):
    """G = scale dY B."""
    M, N = _mat(dY, "dY")
    r = _mat(B, "B")[1]
    _need(B, torch.bfloat16, "B", (N, r))
    G = _out(out, (M, r), dY.device, "G")
    ws, ws_bytes = _workspace(workspace, lib().qlora_lora_grad_in_workspace_bytes(N, r), dY.device)
    check(lib().qlora_lora_grad_in(_ptr(dY), M, N, _ptr(B), r, float(scale), _ptr(G), _ptr(ws), ws_bytes,
                                   _stream(dY)), "qlora_lora_grad_in")
    return G


def nf4_matmul_dx(dY, w, G, A, out=None):
    """dX = dY deq(W) + G A (G = scale dY B)."""
    M = _mat(dY, "dY")[0]
    r = _mat(A, "A")[0]
    _need(dY, torch.bfloat16, "dY", (M, w.rows))
    _need(G, torch.bfloat16, "G", (M, r))
    _need(A, torch.bfloat16, "A", (r, w.cols))
    dX = _out(out, (M, w.cols), dY.device, "dX")
    st = w.struct()
    check(lib().qlora_nf4_matmul_dx(_ptr(dY), M, ctypes.byref(st), _ptr(G), _ptr(A), r, _ptr(dX), _stream(dY)),
          "qlora_nf4_matmul_dx")
    return dX


def deq_matmul_fwd_group(members):
    """Y_i = X_i Wd_i^T + T_i B_i^T from dequantized bf16 weights Wd_i [N, K]
    (as dequantize / dequantize_group write them), up to 4 products sharing M
    in one launch (qlora_deq_matmul_fwd_group).  members: sequence of dicts
    with X, Wd, T, B and optional out.  Returns [Y, ...], bit-identical to
    nf4_matmul_fwd on the weights the Wd were dequantized from."""
    members = list(members)
    if not 1 <= len(members) <= 4:
        raise ValueError("a group holds 1 to 4 products")
    descs, outs = [], []
    for i, mb in enumerate(members):
        X, Wd, T, B = mb["X"], mb["Wd"], mb["T"], mb["B"]
        M = _mat(X, "members[%d].X" % i)[0]
        N, K = _mat(Wd, "members[%d].Wd" % i)
        r = _mat(B, "members[%d].B" % i)[1]
        _need(X, torch.bfloat16, "members[%d].X" % i, (M, K))
        _need(T, torch.bfloat16, "members[%d].T" % i, (M, r))
        _need(B, torch.bfloat16, "members[%d].B" % i, (N, r))
        Y = _out(mb.get("out"), (M, N), X.device, "members[%d].out" % i)
        outs.append(Y)
        descs.append(DeqMatmulFwdDescStruct(_ptr(X), M, _ptr(Wd), N, K, _ptr(T), _ptr(B), r, _ptr(Y)))
    arr = (DeqMatmulFwdDescStruct * len(descs))(*descs)
    check(lib().qlora_deq_matmul_fwd_group(len(descs), arr, _stream(members[0]["X"])), "qlora_deq_matmul_fwd_group")
    return outs


def deq_matmul_fwd(X, Wd, T, B, out=None):
    """Y = X Wd^T + T B^T with Wd the dequantized bf16 weight [N, K]."""
    M = _mat(X, "X")[0]
    N, K = _mat(Wd, "Wd")
    r = _mat(B, "B")[1]
    _need(X, torch.bfloat16, "X", (M, K))
    _need(T, torch.bfloat16, "T", (M, r))
    _need(B, torch.bfloat16, "B", (N, r))
    Y = _out(out, (M, N), X.device, "Y")
    check(lib().qlora_deq_matmul_fwd(_ptr(X), M, _ptr(Wd), N, K, _ptr(T), _ptr(B), r, _ptr(Y), _stream(X)),
          "qlora_deq_matmul_fwd")
    return Y


def deq_matmul_dx(dY, Wd, G, A, out=None):
    """dX = dY Wd + G A with Wd the dequantized bf16 weight [N, K]."""
    M = _mat(dY, "dY")[0]
    N, K = _mat(Wd, "Wd")
    r = _mat(A, "A")[0]
    _need(dY, torch.bfloat16, "dY", (M, N))
    _need(G, torch.bfloat16, "G", (M, r))
    _need(A, torch.bfloat16, "A", (r, K))
    dX = _out(out, (M, K), dY.device, "dX")
    check(lib().qlora_deq_matmul_dx(_ptr(dY), M, _ptr(Wd), N, K, _ptr(G), _ptr(A), r, _ptr(dX), _stream(dY)),
          "qlora_deq_matmul_dx")
    return dX


def lora_grads(X, dY, G, T, need_dA=True, need_dB=True, workspace=None, dA_out=None, dB_out=None):
    """dA = G^T X, dB = dY^T T (G and T carry the scale)."""
    M, K = _mat(X, "X")
    N = _mat(dY, "dY")[1]
    r = _mat(G, "G")[1]
    _need(dY, torch.bfloat16, "dY", (M, N))
    _need(G, torch.bfloat16, "G", (M, r))
    _need(T, torch.bfloat16, "T", (M, r))
    dev = X.device
    dA = _out(dA_out, (r, K), dev, "dA") if need_dA else None
    dB = _out(dB_out, (N, r), dev, "dB") if need_dB else None
    ws, ws_bytes = _workspace(workspace, lib().qlora_lora_grads_workspace_bytes(M, N, K, r), dev)
    check(lib().qlora_lora_grads(_ptr(X), _ptr(dY), _ptr(G), _ptr(T), M, N, K, r, _ptr(dA), _ptr(dB), _ptr(ws),
                                 ws_bytes, _stream(X)), "qlora_lora_grads")
    return dA, dB


def lora_grads_group(members, workspace=None):
    """dA and dB of up to 8 linears in one contraction launch plus at most one
    partial-sum launch (qlora_lora_grads_group).  members: sequence of dicts
    with X, dY, G, T (as for lora_grads) and optional need_dA / need_dB,
    dA_out / dB_out.  Returns [(dA, dB), ...], bit-identical to lora_grads of
    each member."""
    members = list(members)
    if not 1 <= len(members) <= 8:
        raise ValueError("a group holds 1 to 8 linears")
    descs, outs = [], []
    for i, mb in enumerate(members):
        X, dY, G, T = mb["X"], mb["dY"], mb["G"], mb["T"]
        M, K = _mat(X, "members[%d].X" % i)
        N = _mat(dY, "members[%d].dY" % i)[1]
        r = _mat(G, "members[%d].G" % i)[1]
        _need(dY, torch.bfloat16, "members[%d].dY" % i, (M, N))
        _need(G, torch.bfloat16, "members[%d].G" % i, (M, r))
        _need(T, torch.bfloat16, "members[%d].T" % i, (M, r))
        dev = X.device
        dA = _out(mb.get("dA_out"), (r, K), dev, "members[%d].dA" % i) if mb.get("need_dA", True) else None
        dB = _out(mb.get("dB_out"), (N, r), dev, "members[%d].dB" % i) if mb.get("need_dB", True) else None
        descs.append(LoraGradsDescStruct(X.data_ptr(), dY.data_ptr(), G.data_ptr(), T.data_ptr(), M, N, K, r,
                                         dA.data_ptr() if dA is not None else None,
                                         dB.data_ptr() if dB is not None else None))
        outs.append((dA, dB))
    arr = (LoraGradsDescStruct * len(descs))(*descs)
    X0 = members[0]["X"]
    ws, ws_bytes = _workspace(workspace, lib().qlora_lora_grads_group_workspace_bytes(len(descs), arr), X0.device)
    check(lib().qlora_lora_grads_group(len(descs), arr, _ptr(ws), ws_bytes, _stream(X0)), "qlora_lora_grads_group")
    return outs


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
