"""Host-side checks of the C ABI: the library loads, exports every function
include/qlora.h declares, answers size queries, and rejects bad arguments
before launching anything (these calls never reach the GPU)."""

import ctypes
import os
import re

import pytest

import bit_nf4_quantized_absmax_amd as q
from bit_nf4_quantized_absmax_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")

OK, INVALID, SHAPE, WS = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[A-Za-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = q.lib()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(L, name), name
    assert sorted(names) == sorted(_capi.EXPORTED)


def test_status_strings_and_version():
    for s in (OK, INVALID, SHAPE, WS, -4, 123):
        assert isinstance(q.status_string(s), str) and q.status_string(s)
    assert q.lib().qlora_version() == 10000


def test_sizes():
    assert q.nf4_sizes(1) == (1, 1, 1)
    assert q.nf4_sizes(4096 * 4096) == (4096 * 4096 // 2, 262144, 1024)
    assert q.nf4_sizes(11008 * 4096) == (11008 * 2048, 704512, 2752)
    with pytest.raises(q.QLoRAError):
        q.nf4_sizes(0)
    L = q.lib()
    assert L.qlora_quantize_workspace_bytes(0) == 0
    assert L.qlora_quantize_workspace_bytes(64) >= 4
    assert L.qlora_linear_workspace_bytes(8192, 4096, 4096, 64, 0) >= 8192 * 64 * 2
    assert L.qlora_linear_workspace_bytes(8192, 4096, 4096, 64, 1) >= 2 * 8192 * 64 * 2
    assert L.qlora_linear_workspace_bytes(8, 4096, 4000, 64, 0) == 0      # K % 64
    assert L.qlora_linear_workspace_bytes(8, 4099, 4096, 64, 0) == 0      # N % 8
    assert L.qlora_linear_workspace_bytes(8, 4096, 4096, 129, 0) == 0     # r > 128
    assert L.qlora_linear_workspace_bytes(8, 4096, 4096, 0, 1) == 0       # r < 1
    assert L.qlora_lora_grads_workspace_bytes(8192, 11008, 4096, 64) > 0


def _fake_weight(rows, cols, base=0x10000):
    # Aligned fake device addresses: only valid for calls that fail validation.
    return _capi.NF4WeightStruct(base, base + 0x1000, base + 0x2000, base + 0x3000, rows, cols)


def test_validation_rejects_before_launch():
    L = q.lib()
    P = ctypes.c_void_p(0x20000)   # aligned, never dereferenced
    w = _fake_weight(64, 64)
    # quantize: null input, bad shape, missing workspace
    assert L.qlora_quantize_nf4(None, ctypes.byref(w), P, 1 << 20, None) == INVALID
    assert L.qlora_quantize_nf4(ctypes.c_void_p(0x20004), ctypes.byref(w), P, 1 << 20, None) == INVALID
    bad = _fake_weight(0, 64)
    assert L.qlora_quantize_nf4(P, ctypes.byref(bad), P, 1 << 20, None) == INVALID
    assert L.qlora_quantize_nf4(P, ctypes.byref(w), None, 0, None) == WS
    assert L.qlora_quantize_nf4(P, ctypes.byref(w), P, 1, None) == WS
    nullw = _capi.NF4WeightStruct(0, 0x11000, 0x12000, 0x13000, 64, 64)
    assert L.qlora_quantize_nf4(P, ctypes.byref(nullw), P, 1 << 20, None) == INVALID
    assert L.qlora_dequantize_nf4(None, P, None) == INVALID
    assert L.qlora_dequantize_nf4(ctypes.byref(w), None, None) == INVALID
    # linear: K % 64, N % 8, r range, scale, pointers, workspace
    wk = _fake_weight(64, 100)
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(wk), P, P, 8, 1.0, P, P, None, 0, None) == SHAPE
    wn = _fake_weight(63, 64)
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(wn), P, P, 8, 1.0, P, P, None, 0, None) == SHAPE
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(w), P, P, 0, 1.0, P, P, None, 0, None) == SHAPE
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(w), P, P, 129, 1.0, P, P, None, 0, None) == SHAPE
    assert L.qlora_linear_fwd(P, -1, ctypes.byref(w), P, P, 8, 1.0, P, P, None, 0, None) == INVALID
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(w), P, P, 8, float("nan"), P, P, None, 0, None) == INVALID
    assert L.qlora_linear_fwd(None, 8, ctypes.byref(w), P, P, 8, 1.0, P, P, None, 0, None) == INVALID
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(w), P, P, 8, 1.0, P, None, None, 0, None) == WS
    assert L.qlora_linear_fwd(P, 8, ctypes.byref(w), P, P, 8, 1.0, P, None, P, 16, None) == WS
    assert L.qlora_linear_bwd(P, P, P, 8, ctypes.byref(w), P, P, 8, 1.0, P, P, P, None, 0, None) == WS
    assert L.qlora_linear_bwd(P, P, P, 8, ctypes.byref(wk), P, P, 8, 1.0, P, P, P, P, 1 << 30, None) == SHAPE
    assert L.qlora_linear_bwd(None, P, P, 8, ctypes.byref(w), P, P, 8, 1.0, P, P, P, P, 1 << 30, None) == INVALID
    # M = 0 is valid and launches nothing
    assert L.qlora_linear_fwd(P, 0, ctypes.byref(w), P, P, 8, 1.0, P, P, None, 0, None) == OK
    assert L.qlora_linear_bwd(P, P, P, 0, ctypes.byref(w), P, P, 8, 1.0, P, P, P, P, 1 << 30, None) == OK
    assert L.qlora_nf4_matmul_fwd(P, 0, ctypes.byref(w), P, P, 8, P, None) == OK
    assert L.qlora_nf4_matmul_dx(P, 0, ctypes.byref(w), P, P, 8, P, None) == OK
    assert L.qlora_nf4_matmul_fwd(P, 8, ctypes.byref(wk), P, P, 8, P, None) == SHAPE
    assert L.qlora_lora_down(P, 0, 64, P, 8, 1.0, P, None) == OK
    assert L.qlora_lora_down(P, 4, 60, P, 8, 1.0, P, None) == SHAPE
    assert L.qlora_lora_down(P, 4, 64, P, 8, float("inf"), P, None) == INVALID
    assert L.qlora_lora_grad_in(P, 4, 60, P, 200, 1.0, P, P, 1 << 20, None) == SHAPE
    assert L.qlora_lora_grad_in(P, 4, 64, P, 8, 1.0, P, None, 0, None) == WS
    assert L.qlora_lora_grad_in_workspace_bytes(11008, 64) == 256
    assert L.qlora_lora_grad_in_workspace_bytes(11008, 65) >= 11008 * 72 * 2
    assert L.qlora_lora_grad_in_workspace_bytes(11001, 64) == 0
    assert L.qlora_lora_grads(P, P, P, P, 4, 64, 64, 8, P, P, None, 0, None) == WS
    assert L.qlora_lora_grads(P, P, P, P, 4, 64, 64, 0, P, P, P, 1 << 30, None) == SHAPE
    assert L.qlora_lora_grads(P, P, P, P, 4, 60, 64, 8, None, P, P, 1 << 30, None) == SHAPE   # dB needs N % 8
    assert L.qlora_lora_grads(P, P, P, P, 4, 64, 60, 8, P, None, P, 1 << 30, None) == SHAPE   # dA needs K % 8
    # grouped forward: bad count, bad descriptor, workspace
    D = _capi.LinearDescStruct
    ok = D(0x20000, ctypes.pointer(w), 0x20000, 0x20000, 8, 1.0, 0x20000, 0)
    arr = (D * 1)(ok)
    assert L.qlora_linear_fwd_group(0, arr, 8, P, 1 << 20, None) == INVALID
    assert L.qlora_linear_fwd_group(9, arr, 8, P, 1 << 20, None) == INVALID
    assert L.qlora_linear_group_workspace_bytes(1, arr, 8) > 0
    assert L.qlora_linear_group_workspace_bytes(0, arr, 8) == 0
    assert L.qlora_linear_fwd_group(1, arr, 8, None, 0, None) == WS
    badk = (D * 1)(D(0x20000, ctypes.pointer(wk), 0x20000, 0x20000, 8, 1.0, 0x20000, 0))
    assert L.qlora_linear_fwd_group(1, badk, 8, P, 1 << 20, None) == SHAPE
    nulx = (D * 1)(D(0, ctypes.pointer(w), 0x20000, 0x20000, 8, 1.0, 0x20000, 0))
    assert L.qlora_linear_fwd_group(1, nulx, 8, P, 1 << 20, None) == INVALID
    assert L.qlora_linear_fwd_group(1, arr, 0, None, 0, None) == OK
    # shared-input LoRA products: member count, r range, K % 8, null arrays, workspace, M = 0
    PA = (ctypes.c_void_p * 3)(0x20000, 0x30000, 0x40000)
    R3 = (ctypes.c_int32 * 3)(64, 64, 64)
    S3 = (ctypes.c_float * 3)(0.25, 0.25, 0.25)
    assert L.qlora_lora_down_shared(P, 8, 64, 0, PA, R3, S3, PA, None) == INVALID
    assert L.qlora_lora_down_shared(P, 8, 64, 9, PA, R3, S3, PA, None) == INVALID
    assert L.qlora_lora_down_shared(P, 8, 60, 3, PA, R3, S3, PA, None) == SHAPE
    assert L.qlora_lora_down_shared(P, 8, 64, 3, PA, (ctypes.c_int32 * 3)(64, 129, 8), S3, PA, None) == SHAPE
    assert L.qlora_lora_down_shared(P, 8, 64, 3, None, R3, S3, PA, None) == INVALID
    assert L.qlora_lora_down_shared(P, 8, 64, 3, PA, R3, (ctypes.c_float * 3)(1, float("nan"), 1), PA, None) == INVALID
    assert L.qlora_lora_down_shared(P, 0, 64, 3, PA, R3, S3, PA, None) == OK
    assert L.qlora_lora_dA_shared_workspace_bytes(8192, 4096, 3, R3) >= 256
    assert L.qlora_lora_dA_shared_workspace_bytes(8192, 4096, 9, R3) == 0
    assert L.qlora_lora_dA_shared(P, 8, 64, 3, PA, R3, PA, None, 0, None) == WS
    assert L.qlora_lora_dA_shared(P, 8, 64, 3, PA, R3, None, P, 1 << 20, None) == INVALID
    assert L.qlora_lora_dA_shared(P, 0, 64, 3, PA, R3, PA, P, 1 << 20, None) == OK
    # dropout: p range, K % 32, keep pointer, workspace, M = 0
    assert L.qlora_dropout_mask(P, 8, 64, 1.0, 1, P, P, None) == INVALID
    assert L.qlora_dropout_mask(P, 8, 64, -0.1, 1, P, P, None) == INVALID
    assert L.qlora_dropout_mask(P, 8, 64, float("nan"), 1, P, P, None) == INVALID
    assert L.qlora_dropout_mask(P, 8, 48, 0.1, 1, P, P, None) == SHAPE
    assert L.qlora_dropout_mask(P, 8, 64, 0.1, 1, P, None, None) == INVALID
    assert L.qlora_dropout_mask(P, 0, 64, 0.1, 1, P, P, None) == OK
    assert L.qlora_dropout_apply(P, 8, 64, None, P, None) == INVALID
    assert L.qlora_nf4_matmul_dx_dropout(P, 8, ctypes.byref(w), P, P, 8, None, P, None) == INVALID
    assert L.qlora_linear_dropout_workspace_bytes(8192, 4096, 4096, 64, 0) >= 8192 * 4096 * 2
    assert L.qlora_linear_dropout_workspace_bytes(8192, 4096, 4000, 64, 0) == 0
    assert L.qlora_linear_fwd_dropout(P, 8, ctypes.byref(w), P, P, 8, 1.0, 0.1, 1, P, None, P, None, 0, None) == WS
    assert L.qlora_linear_fwd_dropout(P, 8, ctypes.byref(w), P, P, 8, 1.0, 1.5, 1, P, None, P, P, 1 << 20, None) \
        == INVALID
    assert L.qlora_linear_bwd_dropout(P, P, None, 8, ctypes.byref(w), P, P, 8, 1.0, 0.1, None, P, P, P, P, 1 << 30,
                                      None) == INVALID
    assert L.qlora_linear_bwd_dropout(P, P, None, 0, ctypes.byref(w), P, P, 8, 1.0, 0.1, P, P, P, P, P, 1 << 30,
                                      None) == OK
    # 16-bit input quantize: input type outside the enum, null or misaligned input, workspace
    assert L.qlora_quantize_nf4_16(P, 0, ctypes.byref(w), P, 1 << 20, None) == INVALID
    assert L.qlora_quantize_nf4_16(P, 3, ctypes.byref(w), P, 1 << 20, None) == INVALID
    assert L.qlora_quantize_nf4_16(None, 1, ctypes.byref(w), P, 1 << 20, None) == INVALID
    assert L.qlora_quantize_nf4_16(ctypes.c_void_p(0x20002), 2, ctypes.byref(w), P, 1 << 20, None) == INVALID
    assert L.qlora_quantize_nf4_16(P, 1, ctypes.byref(w), None, 0, None) == WS
    # 4-bit type outside the enum (NF4 0, FP4 1, Int4 2)
    for bad_t in (-1, 3):
        wt = _capi.NF4WeightStruct(0x10000, 0x11000, 0x12000, 0x13000, 64, 64, bad_t)
        assert L.qlora_quantize_nf4(P, ctypes.byref(wt), P, 1 << 20, None) == INVALID
        assert L.qlora_dequantize_nf4(ctypes.byref(wt), P, None) == INVALID
        assert L.qlora_linear_fwd(P, 8, ctypes.byref(wt), P, P, 8, 1.0, P, P, P, 1 << 20, None) == INVALID
    for good_t in (1, 2):
        wt = _capi.NF4WeightStruct(0x10000, 0x11000, 0x12000, 0x13000, 64, 64, good_t)
        assert L.qlora_linear_fwd(P, 0, ctypes.byref(wt), P, P, 8, 1.0, P, P, None, 0, None) == OK
    # misaligned weight buffers
    mis = _capi.NF4WeightStruct(0x10008, 0x11000, 0x12000, 0x13000, 64, 64)
    assert L.qlora_dequantize_nf4(ctypes.byref(mis), P, None) == INVALID
    # size overflow
    huge = _fake_weight(1 << 20, 1 << 20)
    assert L.qlora_dequantize_nf4(ctypes.byref(huge), P, None) == SHAPE


def test_codec_group_validation_and_workspace():
    L = q.lib()
    P = ctypes.c_void_p(0x20000)
    shapes = [(4096, 4096), (11008, 4096), (3, 65)]
    ws = (_capi.NF4WeightStruct * 3)(*[_fake_weight(r, c, 0x100000 * (i + 1)) for i, (r, c) in enumerate(shapes)])
    total = L.qlora_quantize_group_workspace_bytes(3, ws)
    single = [L.qlora_quantize_workspace_bytes(r * c) for r, c in shapes]
    assert total == sum((b + 255) // 256 * 256 for b in single)
    assert L.qlora_quantize_group_workspace_bytes(0, ws) == 0
    assert L.qlora_quantize_group_workspace_bytes(9, ws) == 0
    assert L.qlora_quantize_group_workspace_bytes(3, None) == 0
    bad = (_capi.NF4WeightStruct * 2)(_fake_weight(64, 64), _fake_weight(0, 64))
    assert L.qlora_quantize_group_workspace_bytes(2, bad) == 0
    Wp = (ctypes.c_void_p * 3)(0x20000, 0x30000, 0x40000)
    assert L.qlora_quantize_nf4_group(0, Wp, 0, ws, P, total, None) == INVALID
    assert L.qlora_quantize_nf4_group(9, Wp, 0, ws, P, total, None) == INVALID
    assert L.qlora_quantize_nf4_group(3, None, 0, ws, P, total, None) == INVALID
    assert L.qlora_quantize_nf4_group(3, Wp, 0, None, P, total, None) == INVALID
    assert L.qlora_quantize_nf4_group(3, Wp, 3, ws, P, total, None) == INVALID          # in_type
    assert L.qlora_quantize_nf4_group(2, Wp, 0, bad, P, 1 << 30, None) == INVALID       # member shape
    Wmis = (ctypes.c_void_p * 3)(0x20000, 0x30004, 0x40000)
    assert L.qlora_quantize_nf4_group(3, Wmis, 0, ws, P, total, None) == INVALID       # misaligned W
    Wnull = (ctypes.c_void_p * 3)(0x20000, None, 0x40000)
    assert L.qlora_quantize_nf4_group(3, Wnull, 1, ws, P, total, None) == INVALID
    assert L.qlora_quantize_nf4_group(3, Wp, 0, ws, P, total - 1, None) == WS
    assert L.qlora_quantize_nf4_group(3, Wp, 2, ws, None, total, None) == WS
    outs = (ctypes.c_void_p * 3)(0x50000, 0x60000, 0x70000)
    assert L.qlora_dequantize_nf4_group(0, ws, outs, None) == INVALID
    assert L.qlora_dequantize_nf4_group(9, ws, outs, None) == INVALID
    assert L.qlora_dequantize_nf4_group(3, None, outs, None) == INVALID
    assert L.qlora_dequantize_nf4_group(3, ws, None, None) == INVALID
    outs_bad = (ctypes.c_void_p * 3)(0x50000, 0x60008, 0x70000)
    assert L.qlora_dequantize_nf4_group(3, ws, outs_bad, None) == INVALID
    assert L.qlora_dequantize_nf4_group(2, bad, outs, None) == INVALID


def test_lora_grads_group_validation_and_workspace():
    L = q.lib()
    D = _capi.LoraGradsDescStruct
    P = 0x20000
    shapes = [(8192, 4096, 4096, 64), (8192, 11008, 4096, 64), (1000, 64, 128, 12)]
    ds = (D * 3)(*[D(P, P, P, P, M, N, K, r, P, P) for M, N, K, r in shapes])
    total = L.qlora_lora_grads_group_workspace_bytes(3, ds)
    assert total == sum(L.qlora_lora_grads_workspace_bytes(M, N, K, r) for M, N, K, r in shapes)
    assert L.qlora_lora_grads_group_workspace_bytes(0, ds) == 0
    assert L.qlora_lora_grads_group_workspace_bytes(9, ds) == 0
    assert L.qlora_lora_grads_group_workspace_bytes(3, None) == 0
    wsp = ctypes.c_void_p(0x40000)
    assert L.qlora_lora_grads_group(0, ds, wsp, total, None) == INVALID
    assert L.qlora_lora_grads_group(9, ds, wsp, total, None) == INVALID
    assert L.qlora_lora_grads_group(3, None, wsp, total, None) == INVALID
    assert L.qlora_lora_grads_group(3, ds, wsp, total - 1, None) == WS
    assert L.qlora_lora_grads_group(3, ds, None, total, None) == WS
    bad_r = (D * 1)(D(P, P, P, P, 64, 64, 64, 129, P, P))
    assert L.qlora_lora_grads_group(1, bad_r, wsp, 1 << 30, None) == SHAPE
    bad_k = (D * 1)(D(P, P, P, P, 64, 64, 60, 8, P, None))      # dA needs K % 8 == 0
    assert L.qlora_lora_grads_group(1, bad_k, wsp, 1 << 30, None) == SHAPE
    bad_n = (D * 1)(D(P, P, P, P, 64, 60, 64, 8, None, P))      # dB needs N % 8 == 0
    assert L.qlora_lora_grads_group(1, bad_n, wsp, 1 << 30, None) == SHAPE
    neg = (D * 1)(D(P, P, P, P, -1, 64, 64, 8, P, P))
    assert L.qlora_lora_grads_group(1, neg, wsp, 1 << 30, None) == INVALID
    nox = (D * 2)(D(P, P, P, P, 64, 64, 64, 8, P, P), D(None, P, P, P, 64, 64, 64, 8, P, None))
    assert L.qlora_lora_grads_group(2, nox, wsp, 1 << 30, None) == INVALID   # dA without X
    mis = (D * 1)(D(P, P, P, P, 64, 64, 64, 8, 0x50008, P))
    assert L.qlora_lora_grads_group(1, mis, wsp, 1 << 30, None) == INVALID   # misaligned dA
    zero = (D * 1)(D(None, None, None, None, 0, 64, 64, 8, None, None))
    assert L.qlora_lora_grads_group(1, zero, wsp, 1 << 30, None) == OK       # M = 0: nothing launched


def test_matmul_fwd_group_validation():
    L = q.lib()
    Dm = _capi.MatmulFwdDescStruct
    P = 0x20000
    w1 = _fake_weight(11008, 4096)
    w2 = _fake_weight(11008, 4096, 0x900000)
    wk = _fake_weight(64, 100)                                  # K % 64 != 0
    ds = (Dm * 2)(Dm(P, 8192, ctypes.pointer(w1), P, P, 64, P), Dm(P, 8192, ctypes.pointer(w2), P, P, 64, P))
    assert L.qlora_nf4_matmul_fwd_group(0, ds, None) == INVALID
    assert L.qlora_nf4_matmul_fwd_group(5, ds, None) == INVALID
    assert L.qlora_nf4_matmul_fwd_group(2, None, None) == INVALID
    uneq = (Dm * 2)(Dm(P, 8192, ctypes.pointer(w1), P, P, 64, P), Dm(P, 4096, ctypes.pointer(w2), P, P, 64, P))
    assert L.qlora_nf4_matmul_fwd_group(2, uneq, None) == INVALID        # members must share M
    badk = (Dm * 2)(Dm(P, 8192, ctypes.pointer(w1), P, P, 64, P), Dm(P, 8192, ctypes.pointer(wk), P, P, 64, P))
    assert L.qlora_nf4_matmul_fwd_group(2, badk, None) == SHAPE
    badr = (Dm * 1)(Dm(P, 8192, ctypes.pointer(w1), P, P, 129, P))
    assert L.qlora_nf4_matmul_fwd_group(1, badr, None) == SHAPE
    nox = (Dm * 2)(Dm(P, 8192, ctypes.pointer(w1), P, P, 64, P), Dm(None, 8192, ctypes.pointer(w2), P, P, 64, P))
    assert L.qlora_nf4_matmul_fwd_group(2, nox, None) == INVALID
    mis = (Dm * 1)(Dm(P, 8192, ctypes.pointer(w1), P, P, 64, 0x30008))
    assert L.qlora_nf4_matmul_fwd_group(1, mis, None) == INVALID
    zero = (Dm * 2)(Dm(None, 0, ctypes.pointer(w1), None, P, 64, None), Dm(None, 0, ctypes.pointer(w2), None, P, 64, None))
    assert L.qlora_nf4_matmul_fwd_group(2, zero, None) == OK             # M = 0: nothing launched


def test_deq_matmul_validation():
    L = q.lib()
    P = 0x20000
    # forward: (X, M, Wd, N, K, T, B, r, Y, stream)
    assert L.qlora_deq_matmul_fwd(P, 8192, None, 4096, 4096, P, P, 64, P, None) == INVALID    # no weight
    assert L.qlora_deq_matmul_fwd(P, 8192, 0x20008, 4096, 4096, P, P, 64, P, None) == INVALID  # misaligned weight
    assert L.qlora_deq_matmul_fwd(P, 8192, P, 4096, 4000, P, P, 64, P, None) == SHAPE         # K % 64
    assert L.qlora_deq_matmul_fwd(P, 8192, P, 4092, 4096, P, P, 64, P, None) == SHAPE         # N % 8
    assert L.qlora_deq_matmul_fwd(P, 8192, P, 4096, 4096, P, P, 0, P, None) == SHAPE          # r
    assert L.qlora_deq_matmul_fwd(P, -1, P, 4096, 4096, P, P, 64, P, None) == INVALID
    assert L.qlora_deq_matmul_fwd(None, 8192, P, 4096, 4096, P, P, 64, P, None) == INVALID    # no X
    assert L.qlora_deq_matmul_fwd(None, 0, P, 4096, 4096, None, P, 64, None, None) == OK      # M = 0
    # dX: (dY, M, Wd, N, K, G, A, r, dX, stream); N % 64 on this route
    assert L.qlora_deq_matmul_dx(P, 8192, P, 4104, 4096, P, P, 64, P, None) == SHAPE
    assert L.qlora_deq_matmul_dx(P, 8192, P, 4096, 4096, P, None, 64, P, None) == INVALID     # no A
    assert L.qlora_deq_matmul_dx(None, 0, P, 4096, 4096, None, P, 64, None, None) == OK
    # group
    Dm = _capi.DeqMatmulFwdDescStruct
    ds = (Dm * 2)(Dm(P, 8192, P, 11008, 4096, P, P, 64, P), Dm(P, 8192, P, 11008, 4096, P, P, 64, P))
    assert L.qlora_deq_matmul_fwd_group(0, ds, None) == INVALID
    assert L.qlora_deq_matmul_fwd_group(5, ds, None) == INVALID
    assert L.qlora_deq_matmul_fwd_group(2, None, None) == INVALID
    uneq = (Dm * 2)(Dm(P, 8192, P, 11008, 4096, P, P, 64, P), Dm(P, 4096, P, 11008, 4096, P, P, 64, P))
    assert L.qlora_deq_matmul_fwd_group(2, uneq, None) == INVALID
    badk = (Dm * 2)(Dm(P, 8192, P, 11008, 4096, P, P, 64, P), Dm(P, 8192, P, 64, 100, P, P, 64, P))
    assert L.qlora_deq_matmul_fwd_group(2, badk, None) == SHAPE
    zero = (Dm * 1)(Dm(None, 0, P, 4096, 4096, None, P, 64, None))
    assert L.qlora_deq_matmul_fwd_group(1, zero, None) == OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    W = torch.zeros(64, 64)
    with pytest.raises(ValueError):
        q.NF4Weight.quantize(W)


def test_binding_workspace_checks_size_before_anything_else():
    import torch
    from bit_nf4_quantized_absmax_amd import ops
    with pytest.raises(ValueError, match="100 needed"):
        ops._workspace(torch.empty(99, dtype=torch.uint8), 100, None)
    with pytest.raises(ValueError, match="needed"):
        ops._workspace(torch.empty(24, dtype=torch.float32), 100, None)   # 96 bytes
    with pytest.raises(ValueError, match="GPU"):
        ops._workspace(torch.empty(100, dtype=torch.uint8), 100, None)
    assert ops._workspace(None, 0, None) == (None, 0)


def test_binding_has_no_method_arithmetic_exports():
    # the LoRA dropout scale is computed by the library from (scale, p)
    assert not hasattr(q, "dropout_scale")


def test_zero_tokens_validate_and_return_ok():
    L = q.lib()
    P = ctypes.c_void_p(0x20000)
    assert L.qlora_lora_grads(P, P, P, P, 0, 64, 64, 8, P, P, P, 1 << 20, None) == OK
    assert L.qlora_lora_grads(P, P, P, P, 0, 64, 64, 8, P, P, None, 0, None) == WS     # still validated
    assert L.qlora_lora_grad_in(P, 0, 64, P, 8, 1.0, P, P, 1 << 20, None) == OK
    w = _fake_weight(64, 64)
    assert L.qlora_linear_fwd_dropout(P, 0, ctypes.byref(w), P, P, 8, 1.0, 0.1, 1, P, None, P, P, 1 << 20,
                                      None) == OK


def test_noalloc_forward_validates_before_touching_the_gpu():
    L = q.lib()
    P = ctypes.c_void_p(0x20000)
    w = _fake_weight(64, 64)
    # T [70000, 128] bf16 does not fit the 16 MiB static scratch without T_out
    assert L.qlora_linear_fwd_noalloc(P, 70000, ctypes.byref(w), P, P, 128, 1.0, P, None, None) == -5
    assert L.qlora_linear_fwd_noalloc(P, 8, ctypes.byref(_fake_weight(64, 100)), P, P, 8, 1.0, P, None, None) == SHAPE
    assert L.qlora_linear_fwd_noalloc(None, 0, ctypes.byref(w), P, P, 8, 1.0, None, None, None) == OK
    assert "SCRATCH" in q.status_string(-5)
    assert _capi.STATIC_SCRATCH_BYTES == 16 << 20


def _small_m_max_with(value):
    # The threshold is read once per process, so each setting gets its own
    # interpreter (host only: the query never touches the GPU).
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("QLORA_SMALL_M_MAX", None)
    if value is not None:
        env["QLORA_SMALL_M_MAX"] = value
    code = ("import ctypes; L = ctypes.CDLL(%r); print(L.qlora_small_m_max())" % _capi.LIB_PATH)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    return int(out.stdout.strip().splitlines()[-1])


def test_small_m_threshold_switch():
    assert _small_m_max_with(None) == 64
    assert _small_m_max_with("16") == 16
    assert _small_m_max_with("0") == 0
    assert _small_m_max_with("1000") == 64   # clamped to the decode kernels' limit
    assert _small_m_max_with("-3") == 64     # not a count: the default
    assert _small_m_max_with("12abc") == 64
