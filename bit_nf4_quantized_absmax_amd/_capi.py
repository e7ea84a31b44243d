"""ctypes declarations of libqlora_mi355x.so (the C ABI in include/qlora.h).

Loading the library does not touch the GPU.  A missing library is an error:
there is no fallback implementation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_mi355x.so")

QLORA_OK = 0
QLORA_ERR_INVALID_ARG = -1
QLORA_ERR_UNSUPPORTED_SHAPE = -2
QLORA_ERR_WORKSPACE = -3
QLORA_ERR_HIP = -4
QLORA_ERR_SCRATCH_LIMIT = -5
STATIC_SCRATCH_BYTES = 16 << 20

EXPORTED = (
    "qlora_status_string", "qlora_version", "qlora_small_m_max", "qlora_nf4_sizes",
    "qlora_quantize_workspace_bytes", "qlora_quantize_nf4", "qlora_quantize_nf4_16", "qlora_dequantize_nf4",
    "qlora_quantize_group_workspace_bytes", "qlora_quantize_nf4_group", "qlora_dequantize_nf4_group",
    "qlora_linear_workspace_bytes", "qlora_linear_fwd", "qlora_linear_fwd_noalloc", "qlora_linear_bwd",
    "qlora_lora_down", "qlora_nf4_matmul_fwd", "qlora_nf4_matmul_fwd_group", "qlora_lora_grad_in_workspace_bytes", "qlora_lora_grad_in",
    "qlora_nf4_matmul_dx", "qlora_deq_matmul_fwd", "qlora_deq_matmul_fwd_group", "qlora_deq_matmul_dx",
    "qlora_lora_grads_workspace_bytes", "qlora_lora_grads",
    "qlora_lora_grads_group_workspace_bytes", "qlora_lora_grads_group",
    "qlora_linear_group_workspace_bytes", "qlora_linear_fwd_group",
    "qlora_lora_down_shared", "qlora_lora_dA_shared_workspace_bytes", "qlora_lora_dA_shared",
    "qlora_dropout_mask", "qlora_dropout_apply", "qlora_nf4_matmul_dx_dropout",
    "qlora_linear_dropout_workspace_bytes", "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout",
)


class QLoRAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, status_string(status), status))


class NF4WeightStruct(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("code8", ctypes.c_void_p),
        ("c2", ctypes.c_void_p),
        ("mean", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("qtype", ctypes.c_int32),
    ]


class LinearDescStruct(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p),
        ("W", ctypes.POINTER(NF4WeightStruct)),
        ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("r", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("Y", ctypes.c_void_p),
        ("T_out", ctypes.c_void_p),
    ]


class MatmulFwdDescStruct(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("W", ctypes.POINTER(NF4WeightStruct)),
        ("T", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("r", ctypes.c_int32),
        ("Y", ctypes.c_void_p),
    ]


class DeqMatmulFwdDescStruct(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("Wd", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("T", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("r", ctypes.c_int32),
        ("Y", ctypes.c_void_p),
    ]


class LoraGradsDescStruct(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p),
        ("dY", ctypes.c_void_p),
        ("G", ctypes.c_void_p),
        ("T", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("r", ctypes.c_int32),
        ("dA", ctypes.c_void_p),
        ("dB", ctypes.c_void_p),
    ]


_lib = None

_vp, _i64, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_wp = ctypes.POINTER(NF4WeightStruct)

_SIGS = {
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_version": (ctypes.c_int, []),
    "qlora_small_m_max": (ctypes.c_int, []),
    "qlora_nf4_sizes": (ctypes.c_int, [_i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "qlora_quantize_workspace_bytes": (_sz, [_i64]),
    "qlora_quantize_nf4": (ctypes.c_int, [_vp, _wp, _vp, _sz, _vp]),
    "qlora_quantize_nf4_16": (ctypes.c_int, [_vp, ctypes.c_int32, _wp, _vp, _sz, _vp]),
    "qlora_dequantize_nf4": (ctypes.c_int, [_wp, _vp, _vp]),
    "qlora_quantize_group_workspace_bytes": (_sz, [ctypes.c_int, _wp]),
    "qlora_quantize_nf4_group": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(_vp), _i32, _wp, _vp, _sz, _vp]),
    "qlora_dequantize_nf4_group": (ctypes.c_int, [ctypes.c_int, _wp, ctypes.POINTER(_vp), _vp]),
    "qlora_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, ctypes.c_int]),
    "qlora_linear_fwd": (ctypes.c_int, [_vp, _i64, _wp, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_vp, _i64, _wp, _vp, _vp, _i32, _f32, _vp, _vp, _vp]),
    "qlora_linear_bwd": (ctypes.c_int, [_vp, _vp, _vp, _i64, _wp, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                                        _vp, _sz, _vp]),
    "qlora_lora_down": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i32, _f32, _vp, _vp]),
    "qlora_nf4_matmul_fwd": (ctypes.c_int, [_vp, _i64, _wp, _vp, _vp, _i32, _vp, _vp]),
    "qlora_nf4_matmul_fwd_group": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(MatmulFwdDescStruct), _vp]),
    "qlora_lora_grad_in_workspace_bytes": (_sz, [_i64, _i32]),
    "qlora_lora_grad_in": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i32, _f32, _vp, _vp, _sz, _vp]),
    "qlora_nf4_matmul_dx": (ctypes.c_int, [_vp, _i64, _wp, _vp, _vp, _i32, _vp, _vp]),
    "qlora_deq_matmul_fwd": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp]),
    "qlora_deq_matmul_fwd_group": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(DeqMatmulFwdDescStruct), _vp]),
    "qlora_deq_matmul_dx": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp]),
    "qlora_lora_grads_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_lora_grads": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp]),
    "qlora_lora_grads_group_workspace_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(LoraGradsDescStruct)]),
    "qlora_lora_grads_group": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(LoraGradsDescStruct), _vp, _sz, _vp]),
    "qlora_linear_group_workspace_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(LinearDescStruct), _i64]),
    "qlora_linear_fwd_group": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(LinearDescStruct), _i64, _vp, _sz, _vp]),
    "qlora_lora_down_shared": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, ctypes.POINTER(_vp),
                                              ctypes.POINTER(_i32), ctypes.POINTER(_f32), ctypes.POINTER(_vp), _vp]),
    "qlora_lora_dA_shared_workspace_bytes": (_sz, [_i64, _i64, ctypes.c_int, ctypes.POINTER(_i32)]),
    "qlora_lora_dA_shared": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, ctypes.POINTER(_vp), ctypes.POINTER(_i32),
                                            ctypes.POINTER(_vp), _vp, _sz, _vp]),
    "qlora_dropout_mask": (ctypes.c_int, [_vp, _i64, _i64, _f32, ctypes.c_uint64, _vp, _vp, _vp]),
    "qlora_dropout_apply": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "qlora_nf4_matmul_dx_dropout": (ctypes.c_int, [_vp, _i64, _wp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "qlora_linear_dropout_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, ctypes.c_int]),
    "qlora_linear_fwd_dropout": (ctypes.c_int, [_vp, _i64, _wp, _vp, _vp, _i32, _f32, _f32, ctypes.c_uint64, _vp,
                                                _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_bwd_dropout": (ctypes.c_int, [_vp, _vp, _vp, _i64, _wp, _vp, _vp, _i32, _f32, _f32, _vp, _vp,
                                                _vp, _vp, _vp, _sz, _vp]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libqlora_mi355x.so is not built (expected at %s); run "
                "`python -m bit_nf4_quantized_absmax_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().qlora_status_string(int(status)).decode()


def check(status, where):
    if status != QLORA_OK:
        raise QLoRAError(status, where)
