"""QLoRA's frozen-base linear layer on AMD Instinct MI355X (gfx950).

NF4 weights with double-quantized absmax constants, dequantized on the fly
inside bf16 MFMA matmuls, plus a 16-bit LoRA branch, forward and backward.
The computation lives in libqlora_mi355x.so (C ABI: include/qlora.h); this
package only marshals torch tensors to it.
"""

from ._capi import EXPORTED, LIB_PATH, QLoRAError, lib, status_string  # noqa: F401
from .ops import (Q4_TYPES, NF4Weight, QLoRALinear, QLoRALinearFn, linear_bwd, linear_fwd,  # noqa: F401
                  linear_fwd_group, lora_dA_shared, lora_down, lora_down_shared, lora_grad_in, lora_grads,
                  nf4_matmul_dx, nf4_matmul_fwd, nf4_sizes, dropout_mask, dropout_apply, nf4_matmul_dx_dropout,
                  linear_fwd_dropout, linear_bwd_dropout, quantize_group, dequantize_group,
                  lora_grads_group, nf4_matmul_fwd_group, deq_matmul_fwd, deq_matmul_fwd_group, deq_matmul_dx)

__all__ = [
    "Q4_TYPES", "NF4Weight", "QLoRALinear", "QLoRALinearFn", "linear_fwd", "linear_fwd_group", "linear_bwd", "lora_down",
    "nf4_matmul_fwd", "lora_grad_in", "nf4_matmul_dx", "lora_grads", "nf4_sizes", "lib",
    "lora_down_shared", "lora_dA_shared", "dropout_mask", "dropout_apply", "nf4_matmul_dx_dropout",
    "linear_fwd_dropout", "linear_bwd_dropout", "quantize_group", "dequantize_group", "lora_grads_group", "nf4_matmul_fwd_group",
    "deq_matmul_fwd", "deq_matmul_fwd_group", "deq_matmul_dx", "QLoRAError", "status_string",
]
