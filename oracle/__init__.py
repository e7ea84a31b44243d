"""CPU oracle for the QLoRA frozen-base linear layer (test infrastructure only).

This package is a plain, slow, obviously-correct NumPy restatement of what the
HIP path computes.  It exists so the GPU results can be checked against an
independent implementation; it is never part of the product path.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code, tables or constant generators
with ``bit_nf4_quantized_absmax_amd`` and imports nothing from it.

Sources (web pages on QLoRA, arXiv 2305.14314):
  * automatone.win, "QLoRA paper explained" -- sections "How it works"
    (4-bit NormalFloat, Double Quantization) and "TL;DR".
  * creativeworksofknowledge.com, "QLoRA: Fine-Tune 70B on One GPU" --
    "The three innovations" (1. NF4, 2. Double quantization) and "Code".
  * aiwiki.com.my, "QLoRA" -- "Key Concepts and Technology".
  * gptget.net, "QLoRA: Efficient Finetuning of Quantized LLMs" -- "Deep
    Analysis / Methodology".

Modules:
  nf4     -- NF4 levels, the 8-bit constant table, quantize / dequantize.
  linear  -- forward and backward of Y = X deq(W)^T + s (X A^T) B^T in fp64.
  bf16    -- fp32 -> bf16 round-to-nearest-even and bf16 -> fp64 decoding.

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, invariants, independent library routines and brute force.
No function here is "parity unpinned".
"""

from . import bf16, nf4, linear  # noqa: F401
