"""Property test of the GPU codec (hypothesis, derandomized): for drawn shapes,
value scales, block patterns and 4-bit tables, qlora_quantize_nf4 and
qlora_dequantize_nf4 match the CPU oracle bit for bit (packed codes, constant
codes, group scales, mean, dequantized bf16)."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import bit_nf4_quantized_absmax_amd as q
from oracle import nf4
from tests.gpu_util import DEV, bf16_bits

pytestmark = pytest.mark.gpu


@settings(max_examples=30, deadline=None, derandomize=True)
@given(rows=st.integers(1, 300), kblocks=st.integers(1, 24), log_scale=st.integers(-60, 60),
       zero_frac=st.sampled_from([0.0, 0.1, 0.5]), qtype=st.sampled_from(["nf4", "fp4", "int4"]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_codec_matches_oracle_on_drawn_inputs(rows, kblocks, log_scale, zero_frac, qtype, seed):
    K = 64 * kblocks
    print("codec property case", rows, K, log_scale, zero_frac, qtype, seed, flush=True)
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, K)) * 2.0 ** log_scale).astype(np.float32)
    if zero_frac > 0:   # whole zero blocks (constant 0) mixed in
        blk = w.reshape(-1, 64)
        blk[rng.random(blk.shape[0]) < zero_frac] = 0.0
    qw = q.NF4Weight.quantize(torch.from_numpy(w).to(DEV), qtype=qtype)
    deq = bf16_bits(qw.dequantize()).reshape(-1)
    torch.cuda.synchronize()
    ref = nf4.quantize(w, qtype)
    assert np.array_equal(qw.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(qw.code8.cpu().numpy(), ref["code8"])
    assert np.array_equal(qw.c2.cpu().numpy().view(np.uint32), ref["c2"].view(np.uint32))
    assert np.float32(qw.mean.cpu().numpy()[0]).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32)
    assert np.array_equal(deq, nf4.dequantize_q(ref))
