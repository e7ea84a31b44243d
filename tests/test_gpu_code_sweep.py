"""Exhaustive GPU check of the first-level code rule (creativeworksofknowledge.com,
"QLoRA: Fine-Tune 70B on One GPU", The three innovations / 1. NF4: each weight
of a block takes the nearest of the 16 levels after division by the block's
absmax; ties go to the lower code, the reading the oracle fixes).

Every fp32 x in [-1, 1] (2 x 0x3F800001 values: both zeros, every subnormal,
both ends) is coded in a block whose slot 0 holds exactly 1.0, so the block
constant is 1 and the quotient x / 1 is x itself.  The packed codes of the
quantizer must equal oracle.nf4.nearest_code over the NF4 decision
thresholds, for every value."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
from oracle import nf4
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

BLOCKS = 1 << 20          # blocks per chunk: 63 Mi test values, 256 MB of fp32 input
ONE_BITS = 0x3F800000     # bit pattern of 1.0f


def _ranges():
    """Bit-pattern ranges [lo, hi) covering [-1, 1]: +0 .. 1, then -0 .. -1."""
    return [(0, ONE_BITS + 1), (0x80000000, 0x80000000 + ONE_BITS + 1)]


@pytest.mark.timeout(900)
def test_code_rule_every_fp32_in_unit_interval():
    print("code sweep: every fp32 in [-1, 1], %d-block chunks" % BLOCKS, flush=True)
    thr = nf4.midpoint_thresholds(nf4.nf4_levels())
    per = 63 * BLOCKS
    checked = 0
    for lo, hi in _ranges():
        for start in range(lo, hi, per):
            stop = min(start + per, hi)
            vals = np.arange(start, stop, dtype=np.uint32).view(np.float32)
            n = len(vals)
            nblk = (n + 62) // 63
            w = np.zeros((nblk, 64), np.float32)
            w[:, 0] = 1.0
            body = np.zeros(nblk * 63, np.float32)   # padding slots hold +0 (also a tested value)
            body[:n] = vals
            w[:, 1:] = body.reshape(nblk, 63)
            qw = q.NF4Weight.quantize(torch.from_numpy(w).to(DEV))
            packed = qw.packed.cpu().numpy()
            del qw
            codes = nf4.unpack_nibbles(packed, nblk * 64).reshape(nblk, 64)
            assert np.all(codes[:, 0] == 15), "absmax slot"
            got = codes[:, 1:].reshape(-1)[:n]
            want = nf4.nearest_code(vals, thr)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, "x = %r (bits %#x): gpu code %d, oracle %d" % (
                float(vals[bad[0]]), int(vals[bad[0]].view(np.uint32)), int(got[bad[0]]), int(want[bad[0]]))
            checked += n
    torch.cuda.synchronize()
    assert checked == 2 * (ONE_BITS + 1)
