"""QLORA_SMALL_M_MAX = 0 sends a small-M forward to the tiled MFMA matmul
instead of the decode-regime kernels; both routes must match the oracle
within the matmul tolerance.  The threshold is read once per process, so the
switched run happens in one child process."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np, torch
import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import DEV, as_f64, assert_close, to_dev_bf16, to_dev_f32
assert q.lib().qlora_small_m_max() == 0
for M in (1, 16, 64):
    N, K, r, s = 320, 512, 64, 0.25
    W = workloads.weight((N, K), 7100 + M)
    X = workloads.activation_bf16((M, K), 7101 + M)
    A = workloads.lora_bf16((r, K), 7102 + M)
    B = workloads.lora_bf16((N, r), 7103 + M)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Y, T = q.linear_fwd(to_dev_bf16(X), w, to_dev_bf16(A), to_dev_bf16(B), s)
    torch.cuda.synchronize()
    wt = nf4.dequantize_q(nf4.quantize(W)).reshape(W.shape)
    Yr, Tr = olin.linear_fwd(X, wt, A, B, s)
    assert_close(as_f64(Y), Yr, "tiled-route Y, M = %d" % M)
    assert_close(as_f64(T), np.float32(s) * Tr, "tiled-route T, M = %d" % M)
print("tiled route ok", flush=True)
"""


def test_small_m_forward_through_the_tiled_route():
    print("small-M switch case: M = 16 with QLORA_SMALL_M_MAX = 0 (child process)", flush=True)
    env = dict(os.environ, QLORA_SMALL_M_MAX="0", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", CHILD], env=env, cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    assert "tiled route ok" in out.stdout
