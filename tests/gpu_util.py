"""Helpers shared by the GPU parity tests (moving seeded host inputs to the
device, reading results back, and the floating-point tolerance)."""

import numpy as np
import torch

from oracle import bf16 as obf16

DEV = "cuda:0"

# Tolerance for the matmul outputs (Y, dX, dA, dB), compared in fp64 with the
# oracle: relative Frobenius error <= 5e-3 and elementwise
# |err| <= 2e-2 * max |ref|.
REL_FRO = 5e-3
REL_MAX = 2e-2


def to_dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def to_dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bf16_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(t):
    return obf16.bf16_bits_to_fp64(bf16_bits(t))


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got)
    mx = np.max(np.abs(ref)) if ref.size else 0.0
    emax = np.max(np.abs(got - ref)) / mx if mx > 0 else (np.max(np.abs(got)) if got.size else 0.0)
    return rel, emax


def assert_close(got, ref, name=""):
    rel, emax = errors(got, ref)
    assert rel <= REL_FRO and emax <= REL_MAX, "%s: rel_fro=%.3g max=%.3g" % (name, rel, emax)
    return rel, emax


GUARD = 4096   # bytes of guard band on each side of a guarded buffer


class Guarded:
    """A device buffer of `nbytes` payload bytes between two guard bands of
    GUARD seeded pattern bytes.  The payload starts as 0xFF bytes (bf16 and
    fp32 NaN), so an output element a kernel fails to write shows up as NaN,
    and intact() reports whether a call wrote outside the payload."""

    def __init__(self, nbytes, seed=0, fill=0xFF):
        nbytes = int(nbytes)
        self.nbytes = nbytes
        g = np.random.default_rng(1000003 + seed)
        self.pattern = torch.from_numpy(g.integers(0, 256, 2 * GUARD, dtype=np.uint8))
        self.full = torch.empty(nbytes + 2 * GUARD, dtype=torch.uint8, device=DEV)
        self.full[:GUARD].copy_(self.pattern[:GUARD])
        self.full[GUARD + nbytes:].copy_(self.pattern[GUARD:])
        self.payload = self.full[GUARD:GUARD + nbytes]
        self.payload.fill_(fill)

    def tensor(self, shape, dtype=torch.bfloat16):
        return self.payload.view(dtype).view(*shape)

    def intact(self):
        torch.cuda.synchronize()
        full = self.full.cpu()
        return (torch.equal(full[:GUARD], self.pattern[:GUARD]) and
                torch.equal(full[GUARD + self.nbytes:], self.pattern[GUARD:]))


def guarded_like(shape, dtype=torch.bfloat16, seed=0):
    """(Guarded, tensor of `shape`) for an output of that shape and dtype."""
    n = 1
    for d in shape:
        n *= int(d)
    g = Guarded(n * torch.empty((), dtype=dtype).element_size(), seed)
    return g, g.tensor(shape, dtype)
