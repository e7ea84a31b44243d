"""GPU parity of the codec (qlora_quantize_nf4, qlora_dequantize_nf4) with the
CPU oracle: packed codes, constant codes, scales, mean and the dequantized
bf16 weights must be bit-identical."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import nf4
from tests.gpu_util import DEV, bf16_bits, to_dev_f32

pytestmark = pytest.mark.gpu


def _gpu_quantize(w2d):
    W = to_dev_f32(w2d)
    qw = q.NF4Weight.quantize(W)
    torch.cuda.synchronize()
    return qw


def _check(w2d, name):
    print("codec case", name, w2d.shape, flush=True)
    qw = _gpu_quantize(w2d)
    ref = nf4.quantize(w2d)
    packed = qw.packed.cpu().numpy()
    code8 = qw.code8.cpu().numpy()
    c2 = qw.c2.cpu().numpy()
    mean = qw.mean.cpu().numpy()[0]
    assert np.array_equal(packed, ref["packed"]), name + ": packed"
    assert np.array_equal(code8, ref["code8"]), name + ": code8"
    assert np.array_equal(c2.view(np.uint32), ref["c2"].view(np.uint32)), name + ": c2"
    assert np.float32(mean).view(np.uint32) == np.float32(ref["mean"]).view(np.uint32), name + ": mean"
    wt = bf16_bits(qw.dequantize())
    assert np.array_equal(wt.reshape(-1), nf4.dequantize_q(ref)), name + ": dequant"
    return qw, ref


@pytest.mark.parametrize("shape", [(1, 1), (1, 63), (3, 65), (7, 1001), (257, 64), (64, 4096 + 64), (1, 64 * 257 + 3)])
def test_codec_odd_shapes(shape):
    rng = np.random.default_rng(sum(shape))
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    _check(w, "odd%s" % (shape,))


def test_codec_linear_1024():
    cfg = workloads.CONFIGS[0]
    w = workloads.linear_inputs(cfg, 0)["W"]
    _check(w, "linear_1024")


@pytest.mark.parametrize("li", [0, 4, 6])
def test_codec_llama7b_shapes(li):
    cfg = workloads.CONFIGS[1]
    lin = cfg.linears[li]
    w = workloads.weight((lin.out_features, lin.in_features), workloads.seed_for(1, 10 * li))
    _check(w, lin.name)


def test_codec_special_blocks():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((40, 1024)) * 0.02).astype(np.float32)
    flat = w.reshape(-1)
    flat[0:64] = 0.0                                  # all-zero block
    flat[64:128] = -0.0                               # all negative-zero block
    flat[128:192] = np.float32(0.25) * np.sign(flat[128:192])   # +-absmax everywhere
    flat[192] = np.float32(-3.0)                      # outlier, negative absmax
    flat[256:320] = np.float32(1e-40)                 # subnormal block
    flat[320:384] = np.float32(1e30)                  # huge finite values
    flat[384:448] = nf4.nf4_levels().repeat(4) * np.float32(0.07)  # exact level multiples
    _check(w, "special_blocks")


def test_codec_constant_absmax_zero_scale():
    rng = np.random.default_rng(6)
    w = np.sign(rng.standard_normal((64, 512))).astype(np.float32) * np.float32(0.03)
    qw, ref = _check(w, "constant_absmax")
    assert np.all(ref["c2"] == 0.0)


def test_codec_all_zero():
    w = np.zeros((128, 256), np.float32)
    qw, ref = _check(w, "all_zero")
    assert np.all(bf16_bits(qw.dequantize()) == 0)


def test_code_rule_near_every_threshold():
    # Blocks whose absmax element is exactly +1 or -1, so x = w / c = w: the
    # other 63 slots sweep every fp32 within 4000 steps of each decision
    # threshold (and the naive-rounding and exact-tie cases among them).
    lv = nf4.nf4_levels().astype(np.float64)
    vals = []
    for i in range(15):
        m = np.float32((lv[i] + lv[i + 1]) / 2)
        k = int(m.view(np.int32)) if m >= 0 else -int((m.view(np.uint32) & np.uint32(0x7FFFFFFF)))
        keys = np.arange(k - 4000, k + 4001, dtype=np.int64)
        bits = np.where(keys >= 0, keys, (-keys) | 0x80000000).astype(np.uint32)
        vals.append(bits.view(np.float32))
    vals = np.concatenate(vals)
    vals = vals[np.abs(vals) <= 1.0]
    nblk = (len(vals) + 62) // 63
    w = np.zeros((nblk, 64), np.float32)
    flat = np.zeros(nblk * 63, np.float32)
    flat[:len(vals)] = vals
    w[:, 1:] = flat.reshape(nblk, 63)
    w[:, 0] = np.where(np.arange(nblk) % 2 == 0, 1.0, -1.0).astype(np.float32)
    _check(w.reshape(1, -1), "threshold_sweep")


@pytest.mark.parametrize("qtype", ["nf4", "fp4", "int4"])
def test_code_rule_near_thresholds_scaled(qtype):
    # Block constants that are not powers of two (so no reciprocal of them is
    # exact), from 1e5 down to below 2^-100, and elements w = fl32(x a) whose
    # quotient x sits from 0 to 60000 fp32 steps either side of every
    # decision threshold of the table: every code decided close to a
    # threshold, inside and outside any approximation band, must match the
    # oracle's rule on the correctly rounded quotient.
    tau = nf4.midpoint_thresholds(nf4.q4_levels(qtype))
    steps = [0, 1, 2, 3, 5, 8, 13, 40, 100, 300, 1000, 3000, 10000, 30000, 60000]
    consts = [np.float32(c) for c in (1.7e5, 0.91, 0.0137, 3.7e-3, 2.3e-20, 1.3e-33, 3.1e-38)]
    vals = []
    for a in consts:
        for t in np.unique(tau):
            for k in steps:
                for sgn in (1, -1):
                    x = np.float32(t)
                    xb = int(x.view(np.int32))
                    key = (xb if x >= 0 else -(xb & 0x7FFFFFFF)) + sgn * k
                    xk = np.array([key if key >= 0 else (-key) | 0x80000000], np.int64).astype(np.uint32).view(np.float32)[0]
                    if abs(float(xk)) <= 1.0:
                        vals.append((a, np.float32(xk * a)))
    per_const = {}
    for a, w in vals:
        per_const.setdefault(float(a), []).append(w)
    blocks = []
    for i, (a, ws) in enumerate(sorted(per_const.items())):
        ws = np.array(ws, np.float32)
        for j in range(0, len(ws), 63):
            blk = np.zeros(64, np.float32)
            blk[0] = np.float32(a) if (i + j) % 2 == 0 else -np.float32(a)
            part = ws[j:j + 63]
            blk[1:1 + len(part)] = part
            blocks.append(blk)
    w = np.concatenate(blocks)[None, :-17]   # ragged end
    print("codec case", qtype, "near thresholds scaled", w.shape, flush=True)
    qw = q.NF4Weight.quantize(to_dev_f32(w), qtype)
    torch.cuda.synchronize()
    ref = nf4.quantize(w, qtype)
    assert np.array_equal(qw.packed.cpu().numpy(), ref["packed"]), qtype + ": packed"
    assert np.array_equal(qw.code8.cpu().numpy(), ref["code8"]), qtype + ": code8"


def _same_weight(a, b, name):
    for f in ("packed", "code8", "c2", "mean"):
        assert torch.equal(getattr(a, f), getattr(b, f)), name + ": " + f


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_codec_group_matches_single_calls(dtype):
    # One grouped quantize (two launches) and one grouped dequantize (one
    # launch) over members of mixed shapes and 4-bit tables, ragged tails
    # included: bit-identical to a single call per member.
    rng = np.random.default_rng(77)
    shapes = [(4096, 4096), (3, 65), (7, 1001), (64, 4096 + 64), (1, 64 * 257 + 3), (11008, 64)]
    qtypes = ["nf4", "fp4", "int4", "nf4", "int4", "fp4"]
    Ws = [torch.from_numpy((rng.standard_normal(sh) * 0.02).astype(np.float32)).to(DEV).to(dtype) for sh in shapes]
    print("codec group case", dtype, shapes, flush=True)
    grp = q.quantize_group(Ws, qtypes)
    singles = [q.NF4Weight.quantize(W, qt) for W, qt in zip(Ws, qtypes)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(grp, singles)):
        _same_weight(a, b, "member %d" % i)
    deq = q.dequantize_group(grp)
    for i, (d, w) in enumerate(zip(deq, singles)):
        assert torch.equal(d.view(torch.int16), w.dequantize().view(torch.int16)), "dequant member %d" % i


def test_codec_group_with_member_over_2_27():
    # A member above 2^27 elements (8192 x 22016) adds its own tree launch
    # inside the group; the small member beside it must be unaffected.
    rng = np.random.default_rng(78)
    big = (torch.randn(8192, 22016, device=DEV, generator=torch.Generator(DEV).manual_seed(5)) * 0.02)
    small = torch.from_numpy((rng.standard_normal((5, 999)) * 0.02).astype(np.float32)).to(DEV)
    print("codec group case big+small", flush=True)
    grp = q.quantize_group([small, big], ["nf4", "nf4"])
    s1 = q.NF4Weight.quantize(small)
    s2 = q.NF4Weight.quantize(big)
    torch.cuda.synchronize()
    _same_weight(grp[0], s1, "small")
    _same_weight(grp[1], s2, "big")
    del big


def test_quantize_is_deterministic():
    rng = np.random.default_rng(8)
    w = to_dev_f32((rng.standard_normal((512, 2048)) * 0.02).astype(np.float32))
    a = q.NF4Weight.quantize(w)
    b = q.NF4Weight.quantize(w)
    for x, y in ((a.packed, b.packed), (a.code8, b.code8), (a.c2, b.c2), (a.mean, b.mean)):
        assert torch.equal(x, y)


def test_codec_beyond_one_grid_pass():
    """A weight larger than one pass of either codec grid (at most 16384
    workgroups: 2^25 elements per pass of the quantizer's block kernel, 2^28
    per pass of the dequantizer), ending in a ragged block: bit-exact end to
    end, every element."""
    n = (1 << 28) + 4099
    _check(workloads.weight((1, n), 7100), "1 x (2^28 + 4099)")
