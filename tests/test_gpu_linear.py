"""GPU parity of the QLoRA linear layer (forward and backward) with the fp64
CPU oracle, through the C ABI.  Tolerance: relative Frobenius error <= 5e-3
and elementwise |err| <= 2e-2 * max|ref| for Y, dX, dA, dB."""

import numpy as np
import pytest
import torch

import bit_nf4_quantized_absmax_amd as q
import workloads
from oracle import linear as olin
from oracle import nf4
from tests.gpu_util import DEV, as_f64, assert_close, bf16_bits, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, r, seed, w_zero=False, a_zero=False, b_zero=False):
    W = workloads.weight((N, K), seed)
    if w_zero:
        W[:] = 0
    X = workloads.activation_bf16((M, K), seed + 1)
    A = workloads.lora_bf16((r, K), seed + 2)
    B = workloads.lora_bf16((N, r), seed + 3)
    dY = workloads.activation_bf16((M, N), seed + 4)
    if a_zero:
        A[:] = 0
    if b_zero:
        B[:] = 0
    return W, X, A, B, dY


def _run(W, X, A, B, dY, scale):
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Xd, Ad, Bd, dYd = (to_dev_bf16(t) for t in (X, A, B, dY))
    Y, T = q.linear_fwd(Xd, w, Ad, Bd, scale)
    dX, dA, dB = q.linear_bwd(dYd, Xd, T, w, Ad, Bd, scale)
    torch.cuda.synchronize()
    return w, Y, T, dX, dA, dB


def _oracle_wt(W):
    ref = nf4.quantize(W)
    return nf4.dequantize_q(ref).reshape(W.shape)


def _full_check(M, N, K, r, scale, seed, name, **kw):
    print("linear case", name, (M, N, K, r), flush=True)
    W, X, A, B, dY = _inputs(M, N, K, r, seed, **kw)
    w, Y, T, dX, dA, dB = _run(W, X, A, B, dY, scale)
    wt = _oracle_wt(W)
    assert np.array_equal(bf16_bits(w.dequantize()), wt), name + ": dequant"
    Yr, Tr = olin.linear_fwd(X, wt, A, B, scale)
    dXr, dAr, dBr = olin.linear_bwd(dY, X, wt, A, B, scale)
    out = {}
    out["Y"] = assert_close(as_f64(Y), Yr, name + " Y")
    if np.any(Tr):
        out["T"] = assert_close(as_f64(T), np.float32(scale) * Tr, name + " T")
    out["dX"] = assert_close(as_f64(dX), dXr, name + " dX")
    if np.any(dAr):
        out["dA"] = assert_close(as_f64(dA), dAr, name + " dA")
    else:
        assert np.all(as_f64(dA) == 0)
    if np.any(dBr):
        out["dB"] = assert_close(as_f64(dB), dBr, name + " dB")
    else:
        assert np.all(as_f64(dB) == 0)
    return out


def test_linear_1024_config():
    cfg = workloads.CONFIGS[0]
    d = workloads.linear_inputs(cfg, 0)
    print("linear case config linear_1024", flush=True)
    w, Y, T, dX, dA, dB = _run(d["W"], d["X"], d["A"], d["B"], d["dY"], cfg.scale)
    wt = _oracle_wt(d["W"])
    Yr, _ = olin.linear_fwd(d["X"], wt, d["A"], d["B"], cfg.scale)
    dXr, dAr, dBr = olin.linear_bwd(d["dY"], d["X"], wt, d["A"], d["B"], cfg.scale)
    assert_close(as_f64(Y), Yr, "Y")
    assert_close(as_f64(dX), dXr, "dX")
    assert_close(as_f64(dA), dAr, "dA")
    assert_close(as_f64(dB), dBr, "dB")


def test_linear_ragged_tiles():
    # several 256-tiles in every dimension plus ragged tails in M, N and K
    _full_check(600, 776, 576, 24, 0.5, 100, "ragged")


@pytest.mark.parametrize("r", [1, 8, 64, 100, 128])
def test_linear_ranks(r):
    _full_check(300, 512, 512, r, 16.0 / r, 200 + r, "rank%d" % r)


def test_lora_isolation_zero_weight():
    # W = 0: Y = s X A^T B^T exactly, so the LoRA branch alone is checked.
    _full_check(256, 512, 512, 16, 2.0, 300, "w_zero", w_zero=True)


def test_lora_isolation_zero_adapters():
    _full_check(256, 512, 512, 16, 2.0, 310, "a_zero", a_zero=True)
    _full_check(256, 512, 512, 16, 2.0, 320, "b_zero", b_zero=True)


def test_identity_input_pins_layout():
    # X = I_K (M = K): Y = deq(W)^T + s A^T B^T.
    M = K = 256
    N, r, s = 320, 16, 0.5
    W, _, A, B, dY = _inputs(M, N, K, r, 400)
    X = workloads.to_bf16_bits(np.eye(K, dtype=np.float32))
    w, Y, T, dX, dA, dB = _run(W, X, A, B, dY, s)
    wt = _oracle_wt(W)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert_close(as_f64(Y), f(wt).T + s * f(A).T @ f(B).T, "identity Y")
    assert_close(as_f64(T), s * f(A).T, "identity T")


@pytest.mark.parametrize("M", [1, 5, 16, 64])
@pytest.mark.parametrize("li", [0, 4, 6])
def test_small_m_llama7b(M, li):
    cfg = workloads.CONFIGS[2]
    lin = cfg.linears[li]
    N, K, r = lin.out_features, lin.in_features, cfg.rank
    print("small-M case", lin.name, M, flush=True)
    W, X, A, B, _ = _inputs(M, N, K, r, 500 + li)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Y, T = q.linear_fwd(to_dev_bf16(X), w, to_dev_bf16(A), to_dev_bf16(B), cfg.scale)
    torch.cuda.synchronize()
    Yr, _ = olin.linear_fwd(X, _oracle_wt(W), A, B, cfg.scale)
    assert_close(as_f64(Y), Yr, "small-M Y")


@pytest.mark.parametrize("M,N,K,r", [
    (1, 776, 576, 8),       # odd number of 64-blocks per row, N not a multiple of 16
    (3, 512, 320, 16),
    (17, 264, 1024, 24),    # two 16-token tiles
    (33, 128, 4160, 64),    # three token tiles, K past one load batch
    (48, 136, 704, 128),
    (64, 512, 13056, 64),   # four token tiles, several load batches
    (8, 256, 512, 100),     # r % 8 != 0 takes the general path
])
def test_small_m_shapes(M, N, K, r):
    print("small-M shape", (M, N, K, r), flush=True)
    W, X, A, B, _ = _inputs(M, N, K, r, 900 + M)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Xd, Ad, Bd = to_dev_bf16(X), to_dev_bf16(A), to_dev_bf16(B)
    s = 16.0 / r
    Y, T = q.linear_fwd(Xd, w, Ad, Bd, s)
    T2 = q.lora_down(Xd, Ad, s)
    Y2 = q.nf4_matmul_fwd(Xd, w, T2, Bd)
    torch.cuda.synchronize()
    Yr, Tr = olin.linear_fwd(X, _oracle_wt(W), A, B, s)
    assert_close(as_f64(Y), Yr, "small-M Y")
    assert_close(as_f64(T), np.float32(s) * Tr, "small-M T")
    assert_close(as_f64(Y2), Yr, "small-M Y (T given)")


def test_small_m_deterministic():
    W, X, A, B, _ = _inputs(16, 1024, 4096, 64, 950)
    w = q.NF4Weight.quantize(to_dev_f32(W))
    Xd, Ad, Bd = to_dev_bf16(X), to_dev_bf16(A), to_dev_bf16(B)
    a = q.linear_fwd(Xd, w, Ad, Bd, 0.25)
    b = q.linear_fwd(Xd, w, Ad, Bd, 0.25)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("M", [1, 3, 16, 40, 100])
def test_linear_fwd_group_matches_single_calls(M):
    """A group of linears with different shapes: every output matches the
    oracle within tolerance.  Outside the streaming decode path (4 < M <= 64
    with K % 256 == 0) the kernels do not split a linear's work between
    workgroups, so the group and the single-linear calls also agree bit for
    bit; the streaming path splits row tiles at workgroup-range boundaries
    that depend on the whole call, which changes the fp32 summation order."""
    print("group case M", M, flush=True)
    shapes = [(512, 1024, 64), (776, 576, 8), (264, 4160, 32), (1024, 512, 16)]
    items, refs = [], []
    for i, (N, K, r) in enumerate(shapes):
        W, X, A, B, _ = _inputs(M, N, K, r, 1000 + 10 * i + M)
        w = q.NF4Weight.quantize(to_dev_f32(W))
        Xd, Ad, Bd = to_dev_bf16(X), to_dev_bf16(A), to_dev_bf16(B)
        s = 16.0 / r
        items.append((Xd, w, Ad, Bd, s))
        refs.append((W, X, A, B, s))
    outs = q.linear_fwd_group(items)
    singles = [q.linear_fwd(*it) for it in items]
    torch.cuda.synchronize()
    for (Y, T), (Y1, T1), (W, X, A, B, s) in zip(outs, singles, refs):
        K = X.shape[1]
        if not (4 < M <= 64 and K % 256 == 0):
            assert torch.equal(Y.view(torch.int16), Y1.view(torch.int16))
            assert torch.equal(T.view(torch.int16), T1.view(torch.int16))
        Yr, Tr = olin.linear_fwd(X, _oracle_wt(W), A, B, s)
        assert_close(as_f64(Y1), Yr, "single Y")
        assert_close(as_f64(T1), np.float32(s) * Tr, "single T")
        assert_close(as_f64(Y), Yr, "group Y")
        assert_close(as_f64(T), np.float32(s) * Tr, "group T")


@pytest.mark.parametrize("M", [5, 16, 33, 64])
def test_small_m_stream_group(M):
    """Streaming decode path (K % 256 == 0): a group with ragged row counts,
    one linear whose single row tile is shared by many workgroups (N = 64,
    K = 16384), and one of a single unit; every output and T against the
    oracle, and the call repeated is bit-identical."""
    print("stream group M", M, flush=True)
    shapes = [(200, 1024, 16), (64, 16384, 64), (64, 256, 8), (520, 2048, 128)]
    items, refs = [], []
    for i, (N, K, r) in enumerate(shapes):
        W, X, A, B, _ = _inputs(M, N, K, r, 1200 + 10 * i + M)
        w = q.NF4Weight.quantize(to_dev_f32(W))
        Xd, Ad, Bd = to_dev_bf16(X), to_dev_bf16(A), to_dev_bf16(B)
        s = 16.0 / r
        items.append((Xd, w, Ad, Bd, s))
        refs.append((W, X, A, B, s))
    outs = q.linear_fwd_group(items)
    again = q.linear_fwd_group(items)
    singles = [q.linear_fwd(*it) for it in items]
    torch.cuda.synchronize()
    for (Y, T), (Y2, T2), (Y1, T1), (W, X, A, B, s) in zip(outs, again, singles, refs):
        assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
        assert torch.equal(T.view(torch.int16), T2.view(torch.int16))
        Yr, Tr = olin.linear_fwd(X, _oracle_wt(W), A, B, s)
        for y, t, name in ((Y, T, "group"), (Y1, T1, "single")):
            assert_close(as_f64(y), Yr, name + " Y")
            assert_close(as_f64(t), np.float32(s) * Tr, name + " T")


def test_llama7b_full_size_sampled():
    """Full 7B shapes at 8192 tokens in the benchmark's launch configuration;
    the oracle checks sampled rows / columns spanning every tile row."""
    cfg = workloads.CONFIGS[1]
    rng = np.random.default_rng(0)
    for li in (0, 4, 6):
        d = workloads.linear_inputs(cfg, li)
        M, N, K = d["M"], d["N"], d["K"]
        print("full-size case", cfg.linears[li].name, (M, N, K), flush=True)
        w, Y, T, dX, dA, dB = _run(d["W"], d["X"], d["A"], d["B"], d["dY"], cfg.scale)
        wt = _oracle_wt(d["W"])
        rows = np.unique(np.concatenate([rng.integers(0, M, 24), [0, M - 1]]))
        assert_close(as_f64(Y)[rows], olin.linear_fwd_rows(d["X"], wt, d["A"], d["B"], cfg.scale, rows), "Y rows")
        assert_close(as_f64(dX)[rows], olin.linear_dx_rows(d["dY"], wt, d["A"], d["B"], cfg.scale, rows),
                     "dX rows")
        cols = np.unique(np.concatenate([rng.integers(0, K, 48), [0, K - 1]]))
        assert_close(as_f64(dA)[:, cols], olin.linear_dA_cols(d["dY"], d["X"], d["B"], cfg.scale, cols), "dA cols")
        nrows = np.unique(np.concatenate([rng.integers(0, N, 48), [0, N - 1]]))
        assert_close(as_f64(dB)[nrows], olin.linear_dB_rows(d["dY"], d["X"], d["A"], cfg.scale, nrows), "dB rows")
        del w, Y, T, dX, dA, dB
        torch.cuda.empty_cache()


def test_deterministic_outputs():
    W, X, A, B, dY = _inputs(512, 768, 1024, 64, 600)
    a = _run(W, X, A, B, dY, 0.25)
    b = _run(W, X, A, B, dY, 0.25)
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_step_entry_points_match_composite():
    M, N, K, r, s = 300, 512, 768, 32, 0.5
    W, X, A, B, dY = _inputs(M, N, K, r, 700)
    w, Y, T, dX, dA, dB = _run(W, X, A, B, dY, s)
    Xd, Ad, Bd, dYd = (to_dev_bf16(t) for t in (X, A, B, dY))
    T2 = q.lora_down(Xd, Ad, s)
    Y2 = q.nf4_matmul_fwd(Xd, w, T2, Bd)
    G2 = q.lora_grad_in(dYd, Bd, s)
    dX2 = q.nf4_matmul_dx(dYd, w, G2, Ad)
    dA2, dB2 = q.lora_grads(Xd, dYd, G2, T2)
    torch.cuda.synchronize()
    for x, y in ((Y, Y2), (T, T2), (dX, dX2), (dA, dA2), (dB, dB2)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_autograd_function():
    M, N, K, r, s = 128, 256, 512, 16, 2.0
    W, X, A, B, dY = _inputs(M, N, K, r, 800)
    layer = q.QLoRALinear(to_dev_f32(W), r=r, alpha=32.0, lora_A=to_dev_bf16(A), lora_B=to_dev_bf16(B))
    x = to_dev_bf16(X).requires_grad_(True)
    y = layer(x)
    y.backward(to_dev_bf16(dY))
    torch.cuda.synchronize()
    wt = _oracle_wt(W)
    Yr, _ = olin.linear_fwd(X, wt, A, B, s)
    dXr, dAr, dBr = olin.linear_bwd(dY, X, wt, A, B, s)
    assert_close(as_f64(y), Yr, "autograd Y")
    assert_close(as_f64(x.grad), dXr, "autograd dX")
    assert_close(as_f64(layer.lora_A.grad), dAr, "autograd dA")
    assert_close(as_f64(layer.lora_B.grad), dBr, "autograd dB")
