#!/usr/bin/env python3
"""Benchmark of the QLoRA frozen-base linear layer on one MI355X.

Workload (the headline): the seven linears of a LLaMA-7B-shaped decoder
layer (q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008), weights
N(0, 0.02) quantized to NF4 with double-quantized constants, 8192 tokens of
bf16 activations N(0, 1), LoRA r = 64, alpha = 16 on every linear.  One step
is the forward and the backward (dX, dA, dB) of all seven linears with the
weights already quantized and every input resident in HBM:
    W~ = deq(W);  T = X A^T;  Y = X W~^T + s T B^T;  G = dY B;
    dX = dY W~ + s G A;  dA = s G^T X;  dB = s dY^T T.
By default (--matmul deq) the step dequantizes the layer's seven weights to
bf16 in one grouped launch (timed, part of the step) and both matmuls of each
linear read those copies; --matmul fused expands the NF4 codes inside every
matmul tile instead.  The outputs of the two are bit-identical.
Metric: algorithmic TFLOP/s = sum over linears of 4 M N K + 6 M r (N + K)
per step, divided by the mean step time of the timed steps (HIP events on
the launch stream; step_ms gives the median and minimum single step).

Also reported on the same JSON line:
  roofline      the dominant kernel (the forward matmul), timed with HIP
                events around each of its launches inside the timed region
  kernels       the same for the dX matmul and the dequantization
  cpu_baseline  the CPU oracle on a bounded token sample of the same step
  small_m       forward-only M = 1 / 16 / 64 over 4 weight sets (> the 256 MB
                Infinity Cache), replayed from HIP graphs (200 replays, mean,
                median and minimum per layer), algorithmic HBM GB/s:
                7 single-linear calls per layer and one grouped call
  quantize      quantize throughput on the 7 weights (algorithmic GB/s)
  dequantize    standalone dequantization to bf16 of the 7 weights over 4
                weight sets, from a HIP graph (algorithmic GB/s, HBM fraction)
  small_config  the 1024 x 1024, M = 128, r = 8 parity configuration:
                quantize, forward, backward (launch-bound, for reference)
  q4_types      NF4 / FP4 / Int4 level tables on a 4096 x 4096 weight:
                reconstruction error, quantize from fp32 and bf16, forward
  shared_input  LoRA products of q / k / v and gate / up (one X): separate
                launches against one shared-input launch
  dropout       the 7B step with LoRA dropout p = 0.05 against without, and
                the keep-mask kernel
  llama33b_layer, llama65b
                fwd + bwd of one 33B / 65B layer; the 65B model's 80 layers
                quantized, with the codec oracle timed on one of its weights

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extras]
                       [--matmul deq|fused] [--copy-probe-mib MiB] [--small-m-only [--small-m-eager]]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "NF4+LoRA linear fwd+bwd TFLOP/s (7B layer, 8192 tok); small-M dequant GB/s"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extras", action="store_true", help="skip small-M and quantize figures")
    p.add_argument("--small-m-only", action="store_true",
                   help="only the small-M (decode) figures, as one JSON line (for profiling that path)")
    p.add_argument("--small-m-eager", action="store_true",
                   help="with --small-m-only: eager calls instead of graph replays (counter passes)")
    p.add_argument("--small-m-pattern", choices=("both", "grouped", "per_linear"), default="both",
                   help="with --small-m-only: the launch patterns to run (profiles of one pattern)")
    p.add_argument("--codec-only", action="store_true",
                   help="only the quantize / dequantize figures, as one JSON line (for profiling the codec)")
    p.add_argument("--cpu-tokens", type=int, default=8192, help="token sample for the CPU oracle")
    p.add_argument("--matmul", choices=("deq", "fused"), default="deq",
                   help="deq: one grouped dequantize per step, then the matmuls from the bf16 weights; "
                        "fused: the NF4 codes expanded inside every matmul tile")
    p.add_argument("--vendor-gemm-only", action="store_true",
                   help="only a same-process comparison of the matmul launches with the vendor library's "
                        "plain bf16 GEMM (torch.mm) on the 7B shapes, as one JSON line")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device-to-device copy of this many MiB first (a reference "
                        "dispatch for scaling hardware byte counters)")
    return p.parse_args()


def linear_flops(M, N, K, r):
    return 4.0 * M * N * K + 6.0 * M * r * (N + K)


def small_m_bytes(M, N, K, r):
    # packed codes + 8-bit constants + fp32 group scales + mean + X + Y + A + B
    return N * K / 2 + N * K / 64 + 4 * N * K / 16384 + 4 + 2 * M * K + 2 * M * N + 2 * r * K + 2 * r * N


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "matmul_llama7b_m8192_hbm_traffic.md")
MATMUL_SOURCES = [os.path.join(ROOT, "bit_nf4_quantized_absmax_amd", "csrc", f)
                  for f in ("matmul.hip", "common.h", "lds_dma.h")]


def matmul_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in MATMUL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed PMC summary, or None
    when there is none or the matmul sources changed since it was taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("source_sha256") != matmul_source_sha256():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("traffic_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Device-resident inputs, outputs and workspaces of one linear."""

    def __init__(self, q, torch, workloads, lin, M, r, seed, dev):
        N, K = lin.out_features, lin.in_features
        self.name, self.M, self.N, self.K, self.r = lin.name, M, N, K, r
        W = workloads.device_normal((N, K), workloads.W_STD, seed, dev)
        self.w = q.NF4Weight.quantize(W)
        del W
        bf = torch.bfloat16
        self.X = workloads.device_normal((M, K), 1.0, seed + 1, dev, bf)
        self.A = workloads.device_normal((r, K), workloads.LORA_STD, seed + 2, dev, bf)
        self.B = workloads.device_normal((N, r), workloads.LORA_STD, seed + 3, dev, bf)
        self.dY = workloads.device_normal((M, N), 1.0, seed + 4, dev, bf)
        self.Y = torch.empty(M, N, dtype=bf, device=dev)
        self.T = torch.empty(M, r, dtype=bf, device=dev)
        self.G = torch.empty(M, r, dtype=bf, device=dev)
        self.dX = torch.empty(M, K, dtype=bf, device=dev)
        self.Wd = torch.empty(N, K, dtype=bf, device=dev)   # the step's dequantized weight
        ws = q.lib().qlora_lora_grads_workspace_bytes(M, N, K, r)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.gws = torch.empty(max(q.lib().qlora_lora_grad_in_workspace_bytes(N, r), 16), dtype=torch.uint8,
                               device=dev)
        self.flops = linear_flops(M, N, K, r)
        self.fwd_mm_flops = 2.0 * M * N * K + 2.0 * M * r * N
        self.dx_mm_flops = 2.0 * M * N * K + 2.0 * M * r * K


# Forward groups of a LLaMA layer: the products computed together (q, k and v
# from one normalized input; gate and up from the next); each group's forward
# matmuls run as one launch over their concatenated tiles.
FWD_GROUPS = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))


def fwd_groups(layers):
    by = {L.name: L for L in layers}
    if sorted(by) == sorted(n for g in FWD_GROUPS for n in g):
        return [[by[n] for n in g] for g in FWD_GROUPS]
    return [[L] for L in layers]


def _timed(events, key, torch, grp):
    if events is None:
        return None
    events.setdefault(key, []).append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                                       grp))
    events[key][-1][0].record()
    return events[key][-1][1]


def vendor_gemm_bench(q, torch, workloads, cfg, dev, reps=10, rounds=3):
    """The dequantized-weight matmuls against the vendor library's plain bf16
    GEMM (torch.mm, which dispatches to hipBLASLt) on the same operands, one
    process, alternating (the library's forward allocates its output per
    call, through torch's caching allocator): a reference for what a tuned
    library reaches on
    these shapes on this chip.  Both are timed on the base product's 2 M N K
    FLOP; ours also runs the rank-r LoRA contraction steps (Y += T B^T,
    dX += G A) inside the same launch, which the library call does not.
    The LoRA products T = X A^T, G = dY B and dA = G^T X, dB = dY^T T are
    compared the same way, as HBM rates on their algorithmic bytes (each
    operand read once, each output written once)."""
    M, r = cfg.tokens, cfg.rank
    bf = torch.bfloat16
    out = {}
    shapes = []
    for lin in cfg.linears:
        key = (lin.out_features, lin.in_features)
        if key not in shapes:
            shapes.append(key)
    for si, (N, K) in enumerate(shapes):
        seed = 77000 + 10 * si
        X = workloads.device_normal((M, K), 1.0, seed, dev, bf)
        Wd = workloads.device_normal((N, K), workloads.W_STD, seed + 1, dev, bf)
        dY = workloads.device_normal((M, N), 1.0, seed + 2, dev, bf)
        T = workloads.device_normal((M, r), 1.0, seed + 3, dev, bf)
        G = workloads.device_normal((M, r), 1.0, seed + 4, dev, bf)
        A = workloads.device_normal((r, K), workloads.LORA_STD, seed + 5, dev, bf)
        B = workloads.device_normal((N, r), workloads.LORA_STD, seed + 6, dev, bf)
        Y = torch.empty(M, N, dtype=bf, device=dev)
        dX, dXv = torch.empty(M, K, dtype=bf, device=dev), torch.empty(M, K, dtype=bf, device=dev)
        calls = {
            "fwd_ours": lambda: q.deq_matmul_fwd(X, Wd, T, B, out=Y),
            "fwd_vendor": lambda: torch.nn.functional.linear(X, Wd),
            "dx_ours": lambda: q.deq_matmul_dx(dY, Wd, G, A, out=dX),
            "dx_vendor": lambda: torch.mm(dY, Wd, out=dXv),
        }
        times = {k: [] for k in calls}
        for fn in calls.values():
            fn()
        torch.cuda.synchronize()
        for _ in range(rounds):
            for k, fn in calls.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                times[k].append(e0.elapsed_time(e1) * 1e3 / reps)
        flops = 2.0 * M * N * K
        ent = dict(M=M, N=N, K=K, r=r)
        for k, ts in times.items():
            us = min(ts)
            ent[k] = dict(us=round(us, 1), TFLOPs=round(flops / (us * 1e-6) / 1e12, 1),
                          frac_bf16_peak=round(flops / (us * 1e-6) / 2.5e15, 4))
        # The LoRA products (HBM-bound): ours (T and G carry the scale; dA and dB
        # in one call) against the library's plain products on the same operands.
        Tv, Gv = torch.empty(M, r, dtype=bf, device=dev), torch.empty(M, r, dtype=bf, device=dev)
        dA, dB = torch.empty(r, K, dtype=bf, device=dev), torch.empty(N, r, dtype=bf, device=dev)
        dAv, dBv = torch.empty(r, K, dtype=bf, device=dev), torch.empty(N, r, dtype=bf, device=dev)
        To, Go = torch.empty(M, r, dtype=bf, device=dev), torch.empty(M, r, dtype=bf, device=dev)
        gws = torch.empty(max(q.lib().qlora_lora_grad_in_workspace_bytes(N, r), 16), dtype=torch.uint8, device=dev)
        ws = torch.empty(max(q.lib().qlora_lora_grads_workspace_bytes(M, N, K, r), 16), dtype=torch.uint8, device=dev)
        At, Gt, dYt = A.t(), G.t(), dY.t()
        lcalls = {
            "T_ours": lambda: q.lora_down(X, A, cfg.scale, out=To),
            "T_vendor": lambda: torch.mm(X, At, out=Tv),
            "G_ours": lambda: q.lora_grad_in(dY, B, cfg.scale, out=Go, workspace=gws),
            "G_vendor": lambda: torch.mm(dY, B, out=Gv),
            "dAdB_ours": lambda: q.lora_grads(X, dY, G, T, workspace=ws, dA_out=dA, dB_out=dB),
            "dAdB_vendor": lambda: (torch.mm(Gt, X, out=dAv), torch.mm(dYt, T, out=dBv)),
        }
        lbytes = {"T": 2.0 * (M * K + r * K + M * r), "G": 2.0 * (M * N + N * r + M * r),
                  "dAdB": 2.0 * (M * K + M * N + 2 * M * r + r * K + N * r)}
        ltimes = {k: [] for k in lcalls}
        for fn in lcalls.values():
            fn()
        torch.cuda.synchronize()
        for _ in range(rounds):
            for k, fn in lcalls.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                ltimes[k].append(e0.elapsed_time(e1) * 1e3 / reps)
        for k, ts in ltimes.items():
            us = min(ts)
            nb = lbytes[k.split("_")[0]]
            ent[k] = dict(us=round(us, 1), GBps=round(nb / (us * 1e-6) / 1e9, 1), frac_hbm=round(nb / (us * 1e-6) / 8e12, 4))
        out["N%d_K%d" % (N, K)] = ent
        del X, Wd, dY, T, G, A, B, Y, dX, dXv, Tv, Gv, dA, dB, dAv, dBv, To, Go, gws, ws, At, Gt, dYt
        torch.cuda.empty_cache()
    return out


def run_step(q, torch, layers, scale, events=None, mode="deq"):
    """One fwd + bwd of every linear.  mode "deq": the layer's weights are
    dequantized to bf16 once (one grouped launch) and both matmuls of every
    linear read those copies; "fused": the matmuls expand the NF4 codes
    themselves.  Per forward group: the LoRA-down of each member, the group's
    forward matmuls (one launch); then per member G, the dX matmul and
    dA / dB."""
    if mode == "deq":
        for i in range(0, len(layers), 8):
            part = layers[i:i + 8]
            end = _timed(events, "dequant", torch, part)
            q.dequantize_group([L.w for L in part], outs=[L.Wd for L in part])
            if end is not None:
                end.record()
    for grp in fwd_groups(layers):
        for L in grp:
            q.lora_down(L.X, L.A, scale, out=L.T)
        end = _timed(events, "fwd", torch, grp)
        if mode == "deq":
            q.deq_matmul_fwd_group([dict(X=L.X, Wd=L.Wd, T=L.T, B=L.B, out=L.Y) for L in grp])
        elif len(grp) > 1:
            q.nf4_matmul_fwd_group([dict(X=L.X, w=L.w, T=L.T, B=L.B, out=L.Y) for L in grp])
        else:
            q.nf4_matmul_fwd(grp[0].X, grp[0].w, grp[0].T, grp[0].B, out=grp[0].Y)
        if end is not None:
            end.record()
        for L in grp:
            q.lora_grad_in(L.dY, L.B, scale, out=L.G, workspace=L.gws)
            end = _timed(events, "dx", torch, [L])
            if mode == "deq":
                q.deq_matmul_dx(L.dY, L.Wd, L.G, L.A, out=L.dX)
            else:
                q.nf4_matmul_dx(L.dY, L.w, L.G, L.A, out=L.dX)
            if end is not None:
                end.record()
            q.lora_grads(L.X, L.dY, L.G, L.T, workspace=L.ws)


def cpu_baseline(cfg, tokens):
    """The oracle (as it stands) on `tokens` tokens of every linear of the step."""
    import workloads
    from oracle import linear as olin
    from oracle import nf4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    total_flops, total_s = 0.0, 0.0
    for li, lin in enumerate(cfg.linears):
        d = workloads.linear_inputs(cfg, li, tokens=tokens)
        qd = nf4.quantize(d["W"])          # weights are pre-quantized in the step: untimed
        t0 = time.perf_counter()
        wt = nf4.dequantize_q(qd).reshape(d["N"], d["K"])
        olin.linear_fwd(d["X"], wt, d["A"], d["B"], cfg.scale)
        olin.linear_bwd(d["dY"], d["X"], wt, d["A"], d["B"], cfg.scale)
        total_s += time.perf_counter() - t0
        total_flops += linear_flops(tokens, d["N"], d["K"], d["r"])
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = None
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    return dict(value=total_flops / total_s / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                affinity_cpus=affinity, cpu_model=cpu_model,
                sample="fp64 NumPy oracle fwd+bwd of all 7 linears (dequantize + products) on %d of the 8192 "
                       "tokens, %.1f s; rate = algorithmic FLOP / time" % (tokens, total_s))


def small_m_bench(q, torch, workloads, cfg, dev, reps=200, graphs=True, patterns=("per_linear", "grouped")):
    """Forward at M = 1/16/64 over 4 weight sets of the 7B layer (> Infinity Cache).

    Two launch patterns, each captured once in a HIP graph and replayed (the
    library makes no allocation and no memset inside a call):
      per_linear  7 linear_fwd calls per layer
      grouped     one linear_fwd_group call over the 7 linears
    A call is 2 launches at M <= 4 (down-projection, dequant-GEMV) and, for
    4 < M <= 64, 4 (down-projection chunks, T, weight stream, tile epilogue)
    except single-linear calls at M <= 16, which take the 2-launch path.
    GB/s = algorithmic bytes of the 7 linears / time per layer.  graphs=False
    replays the calls eagerly instead (for counter passes, which do not
    support graph replays)."""
    import ctypes
    from bit_nf4_quantized_absmax_amd._capi import LinearDescStruct
    r = cfg.rank
    sets = []
    for s in range(4):
        ws = []
        for li, lin in enumerate(cfg.linears):
            W = workloads.device_normal((lin.out_features, lin.in_features), workloads.W_STD,
                                        90000 + 100 * s + li, dev)
            ws.append(q.NF4Weight.quantize(W))
            del W
        sets.append(ws)
    out = {}
    for M in cfg.small_m:
        lin_in = []
        for li, lin in enumerate(cfg.linears):
            N, K = lin.out_features, lin.in_features
            X = workloads.device_normal((M, K), 1.0, 91000 + li, dev, torch.bfloat16)
            A = workloads.device_normal((r, K), workloads.LORA_STD, 92000 + li, dev, torch.bfloat16)
            B = workloads.device_normal((N, r), workloads.LORA_STD, 93000 + li, dev, torch.bfloat16)
            Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            T = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
            nws = max(q.lib().qlora_linear_workspace_bytes(M, N, K, r, 0), 16)
            wsp = torch.empty(nws, dtype=torch.uint8, device=dev)
            lin_in.append((X, A, B, Y, T, wsp))
        nbytes = sum(small_m_bytes(M, l.out_features, l.in_features, r) for l in cfg.linears)
        group_items = [[(X, w, A, B, cfg.scale, T, Y) for (X, A, B, Y, T, _), w in zip(lin_in, ws)] for ws in sets]
        structs = [[w.struct() for w in ws] for ws in sets]
        descs = [(LinearDescStruct * len(cfg.linears))(*[
            LinearDescStruct(X.data_ptr(), ctypes.pointer(st), A.data_ptr(), B.data_ptr(), r, cfg.scale,
                             Y.data_ptr(), T.data_ptr()) for (X, A, B, Y, T, _), st in zip(lin_in, sts)])
            for sts in structs]
        gws_bytes = max(q.lib().qlora_linear_group_workspace_bytes(len(cfg.linears), d, M) for d in descs)
        gws = torch.empty(max(gws_bytes, 16), dtype=torch.uint8, device=dev)

        def per_linear(ws):
            for (X, A, B, Y, T, wsp), w in zip(lin_in, ws):
                q.linear_fwd(X, w, A, B, cfg.scale, T_out=T, out=Y, workspace=wsp)

        def grouped(si):
            q.linear_fwd_group(group_items[si], workspace=gws)

        res = {}
        for name, fn in (("per_linear", lambda si: per_linear(sets[si])), ("grouped", grouped)):
            if name not in patterns:
                continue
            for si in range(len(sets)):
                fn(si)
            torch.cuda.synchronize()
            if graphs:
                stream = torch.cuda.Stream()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    for si in range(len(sets)):
                        fn(si)
            else:
                class _Eager:
                    def replay(self):
                        for si in range(len(sets)):
                            fn(si)
                graph = _Eager()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            evs[0].record()
            for i in range(reps):
                graph.replay()
                evs[i + 1].record()
            torch.cuda.synchronize()
            us = evs[0].elapsed_time(evs[-1]) * 1e3 / (reps * len(sets))
            per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 / len(sets) for i in range(reps))
            gbs = nbytes / (us * 1e-6) / 1e9
            res[name] = dict(us_per_layer=round(us, 2), median_us=round(per[reps // 2], 2), min_us=round(per[0], 2),
                             reps=reps, GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
            del graph
        if "per_linear" in res:
            res["per_linear"]["launches_per_layer"] = (2 if M <= 16 else 3) * len(cfg.linears)
        if "grouped" in res:
            res["grouped"]["launches_per_layer"] = 2 if M <= 4 else 3
        res["bytes_per_layer"] = int(nbytes)
        out["M%d" % M] = res
    del sets
    torch.cuda.empty_cache()
    return out


def quantize_bench(q, torch, workloads, cfg, dev, reps=10, grouped=False):
    """Quantization (fp32 weights -> packed codes + double-quantized
    constants) of the 7 weights of a layer, over 4 weight sets (> the 256 MB
    Infinity Cache), through the C ABI with preallocated outputs and
    workspaces, captured once in a HIP graph and replayed: one
    qlora_quantize_nf4 call per weight, or (grouped) one
    qlora_quantize_nf4_group call per layer.  Algorithmic bytes per parameter:
    4 (fp32) read, 1/2 (codes) + 1/64 (constant codes) + 4/16384 (group
    scales) written."""
    import ctypes
    from bit_nf4_quantized_absmax_amd._capi import NF4WeightStruct
    lib = q.lib()
    sets = []
    for si in range(4):
        items = []
        for li, lin in enumerate(cfg.linears):
            rows, cols = lin.out_features, lin.in_features
            W = workloads.device_normal((rows, cols), workloads.W_STD, 95000 + 100 * si + li, dev)
            w = q.NF4Weight.empty(rows, cols, W.device)
            nws = lib.qlora_quantize_workspace_bytes(rows * cols)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
            items.append((W, w, w.struct(), ws, nws))
        if grouped:
            sts = (NF4WeightStruct * len(items))(*[it[2] for it in items])
            ptrs = (ctypes.c_void_p * len(items))(*[it[0].data_ptr() for it in items])
            gws_bytes = lib.qlora_quantize_group_workspace_bytes(len(items), sts)
            gws = torch.empty(gws_bytes, dtype=torch.uint8, device=dev)
            items = dict(items=items, sts=sts, ptrs=ptrs, ws=gws, nws=gws_bytes)
        sets.append(items)

    def run(stream):
        for items in sets:
            if grouped:
                rc = lib.qlora_quantize_nf4_group(len(items["items"]), items["ptrs"], 0, items["sts"],
                                                  items["ws"].data_ptr(), items["nws"], stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("qlora_quantize_nf4_group failed: %d" % rc)
                continue
            for W, _, st, ws, nws in items:
                rc = lib.qlora_quantize_nf4(W.data_ptr(), ctypes.byref(st), ws.data_ptr(), nws, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("qlora_quantize_nf4 failed: %d" % rc)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run(stream)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record()
    for i in range(reps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 / 4 for i in range(reps))
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / (4 * reps)
    params = sum(l.out_features * l.in_features for l in cfg.linears)
    nbytes = params * (4 + 0.5 + 1 / 64 + 4 / 16384)
    del graph, sets
    torch.cuda.empty_cache()
    return dict(us_per_layer=round(us, 2), median_us=round(per[reps // 2], 2), min_us=round(per[0], 2),
                params=int(params), GBps=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac_hbm=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                launches_per_layer=2 if grouped else 2 * len(cfg.linears))


def q4_types_bench(q, torch, workloads, dev, reps=10):
    """The three 4-bit level tables (NF4, and FP4 / Int4, the types the pages
    compare it with) on the 7B q_proj shape, 4096 x 4096 weights N(0, 0.02):
    relative RMS error of the dequantized weight, quantize time from fp32 and
    from bf16 input (HBM GB/s: input read + codes and constants written), and
    the fused forward matmul at M = 8192 (same kernel, other table)."""
    N = K = 4096
    M, r = 8192, 64
    W = workloads.device_normal((N, K), workloads.W_STD, 97000, dev)
    Wb = W.to(torch.bfloat16)
    X = workloads.device_normal((M, K), 1.0, 97001, dev, torch.bfloat16)
    T = workloads.device_normal((M, r), 1.0, 97002, dev, torch.bfloat16)
    B = workloads.device_normal((N, r), workloads.LORA_STD, 97003, dev, torch.bfloat16)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    w64 = W.to(torch.float64)
    ref_ms = float(torch.mean(w64 * w64))
    out_bytes = N * K * (0.5 + 1 / 64 + 4 / 16384)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res, ws = {}, {}
    for qt in q.Q4_TYPES:
        w = ws[qt] = q.NF4Weight.quantize(W, qt)
        err = w.dequantize().to(torch.float64) - w64
        rel = (float(torch.mean(err * err)) / ref_ms) ** 0.5
        ms32 = timed(lambda: q.NF4Weight.quantize(W, qt))
        ms16 = timed(lambda: q.NF4Weight.quantize(Wb, qt))
        res[qt] = dict(rel_rms_error=round(rel, 5),
                       quantize_fp32_us=round(ms32 * 1e3, 1),
                       quantize_fp32_GBps=round((4 * N * K + out_bytes) / (ms32 * 1e-3) / 1e9, 1),
                       quantize_bf16_us=round(ms16 * 1e3, 1),
                       quantize_bf16_GBps=round((2 * N * K + out_bytes) / (ms16 * 1e-3) / 1e9, 1))
        del err
    # the matmuls in interleaved rounds (the last round is reported), so that
    # clock ramps do not favour one table
    flops = 2.0 * M * N * K + 2.0 * M * r * N
    for _ in range(3):
        for qt in q.Q4_TYPES:
            ms_mm = timed(lambda: q.nf4_matmul_fwd(X, ws[qt], T, B, out=Y))
            res[qt].update(fwd_matmul_us=round(ms_mm * 1e3, 1),
                           fwd_matmul_TFLOPs=round(flops / (ms_mm * 1e-3) / 1e12, 1))
    del W, Wb, X, T, B, Y, w64, ws
    torch.cuda.empty_cache()
    res["note"] = ("4096 x 4096 weight; quantize times include workspace allocation by the Python binding; "
                   "matmul at M = 8192, r = 64")
    return res


def shared_input_bench(q, torch, workloads, dev, reps=20):
    """LoRA products of linears that read the same X at the 7B shapes, M =
    8192, r = 64: q / k / v (K = 4096, three members) and gate / up (K = 4096,
    two members).  T = s X A_i^T and dA = G_i^T X, per linear (one launch each)
    against one shared-input launch; HBM GB/s of the shared launch counts X
    once plus the adapters and outputs."""
    M, K, r = 8192, 4096, 64
    out = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    X = workloads.device_normal((M, K), 1.0, 98000, dev, torch.bfloat16)
    dY = torch.zeros(M, 8, dtype=torch.bfloat16, device=dev)
    for name, n in (("qkv", 3), ("gate_up", 2)):
        As = [workloads.device_normal((r, K), workloads.LORA_STD, 98100 + i, dev, torch.bfloat16) for i in range(n)]
        Gs = [workloads.device_normal((M, r), 0.05, 98200 + i, dev, torch.bfloat16) for i in range(n)]
        Ts = [torch.empty(M, r, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        dAs = [torch.empty(r, K, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        sc = [0.25] * n
        gws = torch.empty(max(q.lib().qlora_lora_grads_workspace_bytes(M, 8, K, r), 16), dtype=torch.uint8,
                          device=dev)
        dws = torch.empty(1 << 26, dtype=torch.uint8, device=dev)
        t_sep = timed(lambda: [q.lora_down(X, A, 0.25, out=T) for A, T in zip(As, Ts)])
        t_sh = timed(lambda: q.lora_down_shared(X, As, sc, outs=Ts))
        a_sep = timed(lambda: [q.lora_grads(X, dY, G, G, need_dB=False, workspace=gws) for G in Gs])
        a_sh = timed(lambda: q.lora_dA_shared(X, Gs, outs=dAs, workspace=dws))
        t_bytes = 2 * M * K + n * (2 * r * K + 2 * M * r)
        a_bytes = 2 * M * K + n * (2 * M * r + 2 * r * K)
        out[name] = dict(members=n,
                         T_separate_us=round(t_sep, 1), T_shared_us=round(t_sh, 1),
                         T_shared_GBps=round(t_bytes / (t_sh * 1e-6) / 1e9, 1),
                         dA_separate_us=round(a_sep, 1), dA_shared_us=round(a_sh, 1),
                         dA_shared_GBps=round(a_bytes / (a_sh * 1e-6) / 1e9, 1))
        del As, Gs, Ts, dAs, gws, dws
    del X, dY
    torch.cuda.empty_cache()
    return out


def dropout_bench(q, torch, workloads, cfg, dev, p=0.05, steps=5):
    """LoRA dropout (p = 0.05, the pages' adapter setting) on the 7B layer at
    8192 tokens: fwd + bwd of the 7 linears through the composite calls with
    and without dropout (same algorithmic FLOP), and the keep-mask kernel on
    X [8192, 4096] (HBM GB/s: X read, X_d written, mask bits written)."""
    M, r = cfg.tokens, cfg.rank
    lins = []
    for i, lin in enumerate(cfg.linears):
        N, K = lin.out_features, lin.in_features
        W = workloads.device_normal((N, K), workloads.W_STD, 99000 + i, dev)
        lins.append(dict(w=q.NF4Weight.quantize(W), N=N, K=K,
                         X=workloads.device_normal((M, K), 1.0, 99100 + i, dev, torch.bfloat16),
                         A=workloads.device_normal((r, K), workloads.LORA_STD, 99200 + i, dev, torch.bfloat16),
                         B=workloads.device_normal((N, r), workloads.LORA_STD, 99300 + i, dev, torch.bfloat16),
                         dY=workloads.device_normal((M, N), 1.0, 99400 + i, dev, torch.bfloat16)))
        del W
    flops = sum(4.0 * M * L["N"] * L["K"] + 6.0 * M * r * (L["N"] + L["K"]) for L in lins)

    def plain():
        for L in lins:
            Y, T = q.linear_fwd(L["X"], L["w"], L["A"], L["B"], cfg.scale)
            q.linear_bwd(L["dY"], L["X"], T, L["w"], L["A"], L["B"], cfg.scale)

    def dropped():
        for i, L in enumerate(lins):
            Y, T, keep = q.linear_fwd_dropout(L["X"], L["w"], L["A"], L["B"], cfg.scale, p, 7 + i)
            q.linear_bwd_dropout(L["dY"], L["X"], T, L["w"], L["A"], L["B"], cfg.scale, p, keep)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_plain = timed(plain, steps)
    ms_drop = timed(dropped, steps)
    X = lins[0]["X"]
    mask_us = timed(lambda: q.dropout_mask(X, p, 1), 20) * 1e3
    nbytes = X.numel() * 2 * 2 + X.numel() / 8
    del lins, X
    torch.cuda.empty_cache()
    return dict(p=p, plain_ms_per_step=round(ms_plain, 3), dropout_ms_per_step=round(ms_drop, 3),
                plain_TFLOPs=round(flops / (ms_plain * 1e-3) / 1e12, 1),
                dropout_TFLOPs=round(flops / (ms_drop * 1e-3) / 1e12, 1),
                mask_us_8192x4096=round(mask_us, 1), mask_GBps=round(nbytes / (mask_us * 1e-6) / 1e9, 1),
                note="composite calls (workspaces allocated by the Python binding each call)")


def layer_bench(q, torch, workloads, cfg, dev, tokens, warmup=1, steps=3, mode="deq"):
    """fwd + bwd of all linears of one layer of `cfg` at `tokens` tokens."""
    layers = [Layer(q, torch, workloads, lin, tokens, cfg.rank, 1000 * cfg.index + 10 * i, dev)
              for i, lin in enumerate(cfg.linears)]
    flops = sum(L.flops for L in layers)
    for _ in range(warmup):
        run_step(q, torch, layers, cfg.scale, mode=mode)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run_step(q, torch, layers, cfg.scale, mode=mode)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del layers
    torch.cuda.empty_cache()
    return dict(tokens=tokens, ms_per_step=round(ms, 3), step_flops=flops,
                TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1), frac_bf16_peak=round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4))


def dequantize_bench(q, torch, workloads, cfg, dev, reps=20, grouped=False):
    """Standalone dequantization (packed codes + constants -> bf16) of the 7
    weights of a layer, over 4 weight sets (> the 256 MB Infinity Cache),
    captured once in a HIP graph with preallocated outputs and replayed: one
    qlora_dequantize_nf4 call per weight, or (grouped) one
    qlora_dequantize_nf4_group call per layer.  Algorithmic bytes per
    parameter: 1/2 (codes) + 1/64 (constant codes) + 4/16384 (group scales)
    read, 2 (bf16) written."""
    import ctypes
    from bit_nf4_quantized_absmax_amd._capi import NF4WeightStruct
    sets, outs = [], []
    for si in range(4):
        ws = []
        for li, lin in enumerate(cfg.linears):
            W = workloads.device_normal((lin.out_features, lin.in_features), workloads.W_STD, 97000 + 100 * si + li, dev)
            ws.append(q.NF4Weight.quantize(W))
            del W
        sets.append([w.struct() for w in ws] + [ws])
        outs.append([torch.empty(l.out_features, l.in_features, dtype=torch.bfloat16, device=dev) for l in cfg.linears])
    lib = q.lib()

    groups = []
    for si in range(4):
        sts = sets[si][:-1]
        groups.append(((NF4WeightStruct * len(sts))(*sts),
                       (ctypes.c_void_p * len(sts))(*[o.data_ptr() for o in outs[si]])))

    def run(stream):
        for si in range(4):
            if grouped:
                rc = lib.qlora_dequantize_nf4_group(len(outs[si]), groups[si][0], groups[si][1], stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("qlora_dequantize_nf4_group failed: %d" % rc)
                continue
            for st, o in zip(sets[si][:-1], outs[si]):
                rc = lib.qlora_dequantize_nf4(ctypes.byref(st), o.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("qlora_dequantize_nf4 failed: %d" % rc)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run(stream)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record()
    for i in range(reps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 / 4 for i in range(reps))
    us = evs[0].elapsed_time(evs[-1]) * 1e3 / (4 * reps)
    params = sum(l.out_features * l.in_features for l in cfg.linears)
    nbytes = params * (0.5 + 1 / 64 + 4 / 16384 + 2)
    del graph, sets, outs
    torch.cuda.empty_cache()
    return dict(us_per_layer=round(us, 2), median_us=round(per[reps // 2], 2), min_us=round(per[0], 2),
                params=int(params), GBps=round(nbytes / (us * 1e-6) / 1e9, 1),
                frac_hbm=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                launches_per_layer=1 if grouped else len(cfg.linears))


def small_config_bench(q, torch, workloads, cfg, dev, reps=20):
    """The small parity configuration (one linear): quantize, forward and
    backward, eager calls; launch-bound at this size, reported for reference."""
    lin = cfg.linears[0]
    N, K, M, r = lin.out_features, lin.in_features, cfg.tokens, cfg.rank
    W = workloads.device_normal((N, K), workloads.W_STD, 98000, dev)
    bf = torch.bfloat16
    X = workloads.device_normal((M, K), 1.0, 98001, dev, bf)
    A = workloads.device_normal((r, K), workloads.LORA_STD, 98002, dev, bf)
    B = workloads.device_normal((N, r), workloads.LORA_STD, 98003, dev, bf)
    dY = workloads.device_normal((M, N), 1.0, 98004, dev, bf)
    w = q.NF4Weight.quantize(W)
    Y, T = q.linear_fwd(X, w, A, B, cfg.scale)

    def med(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return round(sorted(ts)[reps // 2], 2)

    return dict(workload=cfg.name, quantize_us=med(lambda: q.NF4Weight.quantize(W)),
                fwd_us=med(lambda: q.linear_fwd(X, w, A, B, cfg.scale)),
                bwd_us=med(lambda: q.linear_bwd(dY, X, T, w, A, B, cfg.scale)),
                fwd_bwd_flops=linear_flops(M, N, K, r),
                note="median of %d eager calls each (workspaces and outputs allocated by the binding)" % reps)


def codec_cpu_baseline(workloads, cfg):
    """The codec oracle (single-threaded NumPy) on one weight of the largest
    shape of `cfg` (drawn on the host, not timed), extrapolated to all of
    its layers by parameter count."""
    from oracle import nf4
    lin = max(cfg.linears, key=lambda l: l.out_features * l.in_features)
    W = workloads.weight((lin.out_features, lin.in_features), 99000)
    t0 = time.perf_counter()
    nf4.quantize(W)
    sec = time.perf_counter() - t0
    params = W.size
    total = cfg.layers * sum(l.out_features * l.in_features for l in cfg.linears)
    return dict(kind="oracle", cores=1, params_per_s=round(params / sec, 1),
                GBps=round(params * (4 + 0.5 + 1 / 64 + 4 / 16384) / sec / 1e9, 3),
                extrapolated_ms_all_layers=round(total / (params / sec) * 1e3, 1),
                sample="oracle quantize of one %s weight (%d x %d, %.1f s), extrapolated x %d layers by parameter count"
                       % (lin.name, lin.out_features, lin.in_features, sec, cfg.layers))


def model_quantize_bench(q, torch, workloads, cfg, dev):
    """Quantize every layer of a multi-layer config, one grouped call
    (qlora_quantize_nf4_group) per layer, weights drawn on the device layer by
    layer (the draws are not timed)."""
    ms = 0.0
    params = 0
    stored = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for layer in range(cfg.layers):
        Ws = [W for _, W in workloads.device_layer_weights(cfg, layer, dev)]
        torch.cuda.synchronize()
        e0.record()
        ws = q.quantize_group(Ws)
        e1.record()
        torch.cuda.synchronize()
        ms += e0.elapsed_time(e1)
        for W, w in zip(Ws, ws):
            params += W.numel()
            stored += w.packed.numel() + w.code8.numel() + 4 * w.c2.numel() + 4 * w.mean.numel()
        del Ws, ws
    torch.cuda.empty_cache()
    nbytes = params * (4 + 0.5 + 1 / 64 + 4 / 16384)
    return dict(layers=cfg.layers, params=int(params), ms_total=round(ms, 2), GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
                stored_bytes=int(stored), bits_per_param=round(8.0 * stored / params, 6),
                note="weights drawn on the device per layer (not timed); includes workspace allocation by the Python binding")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_nf4_quantized_absmax_amd as q
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 18                 # float32 elements
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    if args.small_m_only:
        c2 = workloads.CONFIGS[2]
        pats = ("per_linear", "grouped") if args.small_m_pattern == "both" else (args.small_m_pattern,)
        sm = small_m_bench(q, torch, workloads, c2, dev, reps=5 if args.small_m_eager else 200,
                           graphs=not args.small_m_eager, patterns=pats)
        print(json.dumps(dict(metric="small-M dequant forward GB/s (7B layer, 7 linears, 4 weight sets)",
                              unit="GB/s", data="synthetic", small_m=sm)), flush=True)
        return
    if args.vendor_gemm_only:
        c1 = workloads.CONFIGS[1]
        print(json.dumps(dict(metric="dequantized-weight matmul vs vendor bf16 GEMM (7B shapes, 8192 tokens)",
                              unit="TFLOP/s", data="synthetic",
                              note="min over 3 rounds of 10 launches each, alternating; FLOP = 2 M N K for both",
                              vendor_gemm=vendor_gemm_bench(q, torch, workloads, c1, dev))), flush=True)
        return
    if args.codec_only:
        c1 = workloads.CONFIGS[1]
        print(json.dumps(dict(metric="NF4 codec GB/s (7B layer, 7 weights, 4 weight sets)", unit="GB/s",
                              data="synthetic", quantize=quantize_bench(q, torch, workloads, c1, dev),
                              quantize_grouped=quantize_bench(q, torch, workloads, c1, dev, grouped=True),
                              dequantize=dequantize_bench(q, torch, workloads, c1, dev),
                              dequantize_grouped=dequantize_bench(q, torch, workloads, c1, dev, grouped=True))),
              flush=True)
        return
    cfg = workloads.CONFIGS[1]
    scale = cfg.scale
    log("building inputs for", cfg.name)
    layers = [Layer(q, torch, workloads, lin, cfg.tokens, cfg.rank, 1000 * cfg.index + 10 * i, dev)
              for i, lin in enumerate(cfg.linears)]
    step_flops = sum(L.flops for L in layers)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        run_step(q, torch, layers, scale, mode=args.matmul)
    torch.cuda.synchronize()
    log("warmup done; timing %d steps" % args.steps)

    events = {"fwd": [], "dx": []}
    t0 = time.perf_counter()
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    gev[0].record()
    for i in range(args.steps):
        run_step(q, torch, layers, scale, events, mode=args.matmul)
        gev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = gev[0].elapsed_time(gev[-1]) / args.steps
    step_ms = sorted(gev[i].elapsed_time(gev[i + 1]) for i in range(args.steps))
    tflops = step_flops / (ms_step * 1e-3) / 1e12
    log("step %.3f ms  %.1f TFLOP/s (wall %.3f s)" % (ms_step, tflops, wall))

    kern = {}
    for key, evs in events.items():
        tot_ms = sum(a.elapsed_time(b) for a, b, _ in evs)
        if key == "dequant":   # HBM-bound: algorithmic bytes (codes, constants, mean read; bf16 written)
            nbytes = sum(L.w.nbytes() + 2 * L.N * L.K for _, _, grp in evs for L in grp)
            kern[key] = dict(launches=len(evs), avg_us=tot_ms * 1e3 / len(evs), bytes_per_launch=nbytes / len(evs),
                             total_ms=tot_ms)
            continue
        flops = sum((L.fwd_mm_flops if key == "fwd" else L.dx_mm_flops) for _, _, grp in evs for L in grp)
        kern[key] = dict(launches=len(evs), avg_us=tot_ms * 1e3 / len(evs),
                         flops_per_launch=flops / len(evs), total_ms=tot_ms)
    dom_key = max((k for k in kern if k != "dequant"), key=lambda k: kern[k]["total_ms"])
    dom = kern[dom_key]
    achieved = dom["flops_per_launch"] / (dom["avg_us"] * 1e-6) / 1e12
    if args.matmul == "deq":
        dom_kernel = "qlora::k_matmul_pre<false, true>" if dom_key == "fwd" else "qlora::k_matmul_pre<true, true>"
    else:
        dom_kernel = "qlora::k_matmul<false, false>" if dom_key == "fwd" else "qlora::k_matmul<true, false>"
    roofline = dict(bound="mfma", achieved=round(achieved, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_PEAK_TFLOPS, 4), traffic=recorded_traffic(dom_kernel),
                    traffic_unit="HBM bytes per launch (PMC FETCH_SIZE + WRITE_SIZE, copy-scaled), recorded in "
                                 "profiles/matmul_llama7b_m8192_hbm_traffic.md, not measured by this run; null "
                                 "once the matmul sources differ from the recorded hash",
                    kernel=dom_kernel + (" (forward)" if dom_key == "fwd" else " (dX)"),
                    avg_launch_us=round(dom["avg_us"], 2),
                    flops_per_launch=dom["flops_per_launch"])
    other = {}
    for k, v in kern.items():
        rec = dict(avg_us=round(v["avg_us"], 2), launches_per_step=v["launches"] // args.steps,
                   share_of_step=round(v["total_ms"] / args.steps / ms_step, 3))
        if "flops_per_launch" in v:
            rec["TFLOPs"] = round(v["flops_per_launch"] / (v["avg_us"] * 1e-6) / 1e12, 1)
        else:
            rec["GBps"] = round(v["bytes_per_launch"] / (v["avg_us"] * 1e-6) / 1e9, 1)
        other[k] = rec

    extras = {}
    if not args.no_extras:
        del layers
        torch.cuda.empty_cache()
        log("small-M forward")
        extras["small_m"] = small_m_bench(q, torch, workloads, workloads.CONFIGS[2], dev)
        log("quantize")
        extras["quantize"] = quantize_bench(q, torch, workloads, cfg, dev)
        extras["quantize_grouped"] = quantize_bench(q, torch, workloads, cfg, dev, grouped=True)
        log("dequantize")
        extras["dequantize"] = dequantize_bench(q, torch, workloads, cfg, dev)
        extras["dequantize_grouped"] = dequantize_bench(q, torch, workloads, cfg, dev, grouped=True)
        log("small parity configuration")
        extras["small_config"] = small_config_bench(q, torch, workloads, workloads.CONFIGS[0], dev)
        log("4-bit types")
        extras["q4_types"] = q4_types_bench(q, torch, workloads, dev)
        log("shared-input LoRA products")
        extras["shared_input"] = shared_input_bench(q, torch, workloads, dev)
        log("LoRA dropout")
        extras["dropout"] = dropout_bench(q, torch, workloads, cfg, dev)
        log("33B layer")
        c3 = workloads.CONFIGS[3]
        extras["llama33b_layer"] = layer_bench(q, torch, workloads, c3, dev, c3.tokens)
        log("65B: quantize 80 layers, one layer at 16384 tokens")
        c4 = workloads.CONFIGS[4]
        extras["llama65b"] = dict(quantize=model_quantize_bench(q, torch, workloads, c4, dev),
                                  layer=layer_bench(q, torch, workloads, c4, dev, c4.tokens))
        if not args.no_cpu:
            log("codec oracle baseline (one 65B weight)")
            extras["llama65b"]["quantize"]["cpu_baseline"] = codec_cpu_baseline(workloads, c4)

    cpu = None
    if not args.no_cpu:
        log("cpu oracle baseline on %d tokens" % args.cpu_tokens)
        cpu = cpu_baseline(cfg, args.cpu_tokens)

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights quantized to NF4+DQ; N(0,1) bf16 activations)",
        "config": {"workload": "llama7b_layer_7linears_fwd_bwd", "tokens": cfg.tokens, "rank": cfg.rank,
                   "alpha": cfg.alpha, "step_flops": step_flops,
                   "shapes": "q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008 (N x K)",
                   "matmul": ("the layer's 7 weights dequantized to bf16 once per step (one grouped launch, "
                              "timed), both matmuls reading those copies" if args.matmul == "deq" else
                              "NF4 codes expanded inside every matmul tile"),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": other,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
