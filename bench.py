#!/usr/bin/env python3
"""Throughput of the ConvRot W8A8 INT8 linear forward on one MI355X.

One step = one forward call through the C ABI over one batch of synthetic
input already resident in HBM.  The default workload is the fused-QKV-shaped
linear M=38656 tokens, K=5376, N=16128, b=128, bf16 activations drawn from
Student-t(4), bf16 output: one ``convrot_linear_forward`` = the rotate +
rowwise INT8 quantise kernel, then the INT8 MFMA GEMM with the fused dequant
epilogue.  ``--workload`` also takes the other workloads (``linear_4096``,
``mlp_16384``: up GEMM, rotquant of g = GELU(u) (the GELU applied as u is
loaded), down GEMM; ``lowrank_38656``:
rotquant, GEMM to r with H rotated and requantised in its epilogue, GEMM to N).  Weights are prepared
(rotated, quantised, packed) before the timed region, as at model load.

Prints ONE JSON line: effective INT8 TOPS (algorithmic 2*M*N*K summed over the
projections, per step time); ``roofline`` for the dominant kernel (its
algorithmic ops or bytes per launch over its average launch time, timed with
HIP events recorded on the stream the kernel runs on); ``kernels`` with every
kernel of the step; ``roofline_rotquant`` for the first rotate+quantise pass;
``cpu_baseline``, the CPU oracle timed on a bounded sample of the same rows,
which also checks the benchmarked outputs on those rows; and ``ceilings``,
the INT8 MFMA rate and the streaming HBM rate measured with the library's
probes, against which ``frac_of_measured_ceiling`` is given.

    python bench.py [--steps 20] [--warmup W] [--workload qkv_38656]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective INT8 TOPS & % INT8 MFMA peak, ConvRot linear M=38656 K=5376"
PEAK_INT8_TOPS = 5033.2      # MI355X dense INT8 MFMA: 256 CUs x 8192 ops/clk x 2.4 GHz (5.0 POP/s)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
RIDGE = PEAK_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # ops per byte
CSRC = os.path.join(ROOT, "w8a8_int8_rotated_amd", "csrc")
SOURCES = {"gemm_i8": os.path.join(CSRC, "gemm_i8.hip"),
           "rotquant": os.path.join(CSRC, "rotquant.hip")}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps before the timed ones (default: as many as take "
                        "--warmup-seconds, at least 5)")
    p.add_argument("--warmup-seconds", type=float, default=0.5,
                   help="GPU time of the default warm-up: the shader clock settles over the "
                        "first tenths of a second of sustained load")
    p.add_argument("--workload", default="qkv_38656")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time replays of the step captured in a HIP graph")
    p.add_argument("--evict-mib", type=int, default=None,
                   help="write this many MiB of scratch before each timed step (cold caches; "
                        "default 512 when the step's working set is under 512 MiB, so the 256 MB "
                        "last-level cache cannot hold it from one step to the next, else 0)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured MFMA and HBM ceilings")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run a plain device copy of this size first (counter calibration)")
    return p.parse_args()


def working_set_bytes(w):
    """Bytes a step touches: the bf16 input, every code matrix and weight,
    every intermediate and the output."""
    ob = 4 if w.out == "f32" else 2
    lin = lambda M, K, N, o: 2 * M * K + M * K + N * K + o * M * N
    if w.kind == "lowrank":
        return lin(w.M, w.K, w.rank, 2) + lin(w.M, w.rank, w.N, ob) - 2 * w.M * w.rank
    if w.kind in ("mlp", "swiglu"):
        up = 2 * w.ffn if w.kind == "swiglu" else w.ffn
        return lin(w.M, w.K, up, 2) + lin(w.M, w.ffn, w.N, ob)
    return lin(w.M, w.K, w.N, ob)


def warmup_steps(args, step, torch):
    """The untimed steps: --warmup of them, or by default as many as take
    --warmup-seconds of GPU time (at least 5); the count is what the JSON
    line reports as warmup."""
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(5):
            step()
        n += 5
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= args.warmup_seconds:
            break
    args.warmup = n


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", txt)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not sha or not val or sha.group(1) != source_sha(SOURCES[kernel]):
        return None
    return float(val.group(1))


class Stage:
    """One kernel launch of the step, with its algorithmic cost."""

    def __init__(self, name, kernel, fn, ops, nbytes, src=None):
        self.name, self.kernel, self.fn = name, kernel, fn
        self.ops, self.bytes = float(ops), float(nbytes)
        self.src = src                    # the tensor a rotquant stage reads
        self.bound = "mfma" if self.ops / self.bytes > RIDGE else "hbm"
        self.ms = None

    def roofline(self, workload):
        if self.bound == "mfma":
            achieved = self.ops / (self.ms * 1e-3) / 1e12
            peak, unit = PEAK_INT8_TOPS, "TFLOP/s"
        else:
            achieved = self.bytes / (self.ms * 1e-3) / 1e9
            peak, unit = PEAK_HBM_GBS, "GB/s"
        return {
            "kernel": self.name, "bound": self.bound, "achieved": round(achieved, 2),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(self.kernel, workload),
            "ops_per_launch": self.ops, "bytes_per_launch": self.bytes,
            "avg_launch_ms": round(self.ms, 5),
        }


def rq_bytes(M, K):
    return 3.0 * M * K + 4.0 * M          # bf16 in, codes out, row scale


def gemm_cost(M, N, K, out_bytes=2, bias=False):
    ops = 2.0 * M * N * K
    nbytes = M * K + N * K + out_bytes * M * N + 4.0 * (M + N) + (4.0 * N if bias else 0)
    return ops, nbytes


def setup(w, cr, torch, np, dev):
    """Device inputs, prepared weights, the step and its stages."""
    b = w.block
    x = w.activations()
    X = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    host = {"x": x}
    stream = torch.cuda.current_stream()
    out_dt = torch.bfloat16 if w.out == "bf16" else torch.float32
    ob = 2 if w.out == "bf16" else 4

    def prep(W):
        Wd = torch.from_numpy(W).to(dev)
        pw = cr.convrot_linear_prepare_weights(Wd, b)
        torch.cuda.synchronize()
        return pw

    M, K = w.M, w.K
    if w.kind == "linear":
        W = w.weight()
        bias = w.bias()
        host.update(W=W, bias=bias)
        pw = prep(W)
        bias_d = None if bias is None else torch.from_numpy(bias).to(dev)
        N = w.N
        Y = torch.empty((M, N), dtype=out_dt, device=dev)
        ws = torch.empty(cr.convrot_linear_workspace_bytes(M, K, N, b), dtype=torch.uint8,
                         device=dev)
        qx = torch.empty((cr.padded_rows(M), K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)

        def step():
            cr.convrot_linear_forward(X, pw, bias=bias_d, out=Y, workspace=ws)

        stages = [
            Stage("rotquant (FWHT + absmax + INT8 codes)", "rotquant",
                  lambda: cr.convrot_rotate_quantize(X, b, q=qx, s=sx, stream=stream),
                  0.0, rq_bytes(M, K), src=X),
            Stage("gemm_i8 (INT8 MFMA + dequant epilogue)", "gemm_i8",
                  lambda: cr.convrot_gemm_dequant(qx, sx, pw, bias=bias_d, out=Y, stream=stream),
                  *gemm_cost(M, N, K, ob, bias is not None)),
        ]
        ops = 2.0 * M * N * K
    elif w.kind == "lowrank":
        A, B = w.weight("w"), w.weight("w2")
        host.update(A=A, B=B)
        pa, pb = prep(A), prep(B)
        r, N = w.rank, w.N
        Y = torch.empty((M, N), dtype=out_dt, device=dev)
        ws = torch.empty(cr.lowrank_convrot_workspace_bytes(M, K, r, N, b), dtype=torch.uint8,
                         device=dev)
        qx = torch.empty((cr.padded_rows(M), K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        H = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        qh = torch.empty((cr.padded_rows(M), r), dtype=torch.int8, device=dev)
        sh = torch.empty(M, dtype=torch.float32, device=dev)

        def step():
            cr.lowrank_convrot_forward(X, pa, pb, out=Y, workspace=ws)

        stages = [
            Stage("rotquant X", "rotquant",
                  lambda: cr.convrot_rotate_quantize(X, b, q=qx, s=sx, stream=stream),
                  0.0, rq_bytes(M, K), src=X),
        ]
        if b in (64, 128) and r <= 512:
            # the library's fused factor 1: H is rotated and requantised in
            # the GEMM epilogue and never written
            stages.append(Stage(
                "lowrank_f1 factor 1 + rotate/requantise H (K -> r)", "gemm_i8",
                lambda: cr.convrot_lowrank_factor1(qx, sx, pa, q_h=qh, s_h=sh, stream=stream),
                *gemm_cost(M, r, K, out_bytes=1)))
        else:
            stages += [
                Stage("gemm_i8 factor 1 (K -> r)", "gemm_i8",
                      lambda: cr.convrot_gemm_dequant(qx, sx, pa, out=H, stream=stream),
                      *gemm_cost(M, r, K)),
                Stage("rotquant H", "rotquant",
                      lambda: cr.convrot_rotate_quantize(H, b, q=qh, s=sh, stream=stream),
                      0.0, rq_bytes(M, r)),
            ]
        stages += [
            Stage("gemm_i8 factor 2 (r -> N)", "gemm_i8",
                  lambda: cr.convrot_gemm_dequant(qh, sh, pb, out=Y, stream=stream),
                  *gemm_cost(M, N, r, ob)),
        ]
        ops = 2.0 * M * r * (K + N)
    elif w.kind == "mlp":
        Wu, Wd = w.weight("w"), w.weight("w2")
        host.update(Wu=Wu, Wd=Wd)
        pu, pd = prep(Wu), prep(Wd)
        F, N = w.ffn, w.N
        Y = torch.empty((M, N), dtype=out_dt, device=dev)
        ws = torch.empty(cr.convrot_mlp_workspace_bytes(M, K, F, N, b), dtype=torch.uint8,
                         device=dev)
        qx = torch.empty((cr.padded_rows(M), K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        G = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        qg = torch.empty((cr.padded_rows(M), F), dtype=torch.int8, device=dev)
        sg = torch.empty(M, dtype=torch.float32, device=dev)

        def step():
            cr.convrot_mlp_forward(X, pu, pd, out=Y, workspace=ws)

        # The stages of the path convrot_mlp_forward takes for this F: GELU
        # applied by rotquant as it loads u (the hook accepts the flag for
        # exactly those F), else in the up projection's epilogue.
        try:
            cr.convrot_rotate_quantize(G[:1], b, gelu=True)
            gelu_on_load = True
        except cr.ConvRotError as e:
            if e.status != cr.EUNSUPPORTED:
                raise
            gelu_on_load = False
        if gelu_on_load:
            up = Stage("gemm_i8 up (K -> F)", "gemm_i8",
                       lambda: cr.convrot_gemm_dequant(qx, sx, pu, out=G, stream=stream),
                       *gemm_cost(M, F, K))
            rqg = Stage("rotquant g = GELU(u) on load", "rotquant",
                        lambda: cr.convrot_rotate_quantize(G, b, q=qg, s=sg, stream=stream,
                                                           gelu=True),
                        0.0, rq_bytes(M, F))
        else:
            up = Stage("gemm_i8 up + GELU (K -> F)", "gemm_i8",
                       lambda: cr.convrot_gemm_dequant(qx, sx, pu, out=G, gelu=True,
                                                       stream=stream),
                       *gemm_cost(M, F, K))
            rqg = Stage("rotquant g", "rotquant",
                        lambda: cr.convrot_rotate_quantize(G, b, q=qg, s=sg, stream=stream),
                        0.0, rq_bytes(M, F))
        stages = [
            Stage("rotquant X", "rotquant",
                  lambda: cr.convrot_rotate_quantize(X, b, q=qx, s=sx, stream=stream),
                  0.0, rq_bytes(M, K), src=X),
            up,
            rqg,
            Stage("gemm_i8 down (F -> N)", "gemm_i8",
                  lambda: cr.convrot_gemm_dequant(qg, sg, pd, out=Y, stream=stream),
                  *gemm_cost(M, N, F, ob)),
        ]
        ops = 2.0 * M * F * (K + N)
    elif w.kind == "swiglu":
        Wgu, Wd = w.weight("w"), w.weight("w2")
        host.update(Wgu=Wgu, Wd=Wd)
        bd = w.down_block
        pgu = cr.convrot_swiglu_prepare(torch.from_numpy(Wgu).to(dev), b)
        pd = cr.convrot_linear_prepare_weights(torch.from_numpy(Wd).to(dev), bd)
        torch.cuda.synchronize()
        F, N = w.ffn, w.N
        Y = torch.empty((M, N), dtype=out_dt, device=dev)
        ws = torch.empty(cr.convrot_swiglu_mlp_workspace_bytes(M, K, F, N, b, bd),
                         dtype=torch.uint8, device=dev)
        qx = torch.empty((cr.padded_rows(M), K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        G = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        qg = torch.empty((cr.padded_rows(M), F), dtype=torch.int8, device=dev)
        sg = torch.empty(M, dtype=torch.float32, device=dev)

        def step():
            cr.convrot_swiglu_mlp_forward(X, pgu, pd, out=Y, workspace=ws)

        fc1_ops, fc1_bytes = gemm_cost(M, 2 * F, K)
        fc1_bytes -= 2.0 * M * F          # writes g [M, F], not the [M, 2F] fc1 output
        stages = [
            Stage("rotquant X", "rotquant",
                  lambda: cr.convrot_rotate_quantize(X, b, q=qx, s=sx, stream=stream),
                  0.0, rq_bytes(M, K), src=X),
            Stage("gemm_i8 fc1 gate|up + SwiGLU epilogue (K -> 2F, writes g)", "gemm_i8",
                  lambda: cr.convrot_gemm_dequant(qx, sx, pgu, out=G, swiglu=True, stream=stream),
                  fc1_ops, fc1_bytes),
            Stage(f"rotquant g (b={bd})", "rotquant",
                  lambda: cr.convrot_rotate_quantize(G, bd, q=qg, s=sg, stream=stream),
                  0.0, rq_bytes(M, F)),
            Stage("gemm_i8 down (F -> N)", "gemm_i8",
                  lambda: cr.convrot_gemm_dequant(qg, sg, pd, out=Y, stream=stream),
                  *gemm_cost(M, N, F, ob)),
        ]
        ops = 2.0 * M * F * (2 * K + N)
    else:
        raise SystemExit(f"unknown workload kind {w.kind}")
    return step, stages, ops, Y, host


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the forward shards along tokens with no exchange, "
                                   "see the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (MI355X); none is visible")
    from w8a8_int8_rotated_amd import convrot as cr
    from w8a8_int8_rotated_amd import workloads as wl

    cr.library()
    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: 3 x {args.copy_probe_mib} MiB device copies")

    t0 = time.time()
    step, stages, ops, Y, host = setup(w, cr, torch, np, dev)
    stream = torch.cuda.current_stream()
    log(f"{w.name}: inputs generated and weights prepared in {time.time() - t0:.1f}s")

    if args.evict_mib is None:
        args.evict_mib = 512 if working_set_bytes(w) < (512 << 20) else 0
    warmup_steps(args, step, torch)
    if args.graph:
        # the step recorded once into a HIP graph and replayed: one launch per
        # step instead of one per kernel (the calls allocate, synchronise and
        # clear nothing, so they record as they run)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` forward calls between two events ----
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    scratch = (torch.empty(args.evict_mib << 20, dtype=torch.uint8, device=dev)
               if args.evict_mib else None)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if scratch is None:
        evs[0].record(stream)
        for i in range(args.steps):
            step()
        evs[-1].record(stream)
        torch.cuda.synchronize()
        total_ms = evs[0].elapsed_time(evs[-1])
        wall = time.perf_counter() - wall0
        # per-step spread from a second pass with an event after each step (an
        # event between steps leaves the GPU idle for a few microseconds, so
        # the figure above has none inside it)
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        pe[0].record(stream)
        for i in range(args.steps):
            step()
            pe[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = [pe[i].elapsed_time(pe[i + 1]) for i in range(args.steps)]
    else:
        # cold caches: a scratch write evicts the last-level cache before
        # each step, outside that step's events
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.fill_(i & 0xff)
            evs[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        per_step = [evs[i].elapsed_time(ends[i]) for i in range(args.steps)]
        total_ms = sum(per_step)
        wall = time.perf_counter() - wall0
    ms_per_step = total_ms / args.steps
    srt = sorted(per_step)
    step_stats = {"median": round(srt[len(srt) // 2], 5), "min": round(srt[0], 5),
                  "p90": round(srt[min(len(srt) - 1, int(0.9 * len(srt)))], 5),
                  "cold_caches": scratch is not None,
                  "source": ("an event around each step, scratch write outside" if scratch is not None
                             else "a second pass of the same steps, an event after each")}
    tops = ops / (ms_per_step * 1e-3) / 1e12
    log(f"forward: {ms_per_step:.4f} ms/step, {tops:.1f} TOPS (wall {wall:.3f}s)")

    # ---- per-kernel durations: the step's kernels, launched through the
    # stage hooks on the same stream with HIP events between them ----
    for _ in range(2):
        for st in stages:
            st.fn()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        for i, st in enumerate(stages):
            st.fn()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    for i, st in enumerate(stages):
        st.ms = sum(e[i].elapsed_time(e[i + 1]) for e in evs) / len(evs)
    for st in stages:
        r = st.roofline(w.name)
        log(f"{st.name}: {st.ms:.4f} ms, {r['achieved']} {r['unit']} ({100 * r['frac']:.1f}%)")
    dominant = max(stages, key=lambda s: s.ms)
    first_rq = next(s for s in stages if s.kernel == "rotquant")
    # the same rotquant launched back to back on its own: in the step it runs
    # right after a GEMM whose output's dirty lines are still being written
    # back from the last-level cache, which takes HBM bandwidth from it
    for _ in range(3):
        first_rq.fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        first_rq.fn()
    e1.record(stream)
    torch.cuda.synchronize()
    rq_alone_ms = e0.elapsed_time(e1) / args.steps
    log(f"{first_rq.name} back to back on its own: {rq_alone_ms:.4f} ms, "
        f"{first_rq.bytes / (rq_alone_ms * 1e-3) / 1e9:.1f} GB/s")

    cfg = {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "block": w.block,
           "activations": "bf16 Student-t(4)" if w.x_dist == "student_t4" else "bf16 normal",
           "out": w.out, "bias": w.bias_std is not None, "seed": w.seed}
    if w.kind == "lowrank":
        cfg["rank"] = w.rank
    if w.kind in ("mlp", "swiglu"):
        cfg["ffn"] = w.ffn
    if w.kind == "swiglu":
        cfg["block_down"] = w.down_block
    if w.n_outliers():
        cfg["outlier_channels"] = w.n_outliers()
        cfg["outlier_gain"] = w.outlier_gain

    result = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": cfg,
        "inputs_sha256": {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
                          for k, v in host.items() if v is not None},
        "env": environment(torch),
        "pct_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        "step_ms": step_stats,
        "launch": "hipGraph replay" if args.graph else "eager",
        "roofline": dominant.roofline(w.name),
        "roofline_rotquant": dict(first_rq.roofline(w.name), back_to_back_alone={
            "avg_launch_ms": round(rq_alone_ms, 5),
            "achieved": round(first_rq.bytes / (rq_alone_ms * 1e-3) / 1e9, 2),
            "frac": round(first_rq.bytes / (rq_alone_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "note": "not after a GEMM: no write-back of its output competes for HBM"}),
        "kernels": [s.roofline(w.name) for s in stages],
        "cpu_baseline": None,
    }

    clk = loaded_clock(dominant, torch, stream)
    result["loaded_clock"] = clk
    if clk and dominant.bound == "mfma":
        # MFMA utilisation at the clock actually held: the INT8 rate of the
        # launch over what every CU's matrix cores deliver at that clock
        # (8,192 INT8 ops per clock per CU, the spec peak's rate at 2.4 GHz)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        cap = cus * 8192.0 * clk["gfx_mhz"] * 1e6 / 1e12
        result["roofline"]["mfma_util_at_loaded_clock"] = round(
            result["roofline"]["achieved"] / cap, 4)
        log(f"loaded clock {clk['gfx_mhz']:.0f} MHz during {dominant.name}: "
            f"{result['roofline']['achieved']:.0f} of {cap:.0f} TOPS at that clock")

    if not args.no_ceilings:
        ceil = ceilings(cr, torch, dev, stream, stages, first_rq)
        result["ceilings"] = ceil
        for r, st in ((result["roofline"], dominant), (result["roofline_rotquant"], first_rq)):
            key = ("mfma_i8_changing_operands" if st.bound == "mfma" else
                   "hbm_stream_rotquant_shape" if st.kernel == "rotquant" else
                   "hbm_write_stream")        # a GEMM bound by its output stores
            r["measured_ceiling"] = key
            r["frac_of_measured_ceiling"] = round(r["achieved"] / ceil[key]["value"], 4)

    if w.kind == "lowrank":
        result["comparison"] = {
            "dense_w8a8": dense_comparison(args, w, host, cr, torch, dev, stream, ms_per_step, Y),
            "bf16_lowrank": bf16_lowrank_comparison(args, w, host, cr, torch, dev, stream,
                                                    ms_per_step),
        }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(args, w, host, Y)

    print(json.dumps(result), flush=True)


def loaded_clock(stage, torch, stream, seconds=0.6):
    """The shader clock while `stage` runs back to back for about `seconds`:
    the host enqueues the launches, then reads the current level of the
    driver's sclk table (pp_dpm_sclk, the entry marked '*') every few
    milliseconds until they finish; the median of the middle 80% of the
    readings.  None when the table is not readable."""
    import glob
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return None

    def read_mhz():
        try:
            with open(paths[0]) as f:
                for ln in f:
                    if ln.strip().endswith("*"):
                        return float(re.search(r"(\d+)\s*Mhz", ln, re.I).group(1))
        except (OSError, AttributeError):
            return None
        return None

    n = max(8, int(seconds / max(stage.ms * 1e-3, 1e-5)))
    done = torch.cuda.Event()
    torch.cuda.synchronize()
    for _ in range(n):
        stage.fn()
    done.record(stream)
    samples = []
    while not done.query():
        v = read_mhz()
        if v is not None:
            samples.append(v)
        time.sleep(0.003)
    torch.cuda.synchronize()
    if len(samples) < 5:
        return None
    k = len(samples) // 10
    mid = sorted(samples[k:len(samples) - k])
    return {"gfx_mhz": mid[len(mid) // 2], "samples": len(samples), "launches": n,
            "kernel": stage.name, "source": "pp_dpm_sclk current level, median while the "
            "kernel runs back to back"}


def environment(torch):
    """The device and host the numbers were taken on."""
    import platform
    props = torch.cuda.get_device_properties(0)
    cpu = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       cpu)
    except OSError:
        pass
    return {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count,
            "hbm_gib": round(props.total_memory / 2**30, 1), "hip": torch.version.hip,
            "torch": torch.__version__, "host_cpu": cpu, "host_threads": os.cpu_count()}


def ceilings(cr, torch, dev, stream, stages, first_rq):
    """Ceilings measured with the library's probes, beside the spec peaks:
    the sustained INT8 MFMA rate on operands that change every round, with
    no memory traffic (the clock under a sustained INT8 load is
    power-limited), and a streaming kernel with the
    first rotquant's traffic (its input's 16-byte items in, 8 bytes out per
    item, no arithmetic), each run right after the step's last kernel, as
    rotquant runs inside the step."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    seed = torch.randint(-2**31, 2**31 - 1, (1024,), dtype=torch.int32, device=dev,
                         generator=torch.Generator(device=dev).manual_seed(0))
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    # The clock takes tens of milliseconds to settle after a change of load:
    # a few-millisecond launch right after the step measures the ramp, not the
    # rate the power limit holds.  One untimed launch of about 0.1 s first,
    # then the median of three more.
    iters = 400_000
    cr.convrot_probe_mfma_i8(iters, seed, sink, stream=stream)
    rates = []
    for _ in range(3):
        e0, e1 = ev(), ev()
        e0.record(stream)
        ops = cr.convrot_probe_mfma_i8(iters, seed, sink, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(ops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    mfma = sorted(rates)[1]

    src = first_rq.src
    n16 = src.numel() * src.element_size() // 16
    dst = torch.empty(n16 * 8, dtype=torch.uint8, device=dev)
    times = []
    for _ in range(5):
        stages[-1].fn()
        e0, e1 = ev(), ev()
        e0.record(stream)
        cr.convrot_probe_stream(src, dst, 0, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    gbs = 24.0 * n16 / (ms * 1e-3) / 1e9
    # writes only, 1 GiB (the traffic of a GEMM whose output dominates)
    wdst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    times = []
    for _ in range(5):
        stages[-1].fn()
        e0, e1 = ev(), ev()
        e0.record(stream)
        cr.convrot_probe_stream(None, wdst, 2, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    wgbs = float(1 << 30) / (sorted(times)[len(times) // 2] * 1e-3) / 1e9
    log(f"ceilings: INT8 MFMA {mfma:.0f} TOPS on changing operands; "
        f"streaming {gbs:.0f} GB/s with the rotquant traffic shape, {wgbs:.0f} GB/s writes only")
    return {
        "mfma_i8_changing_operands": {
            "value": round(mfma, 1), "unit": "TOPS",
            "frac_of_spec": round(mfma / PEAK_INT8_TOPS, 4),
            "probe": "v_mfma_i32_32x32x32_i8 rounds, one workgroup per CU, operands remixed "
                     "every round; sustained: median of 3 launches of about 0.1 s after an "
                     "untimed one"},
        "hbm_stream_rotquant_shape": {
            "value": round(gbs, 1), "unit": "GB/s",
            "frac_of_spec": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": 24.0 * n16,
            "probe": "16 B non-temporal load, 8 B store per item, grid-stride; each run right "
                     "after the step's last kernel; median of 5"},
        "hbm_write_stream": {
            "value": round(wgbs, 1), "unit": "GB/s",
            "frac_of_spec": round(wgbs / PEAK_HBM_GBS, 4), "bytes_per_launch": float(1 << 30),
            "probe": "16 B store per item over 1 GiB, grid-stride, nothing read; each run right "
                     "after the step's last kernel; median of 5"},
    }


def dense_comparison(args, w, host, cr, torch, dev, stream, lowrank_ms, Y_lowrank):
    """The dense W8A8 linear the low-rank layer approximates: W = B A formed in
    fp64, stored fp32 and prepared like any weight, run on the same
    activations and timed the same way outside the step.  Reports its TOPS,
    the low-rank step's dense-equivalent TOPS (2 M N K over the low-rank
    time), and both outputs' normwise error against the fp64 product W x on
    sampled rows."""
    import numpy as np
    A64, B64 = host["A"].astype(np.float64), host["B"].astype(np.float64)
    W64 = B64 @ A64
    W = W64.astype(np.float32)
    pw = cr.convrot_linear_prepare_weights(torch.from_numpy(W).to(dev), w.block)
    X = torch.from_numpy(host["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    Y = torch.empty((w.M, w.N), dtype=Y_lowrank.dtype, device=dev)
    ws = torch.empty(cr.convrot_linear_workspace_bytes(w.M, w.K, w.N, w.block),
                     dtype=torch.uint8, device=dev)
    run = lambda: cr.convrot_linear_forward(X, pw, out=Y, workspace=ws, stream=stream)
    for _ in range(args.warmup):
        run()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    dense_ops = 2.0 * w.M * w.N * w.K
    rows = np.sort(np.random.default_rng(99).choice(w.M, 64, replace=False))
    xf = ((host["x"][rows].astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    y64 = xf @ W64.T
    idx = torch.from_numpy(rows).to(dev)
    to64 = lambda t: t[idx].float().cpu().numpy().astype(np.float64)
    err = lambda y: float(np.linalg.norm(y - y64) / np.linalg.norm(y64))
    e_dense, e_lr = err(to64(Y)), err(to64(Y_lowrank))
    log(f"dense W8A8 comparison (W = B A): {ms:.4f} ms, {dense_ops / ms / 1e9:.1f} TOPS; "
        f"low-rank step {lowrank_ms:.4f} ms = {dense_ops / lowrank_ms / 1e9:.1f} dense-equivalent "
        f"TOPS; normwise error vs fp64 W x: dense {e_dense:.4f}, low-rank {e_lr:.4f}")
    return {"variant": "dense W8A8 linear, W = B A (fp64 product stored fp32), same X",
            "ms_per_step": round(ms, 5), "tops": round(dense_ops / ms / 1e9, 2),
            "lowrank_dense_equivalent_tops": round(dense_ops / lowrank_ms / 1e9, 2),
            "lowrank_speedup": round(ms / lowrank_ms, 3),
            "normwise_err_vs_fp64": {"dense": round(e_dense, 5), "lowrank": round(e_lr, 5),
                                     "rows": 64}}


def bf16_lowrank_comparison(args, w, host, cr, torch, dev, stream, int8_ms):
    """The same low-rank layer with bf16 factors and no rotation or
    quantisation (the variant where the low-rank linears stay bf16), timed
    the same way outside the step, for comparison only."""
    import numpy as np
    from w8a8_int8_rotated_amd import workloads as wl
    to_b = lambda a: torch.from_numpy(wl.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).to(dev)
    X = torch.from_numpy(host["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    A, B = to_b(host["A"]), to_b(host["B"])
    Y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(cr.lowrank_bf16_workspace_bytes(w.M, w.rank), dtype=torch.uint8,
                     device=dev)
    run = lambda: cr.lowrank_bf16_forward(X, A, B, out=Y, workspace=ws, stream=stream)
    for _ in range(args.warmup):
        run()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = 2.0 * w.M * w.rank * (w.K + w.N)
    log(f"bf16 low-rank comparison: {ms:.4f} ms, {flops / ms / 1e9:.1f} TFLOP/s")
    return {"variant": "bf16 factors, no rotation or quantisation", "ms_per_step": round(ms, 5),
            "tflops_bf16": round(flops / ms / 1e9, 2),
            "int8_speedup": round(ms / int8_ms, 3)}


def cpu_baseline(args, w, host, Y):
    """The oracle (as it stands) on the host cores, stage by stage: weight
    preparation (every weight, in full), rotate+quantise of every row, and the
    whole forward (rotate+quantise, INT32 contraction, epilogue) on a bounded,
    seeded sample of rows, which also checks the benchmarked GPU outputs on
    those rows.  For the two small linear workloads the whole forward runs on
    every row, on all threads and on one."""
    import numpy as np
    import oracle

    M, b, x = w.M, w.block, host["x"]
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    if w.kind == "linear":
        qw, sw = oracle.prepare_weights(host["W"], b)
        run = lambda rows: oracle.linear_forward(x[rows], qw, sw, b, bias=host["bias"], out=w.out)
        ops_row = 2.0 * w.N * w.K
    elif w.kind == "lowrank":
        qa, sa = oracle.prepare_weights(host["A"], b)
        qb, sb = oracle.prepare_weights(host["B"], b)
        run = lambda rows: oracle.lowrank_forward(x[rows], qa, sa, qb, sb, b, out=w.out)
        ops_row = 2.0 * w.rank * (w.K + w.N)
    elif w.kind == "swiglu":
        qgu, sgu = oracle.prepare_weights(host["Wgu"], b)
        qd, sd = oracle.prepare_weights(host["Wd"], w.down_block)
        run = lambda rows: oracle.swiglu_mlp_forward(x[rows], qgu, sgu, qd, sd, b, w.down_block,
                                                     out=w.out)
        ops_row = 2.0 * w.ffn * (2 * w.K + w.N)
    else:
        qu, su = oracle.prepare_weights(host["Wu"], b)
        qd, sd = oracle.prepare_weights(host["Wd"], b)
        run = lambda rows: oracle.mlp_forward(x[rows], qu, su, qd, sd, b, out=w.out)
        ops_row = 2.0 * w.ffn * (w.K + w.N)
    prep_s = time.perf_counter() - t0
    # rotate + quantise of every row of X (the first stage of the forward)
    t0 = time.perf_counter()
    oracle.rotate_quantize(x, b, "bf16")
    rq_s = time.perf_counter() - t0
    rq_gbs = (3.0 * M * w.K + 4.0 * M) / rq_s / 1e9

    rng = np.random.default_rng(1234)
    full = w.name in ("tiny", "linear_4096")
    if full:
        rows = np.arange(M)
    else:
        # the time per row, from probes large enough that a call's fixed cost
        # (threads, intermediates) does not dominate
        k = 16
        while True:
            probe = np.sort(rng.choice(M, min(M, k), replace=False))
            t0 = time.perf_counter()
            run(probe)
            dt_probe = time.perf_counter() - t0
            if dt_probe >= 0.25 or k >= M:
                break
            k *= 4
        per_row = dt_probe / len(probe)
        n = int(min(M, max(64, args.cpu_seconds / max(per_row, 1e-9))))
        rows = np.sort(rng.choice(M, n, replace=False))
        rows[0], rows[-1] = 0, M - 1
        rows = np.unique(rows)
    t0 = time.perf_counter()
    y_ref = run(rows)
    dt = time.perf_counter() - t0
    cpu_tops = ops_row * len(rows) / dt / 1e12
    one = None
    if full:
        oracle.set_num_threads(1)
        try:
            t0 = time.perf_counter()
            run(rows)
            dt1 = time.perf_counter() - t0
        finally:
            oracle.set_num_threads(threads)
        one = {"seconds": round(dt1, 2), "value": round(ops_row * len(rows) / dt1 / 1e12, 5),
               "unit": "TOPS", "cores": 1}
    log(f"oracle: weight prep {prep_s:.1f}s; rotate+quantise of all {M} rows {rq_s:.2f}s "
        f"({rq_gbs:.2f} GB/s); forward on {len(rows)} rows {dt:.2f}s = {cpu_tops:.4f} TOPS on "
        f"{threads} threads" + (f", {one['value']:.4f} TOPS on 1 thread" if one else ""))

    import torch
    yg = Y[torch.from_numpy(rows).to(Y.device)].cpu()
    if w.out == "bf16":
        yg = yg.view(torch.int16).numpy().view(np.uint16)
        a = (yg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        r = (y_ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        yg = yg.numpy()
        a, r = yg.astype(np.float64), y_ref.astype(np.float64)
    err = float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-30))
    mism = int(np.count_nonzero(yg != y_ref))
    what = {"linear": "", "lowrank": ", both factors and the requantised h",
            "mlp": ", GELU", "swiglu": ", SwiGLU"}[w.kind]
    base = {
        "value": round(cpu_tops, 5),
        "unit": "TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{'all' if full else len(rows)} of {M} rows"
                   f"{'' if full else ' (seeded)'}, every projection over its full width and "
                   f"depth: rotate+quantise of those rows, INT32 contraction and epilogue{what}"),
        "seconds": round(dt, 2),
        "stages": {
            "prepare_weights": {"seconds": round(prep_s, 2), "rows": "every weight row"},
            "rotate_quantize": {"seconds": round(rq_s, 2), "rows": M,
                                "value": round(rq_gbs, 3), "unit": "GB/s"},
            "forward": {"seconds": round(dt, 2), "rows": int(len(rows)),
                        "value": round(cpu_tops, 5), "unit": "TOPS"},
        },
    }
    if one:
        base["single_thread"] = one
    parity = {"rows": int(len(rows)), "normwise_err": err, "mismatches": mism,
              "tolerance": 1e-3 if w.out == "bf16" else 1e-5}
    return base, parity


if __name__ == "__main__":
    main()
