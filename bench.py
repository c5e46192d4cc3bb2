#!/usr/bin/env python3
"""Benchmark of the W4A16 hot path on one MI355X.

Headline (`value`): decode GEMV throughput in HBM GB/s on a Llama-2-7B-shaped
stack at m=1: 32 layers x 7 linears (q,k,v,o 4096x4096; gate,up 11008x4096;
down 4096x11008), INT4 g=128 asymmetric, seeded synthetic weights
N(0, 0.02) with 0.1 % outlier columns x50.  One step is one decode token
through all 224 linears (3.45 GB of packed weights, far more than the 256 MB
Infinity Cache), replayed from a captured HIP graph with every input already
resident in HBM.  GB/s counts algorithmic bytes: packed codes (0.5 B/weight),
fp16 scales and zero-points (4/g B/weight), x and y once per linear.

Also measured in the same run and reported as extra keys:
  prefill  -- q4_gemm at m=2048 on the three 7B projection shapes (TFLOP/s),
  decode70b -- q4_gemv at m=8 over 80 layers of 70B-shaped linears (GB/s),
  stress   -- 8192x28672 Student-t weights with constant and zero groups,
              g=128 and g=32, asymmetric and symmetric: quantize+pack,
              dequant and the m=1 GEMV (GB/s),
  single_gemv_4096x4096 -- one 4096x4096 linear at m=1 over 64 packed copies,
  w8a16    -- INT8 decode (8 fused 7B layers, per-channel) and prefill (g=128),
  kv_codec -- the KV-cache codec on one 70B-shaped layer cache (GB/s) and the
              decode-time flush of 256 window blocks into a block pool,
  w8a8_smoothquant -- the int8 product at m=2048 on the 7B shapes (TOP/s) and
              the whole smoothed layer (activation quantization + product),
  gptq_awq -- GPTQ and AWQ on one 4096x4096 linear: time per layer and the
              output error relative to plain rounding,
  cpu_baseline -- the CPU oracle timed on this host's cores on bounded samples
              of each workload (its figure for a workload also sits next to
              the GPU figure, as `oracle_*` keys).

The inputs of every timed linear-layer call are built by the functions in the
"workloads" section below; `timed_linear_calls()` lists those calls, and the
parity tests run the oracle on exactly these inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
       python bench.py --trace-summary CSV [--last N]   (rocprofv3 kernel trace)
"""
import argparse
import collections
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix peak
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n_out, n_in, m, g, bits=4):
    """Bytes the method must move for one linear: codes, s and z, x and y."""
    return n_out * n_in * bits // 8 + 4 * n_out * (n_in // g) + 2 * m * n_in + 2 * m * n_out


def quantize_bytes(n_out, n_in, g, bits=4):
    """Bytes a quantize+pack (or dequant) pass moves: fp32 weights one way,
    packed codes and fp16 scale and zero-point the other."""
    return n_out * n_in * 4 + n_out * n_in * bits // 8 + 4 * n_out * (n_in // g)


# ---------------------------------------------------------------------------
# Workloads: the inputs of every timed linear-layer call.
# ---------------------------------------------------------------------------
Call = collections.namedtuple("Call", "leg index kind bits m n_out n_in group_size symmetric")

STRESS_SHAPE = (8192, 28672)
SINGLE_COPIES = 64


def decode7b_weight(layer, j, dev):
    """fp32 weights of fused linear j (qkv, o, gate_up, down) of 7B layer `layer`."""
    import torch
    from w4a16_dequant_gemv_amd import synthetic as syn
    lin = syn.LLAMA7B_LINEARS
    _, idx = syn.FUSED_LAYOUT[j]
    return torch.cat([syn.normal_weight_device(lin[i].n_out, lin[i].n_in, syn.llama7b_seed(layer, i), 0.02,
                                               syn.n_outliers(lin[i].n_in), dev) for i in idx])


def decode7b_x(j, dev, int8=False):
    from w4a16_dequant_gemv_amd import synthetic as syn
    n_in = syn.fused_linears(syn.LLAMA7B_LINEARS)[j].n_in
    return syn.activations_f16_device(1, n_in, (2200 if int8 else 2100) + j, dev)


def split_of(i):
    """Linear i of a 7B layer -> (fused index, first row within it)."""
    from w4a16_dequant_gemv_amd import synthetic as syn
    for j, (_, idx) in enumerate(syn.FUSED_LAYOUT):
        if i in idx:
            return j, sum(syn.LLAMA7B_LINEARS[t].n_out for t in idx[:idx.index(i)])
    raise ValueError(i)


def decode70b_weight(layer, j, dev):
    import torch
    from w4a16_dequant_gemv_amd import synthetic as syn
    lin = syn.LLAMA70B_LINEARS
    _, idx = syn.FUSED_LAYOUT[j]
    return torch.cat([syn.normal_weight_device(lin[i].n_out, lin[i].n_in, syn.llama70b_seed(layer, i), 0.015, 0, dev)
                      for i in idx])


def decode70b_x(j, dev):
    from w4a16_dequant_gemv_amd import synthetic as syn
    return syn.activations_f16_device(8, syn.fused_linears(syn.LLAMA70B_LINEARS)[j].n_in, 3100 + j, dev)


def stress_weight(g, dev):
    """8192x28672 = 0.02 * Student-t(3), 1 % constant and 0.1 % zero groups of g."""
    from w4a16_dequant_gemv_amd import synthetic as syn
    return syn.student_t_weight_device(*STRESS_SHAPE, 5, g, dev)


def stress_x(dev):
    from w4a16_dequant_gemv_amd import synthetic as syn
    return syn.activations_f16_device(1, STRESS_SHAPE[1], 5100, dev)


def single_weight(dev):
    from w4a16_dequant_gemv_amd import synthetic as syn
    return syn.normal_weight_device(4096, 4096, 1, 0.02, 8, dev)


def single_copy(w, c):
    """Copy c of the 4096x4096 weights cycled by the single-linear leg."""
    return w.mul(1.0 + c * 1e-3) if c else w


def single_x(dev):
    from w4a16_dequant_gemv_amd import synthetic as syn
    return syn.activations_f16_device(1, 4096, 101, dev)


def prefill_weight(i, dev):
    from w4a16_dequant_gemv_amd import synthetic as syn
    pl = syn.PREFILL_LINEARS[i]
    return syn.normal_weight_device(pl.n_out, pl.n_in, 4000 + i, 0.02, syn.n_outliers(pl.n_in), dev)


def prefill_x(i, dev):
    from w4a16_dequant_gemv_amd import synthetic as syn
    return syn.activations_f16_device(syn.PREFILL_M, syn.PREFILL_LINEARS[i].n_in, 4100 + i, dev)


def timed_linear_calls():
    """Every linear-layer call the benchmark times, with the workload that
    builds its inputs (leg, index).  The benchmark checks at run time that it
    makes no other call."""
    from w4a16_dequant_gemv_amd import synthetic as syn
    out = []
    for j, lin in enumerate(syn.fused_linears(syn.LLAMA7B_LINEARS)):
        out.append(Call("decode7b", j, "gemv", 4, 1, lin.n_out, lin.n_in, 128, False))
        out.append(Call("w8a16_decode", j, "gemv", 8, 1, lin.n_out, lin.n_in, lin.n_in, False))
    for i, lin in enumerate(syn.LLAMA7B_LINEARS):
        out.append(Call("decode7b_split", i, "gemv", 4, 1, lin.n_out, lin.n_in, 128, False))
    for j, lin in enumerate(syn.fused_linears(syn.LLAMA70B_LINEARS)):
        out.append(Call("decode70b", j, "gemv", 4, 8, lin.n_out, lin.n_in, 128, False))
    for g in (128, 32):
        for sym in (False, True):
            out.append(Call("stress", 0, "gemv", 4, 1, *STRESS_SHAPE, g, sym))
    out.append(Call("single", 0, "gemv", 4, 1, 4096, 4096, 128, False))
    for i, pl in enumerate(syn.PREFILL_LINEARS):
        out.append(Call("prefill", i, "gemm", 4, syn.PREFILL_M, pl.n_out, pl.n_in, 128, False))
        out.append(Call("w8a16_prefill", i, "gemm", 8, syn.PREFILL_M, pl.n_out, pl.n_in, 128, False))
    return out


# Calls made while capturing the timed graphs: (kind, bits, m, n_out, n_in, group_size).
_MADE = set()


def gemv(x, qw, y):
    import w4a16_dequant_gemv_amd as w4
    _MADE.add(("gemv", qw.bits, x.shape[0], qw.n_out, qw.n_in, qw.group_size))
    return w4.gemv(x, qw, y)


def gemm(x, qw, y):
    import w4a16_dequant_gemv_amd as w4
    _MADE.add(("gemm", qw.bits, x.shape[0], qw.n_out, qw.n_in, qw.group_size))
    return w4.gemm(x, qw, y)


def check_calls():
    known = {(c.kind, c.bits, c.m, c.n_out, c.n_in, c.group_size) for c in timed_linear_calls()}
    extra = _MADE - known
    if extra:
        raise RuntimeError(f"timed calls missing from timed_linear_calls(): {sorted(extra)}")


# ---------------------------------------------------------------------------
# Timing helpers.
# ---------------------------------------------------------------------------
def time_graph(graph, steps, warmup):
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) * 1e-3, wall


def replay_percentiles(graph, replays, scale=1.0):
    """p10 / p50 / p90 of single graph replays, each bracketed by its own pair
    of HIP events (a separate pass after the headline timing, which stays one
    bracket over all its steps); `scale` converts a replay's seconds into the
    reported unit."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(replays):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e-3 * scale for i in range(replays))

    def q(f):
        return round(t[min(len(t) - 1, int(f * len(t)))], 4)
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "replays": replays}


def settle(graph, seconds=0.25):
    """Untimed replays for at least `seconds`: under MFMA load the clock settles
    at its loaded value only after some 0.1 s, and the first replays after a
    lighter phase run up to 20 % slower."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        graph.replay()
        torch.cuda.synchronize()


def time_graph_eager(fn, steps, warmup):
    """HIP-event time of `steps` eager calls of fn (large kernels: launch cost
    is negligible next to them)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3, time.perf_counter() - t0


def capture(fn):
    """Capture fn() (a sequence of library launches) into a CUDA/HIP graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def gemv_sources_digest():
    h = hashlib.sha256()
    for f in ("q4_gemv.hip", "q4_device.h"):
        with open(os.path.join(ROOT, "w4a16_dequant_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counters_traffic(bytes_per_launch):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current GEMV source; otherwise None."""
    path = os.path.join(PROFILES, "gemv_llama7b_m1_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not t or m.group(1) != gemv_sources_digest():
        return None
    return float(t.group(1))


# ---------------------------------------------------------------------------
# GPU legs.
# ---------------------------------------------------------------------------
def bench_decode(args, dev, host):
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    from w4a16_dequant_gemv_amd.api import QuantizedWeight
    layers = syn.LLAMA7B_LAYERS
    t0 = time.perf_counter()
    fused = syn.fused_linears(syn.LLAMA7B_LINEARS)
    xs = [decode7b_x(j, dev) for j in range(len(fused))]
    gemvs = []
    for layer in range(layers):
        for j, lin in enumerate(fused):
            w = decode7b_weight(layer, j, dev)
            qw = w4.quantize_pack(w, 128)
            if layer == 0 and host is not None:
                host.setdefault("decode7b", []).append((lin.name, w.cpu().numpy(), xs[j].cpu().numpy()))
            del w
            gemvs.append((lin.name, qw, xs[j], torch.empty((1, qw.n_out), dtype=torch.float16, device=dev)))
    torch.cuda.synchronize()
    log(f"decode stack: {layers} layers x 7 linears quantized in {time.perf_counter() - t0:.1f} s")

    def step():
        for _, qw, x, y in gemvs:
            gemv(x, qw, y)

    graph = capture(step)
    step_bytes = sum(algorithmic_bytes(qw.n_out, qw.n_in, 1, 128) for _, qw, _, _ in gemvs)
    elapsed, wall = time_graph(graph, args.steps, args.warmup)
    launches = len(gemvs)
    per_launch_s = elapsed / (args.steps * launches)
    res = dict(step_bytes=step_bytes, launches=launches, elapsed=elapsed, wall=wall,
               ms_per_step=elapsed / args.steps * 1e3,
               gbs=step_bytes * args.steps / elapsed / 1e9,
               per_launch_us=per_launch_s * 1e6,
               bytes_per_launch=step_bytes / launches,
               ms_per_step_percentiles=None if args.decode_only else
               replay_percentiles(graph, max(10, args.steps), 1e3))
    # The same weights with one launch per linear (7 per layer): row slices
    # of the fused matrices are themselves valid packed weights.
    res["gbs_7_launches_per_layer"] = None
    if not args.decode_only:
        per_linear = []
        for layer in range(layers):
            for i, lin in enumerate(syn.LLAMA7B_LINEARS):
                j, off = split_of(i)
                _, qw, x, y = gemvs[layer * len(fused) + j]
                sl = slice(off, off + lin.n_out)
                per_linear.append((QuantizedWeight(qw.qweight[sl], qw.scales[sl], qw.zeros[sl], lin.n_out, qw.n_in,
                                                   128), x, y[:, sl]))
        graph7 = capture(lambda: [gemv(x, q, y) for q, x, y in per_linear])
        el7, _ = time_graph(graph7, max(1, args.steps // 2), 1)
        res["gbs_7_launches_per_layer"] = round(step_bytes * max(1, args.steps // 2) / el7 / 1e9, 1)
        del graph7
    return res


def bench_prefill(args, dev, bits=4):
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    out, tot_flop, tot_t = [], 0, 0.0
    for i, lin in enumerate(syn.PREFILL_LINEARS):
        w = prefill_weight(i, dev)
        qw = w4.quantize_pack(w, 128, bits=bits)
        del w
        x = prefill_x(i, dev)
        y = torch.empty((syn.PREFILL_M, lin.n_out), dtype=torch.float16, device=dev)
        reps = 20
        g = capture(lambda: [gemm(x, qw, y) for _ in range(reps)])
        settle(g)
        el, _ = time_graph(g, 5, 3)
        t = el / (5 * reps)
        flop = 2 * syn.PREFILL_M * lin.n_out * lin.n_in
        out.append(dict(shape=f"{syn.PREFILL_M}x{lin.n_out}x{lin.n_in}", us=round(t * 1e6, 2),
                        tflops=round(flop / t / 1e12, 1),
                        us_percentiles=replay_percentiles(g, 10, 1e6 / reps)))
        tot_flop += flop
        tot_t += t
        del qw, x, y, g
    torch.cuda.empty_cache()
    return dict(shapes=out, tflops=round(tot_flop / tot_t / 1e12, 1))


def bench_decode70b(args, dev):
    """80 layers of 70B-shaped linears at m=8, stored fused like the 7B stack:
    qkv [10240, 8192], o [8192, 8192], gate_up [57344, 8192], down [8192, 28672]."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    layers = syn.LLAMA70B_LAYERS if not args.quick else 8
    fused = syn.fused_linears(syn.LLAMA70B_LINEARS)
    xs = [decode70b_x(j, dev) for j in range(len(fused))]
    gemvs = []
    t0 = time.perf_counter()
    for layer in range(layers):
        for j in range(len(fused)):
            w = decode70b_weight(layer, j, dev)
            qw = w4.quantize_pack(w, 128)
            del w
            gemvs.append((qw, xs[j], torch.empty((8, qw.n_out), dtype=torch.float16, device=dev)))
    torch.cuda.synchronize()
    log(f"70B stack: {layers} layers quantized in {time.perf_counter() - t0:.1f} s")
    g = capture(lambda: [gemv(x, qw, y) for qw, x, y in gemvs])
    el, _ = time_graph(g, 5, 3)
    nbytes = sum(algorithmic_bytes(qw.n_out, qw.n_in, 8, 128) for qw, _, _ in gemvs)
    res = dict(layers=layers, m=8, gemvs_per_pass=len(gemvs), ms_per_pass=round(el / 5 * 1e3, 3),
               gbs=round(nbytes * 5 / el / 1e9, 1), resident_gb=round(nbytes / 1e9, 2),
               ms_per_pass_percentiles=None if args.decode70b_only else replay_percentiles(g, 5, 1e3))
    del gemvs, g
    torch.cuda.empty_cache()
    return res


def bench_single(args, dev):
    """One 4096x4096 linear at m=1 (g=128), cycled over 64 distinct packed copies
    (about 570 MB, beyond the 256 MB Infinity Cache) inside one graph: the
    latency-dominated single-GEMV case."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    n_out = n_in = 4096
    w = single_weight(dev)
    qws = [w4.quantize_pack(single_copy(w, c), 128) for c in range(SINGLE_COPIES)]
    del w
    x = single_x(dev)
    y = torch.empty((1, n_out), dtype=torch.float16, device=dev)
    gr = capture(lambda: [gemv(x, q, y) for q in qws])
    el, _ = time_graph(gr, 3, 1)
    t = el / (3 * len(qws))
    del qws, gr
    torch.cuda.empty_cache()
    return dict(us_per_launch=round(t * 1e6, 2),
                gbs=round(algorithmic_bytes(n_out, n_in, 1, 128) / t / 1e9, 1))


def bench_int8(args, dev):
    """W8A16: decode at m=1 over 8 layers of the fused 7B linears with INT8
    per-channel weights (1.7 GB, beyond the Infinity Cache), and prefill at
    m=2048 on the 7B projection shapes with INT8 g=128 weights."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    fused = syn.fused_linears(syn.LLAMA7B_LINEARS)
    xs = [decode7b_x(j, dev, int8=True) for j in range(len(fused))]
    layers, gemvs = 8, []
    for layer in range(layers):
        for j in range(len(fused)):
            w = decode7b_weight(layer, j, dev)
            qw = w4.quantize_pack(w, None, bits=8)
            del w
            gemvs.append((qw, xs[j], torch.empty((1, qw.n_out), dtype=torch.float16, device=dev)))
    g = capture(lambda: [gemv(x, qw, y) for qw, x, y in gemvs])
    el, _ = time_graph(g, 10, 2)
    nbytes = sum(algorithmic_bytes(qw.n_out, qw.n_in, 1, qw.n_in, 8) for qw, _, _ in gemvs)
    res = dict(decode_layers=layers, decode_m=1, decode_group="per-channel",
               decode_gbs=round(nbytes * 10 / el / 1e9, 1),
               decode_us_per_launch=round(el / (10 * len(gemvs)) * 1e6, 2))
    del gemvs, g
    pre = bench_prefill(args, dev, bits=8)
    res["prefill_g128_shapes"] = [dict(shape=s["shape"], tflops=s["tflops"]) for s in pre["shapes"]]
    res["prefill_g128_tflops"] = pre["tflops"]
    return res


def bench_stress_and_quantize(args, dev, host):
    """Quantizer stress: 8192x28672 Student-t(3) weights with constant and zero
    groups, for g=128 and g=32 in both modes: quantize+pack and dequant GB/s,
    then the m=1 GEMV over three packed copies (3 x 125-147 MB, beyond the
    Infinity Cache)."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    n_out, n_in = STRESS_SHAPE
    x = stress_x(dev)
    res = {}
    for g in (128, 32):
        w = stress_weight(g, dev)
        if host is not None:
            host.setdefault("stress", {})[g] = w[:512].cpu().numpy()
        for sym in (False, True):
            mode = "sym" if sym else "asym"
            qws = [w4.quantize_pack(w, g, sym)]
            for c in range(1, 3):
                qws.append(w4.quantize_pack(w.mul(1.0 + c * 1e-3), g, sym))
            y = torch.empty((1, n_out), dtype=torch.float16, device=dev)
            reps = 8
            gr = capture(lambda: [gemv(x, qws[r % 3], y) for r in range(reps * 3)])
            el, _ = time_graph(gr, 3, 1)
            t = el / (3 * reps * 3)
            res[f"gemv_g{g}_{mode}_gbs"] = round(algorithmic_bytes(n_out, n_in, 1, g) / t / 1e9, 1)
            res[f"gemv_g{g}_{mode}_us"] = round(t * 1e6, 2)
            del gr
            qw = qws[0]
            gq = capture(lambda: [w4.quantize_pack(w, g, sym, out=qw) for _ in range(5)])
            el, _ = time_graph(gq, 2, 1)
            res[f"quantize_g{g}_{mode}_gbs"] = round(quantize_bytes(n_out, n_in, g) * 10 / el / 1e9, 1)
            del gq, qws
        out = torch.empty_like(w)
        gd = capture(lambda: [w4.dequant(qw, out) for _ in range(5)])
        el, _ = time_graph(gd, 2, 1)
        res[f"dequant_g{g}_gbs"] = round(quantize_bytes(n_out, n_in, g) * 10 / el / 1e9, 1)
        del w, out, gd, qw
        torch.cuda.empty_cache()
    # the keys of the earlier single-mode report
    res["gemv_g128_gbs"], res["gemv_g32_gbs"] = res["gemv_g128_asym_gbs"], res["gemv_g32_asym_gbs"]
    return res


def bench_kv(args, dev):
    """KV-cache codec on one layer of a Llama-3-70B-shaped cache (batch 32, 8
    KV heads, 32768 tokens, head dim 128: 2.1 GB of fp16 per side): K
    quantized per channel over 128-token blocks and V per token (one pass
    over both), the matching dequantization, and the decode-time flush of one
    128-token window block per sequence and head (256 blocks) into a pool."""
    import torch
    from w4a16_dequant_gemv_amd import kv, synthetic as syn
    c = syn.KV70B
    T, D = c["block"], c["head_dim"]
    blocks = c["batch"] * c["kv_heads"] * c["seq"] // T
    k = syn.kv_values_device((blocks, T, D), 6200, dev)
    v = syn.kv_values_device((blocks, T, D), 6201, dev, n_outlier_channels=0)
    qk, sk = kv.quant_channels(k)
    qv, sv = kv.quant_tokens(v)

    def quant():
        kv.quant_channels(k, q=qk, scale=sk)
        kv.quant_tokens(v, q=qv, scale=sv)

    elems = blocks * T * D
    q_bytes = 2 * (elems * 2 + elems) + sk.numel() * 4 + sv.numel() * 4
    quant()
    el, _ = time_graph_eager(quant, 5, 2)
    res = dict(cache=f"{c['batch']}x{c['kv_heads']}x{c['seq']}x{D} per side, blocks of {T}",
               quant_gbs=round(q_bytes * 5 / el / 1e9, 1), quant_ms=round(el / 5 * 1e3, 3))
    ok, ov = torch.empty_like(k), torch.empty_like(v)

    def deq():
        kv.dequant_channels(qk, sk, out=ok)
        kv.dequant_tokens(qv, sv, out=ov)

    deq()
    el, _ = time_graph_eager(deq, 5, 2)
    res["dequant_gbs"] = round(q_bytes * 5 / el / 1e9, 1)
    res["dequant_ms"] = round(el / 5 * 1e3, 3)
    res["quant_frac"] = round(res["quant_gbs"] / HBM_PEAK_GBS, 4)
    del ok, ov, qk, qv
    # decode-time flush: every (sequence, head) hands one full block to the pool
    P = c["batch"] * c["kv_heads"]
    pool = kv.KVBlockPool(4 * P, T, D, dev)
    kb, vb = k[:P].contiguous(), v[:P].contiguous()
    dst = torch.randperm(4 * P, device=dev)[:P].to(torch.int32)
    g = capture(lambda: [pool.flush(kb, vb, dst) for _ in range(20)])
    el, _ = time_graph(g, 5, 2)
    t_flush = el / (5 * 20)
    f_bytes = 2 * P * T * D * 2 + 2 * P * T * D + P * (D + T) * 4 + P * 4
    res["flush_blocks"] = P
    res["flush_us"] = round(t_flush * 1e6, 2)
    res["flush_gbs"] = round(f_bytes / t_flush / 1e9, 1)
    del k, v, kb, vb, pool
    torch.cuda.empty_cache()
    return res


def bench_w8a8(args, dev):
    """W8A8 with SmoothQuant at prefill (m = 2048) on the 7B projection shapes:
    the int8 product alone (TOP/s against the 5.0 POP/s dense int8 peak) and
    the whole layer per call (per-token activation quantization of x / s, then
    the product)."""
    import torch
    from w4a16_dequant_gemv_amd import synthetic as syn, w8a8
    out, tot_op, tot_t, tot_layer_t = [], 0, 0.0, 0.0
    for i, lin in enumerate(syn.PREFILL_LINEARS):
        w = prefill_weight(i, dev)
        calib = syn.activations_f16_device(512, lin.n_in, 4200 + i, dev)
        act_max = torch.zeros(lin.n_in, dtype=torch.float32, device=dev)
        w8a8.absmax_update(calib, act_max)
        layer = w8a8.W8A8Linear.from_float(w, act_max)
        del w, calib
        x = prefill_x(i, dev)
        qx, sx = w8a8.quantize_act(x, layer.s)
        y = torch.empty((syn.PREFILL_M, lin.n_out), dtype=torch.float16, device=dev)
        reps = 20
        g = capture(lambda: [w8a8.gemm(qx, sx, layer.qw, layer.sw, y) for _ in range(reps)])
        settle(g)
        el, _ = time_graph(g, 5, 3)
        t = el / (5 * reps)
        gl = capture(lambda: [(w8a8.quantize_act(x, layer.s, qx, sx), w8a8.gemm(qx, sx, layer.qw, layer.sw, y))
                              for _ in range(reps)])
        el, _ = time_graph(gl, 5, 3)
        tl = el / (5 * reps)
        op = 2 * syn.PREFILL_M * lin.n_out * lin.n_in
        out.append(dict(shape=f"{syn.PREFILL_M}x{lin.n_out}x{lin.n_in}", gemm_us=round(t * 1e6, 2),
                        tops=round(op / t / 1e12, 1), layer_us=round(tl * 1e6, 2)))
        tot_op += op
        tot_t += t
        tot_layer_t += tl
        del layer, x, qx, y, g, gl
    torch.cuda.empty_cache()
    tops = round(tot_op / tot_t / 1e12, 1)
    return dict(shapes=out, tops=tops, frac_int8_peak=round(tops / INT8_PEAK_TOPS, 4),
                layer_tops=round(tot_op / tot_layer_t / 1e12, 1))


def bench_producers(args, dev):
    """GPTQ (512 calibration tokens) and AWQ (128 tokens, 21-point grid) on one
    4096x4096 linear, INT4 g=128: wall time per layer on the GPU and each
    method's output error on its calibration tokens relative to plain
    rounding (the quantity both methods minimize)."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import producers, synthetic as syn
    n = 4096
    w = syn.normal_weight_device(n, n, 4300, 0.02, syn.n_outliers(n), dev)
    x = syn.activations_f16_device(512, n, 4301, dev)
    x[:, :8] *= 8                      # a few outlier activation channels
    res = {}

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        return out, time.perf_counter() - t0

    producers.gptq(w[:256], x[:64], 128)           # warm the launch paths
    u, t_fac = timed(lambda: producers.gptq_factor(x))
    g, t_loop = timed(lambda: producers.gptq_quantize(w, u, 128))
    xa = x[:128].contiguous()
    (qa, s_awq, best, losses), t_awq = timed(lambda: producers.awq(w, xa, 128))
    r = w4.quantize_pack(w, 128)

    def out_err(xx, wd):
        return ((xx.double() @ (w.double() - wd.double()).t()) ** 2).sum().item()

    e_r = out_err(x, w4.dequant(r))
    res["gptq"] = dict(tokens=512, factor_ms=round(t_fac * 1e3, 1), loop_ms=round(t_loop * 1e3, 1),
                       err_vs_rounding=round(out_err(x, w4.dequant(g)) / e_r, 4))
    e_ra = out_err(xa, w4.dequant(r))
    eff = w4.dequant(qa) / s_awq[None, :]
    res["awq"] = dict(tokens=128, grid=20, ms=round(t_awq * 1e3, 1), alpha=round(int(best.item()) / 20, 2),
                      err_vs_rounding=round(out_err(xa, eff) / e_ra, 4))
    del w, x, u, g, r, qa
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on bounded samples of each workload.
# ---------------------------------------------------------------------------
def cpu_baseline(args, dev, host):
    """Times the CPU oracle (dequantize, then the binary64 product; the
    quantizer for quantize+pack) on this host's cores.  Every figure is on the
    same algorithmic bytes (GB/s) or flops (GFLOP/s) as the GPU figure it is
    reported beside.  Each leg repeats its sample until `budget` seconds of
    CPU time have passed (at least once)."""
    import numpy as np
    import oracle
    from w4a16_dequant_gemv_amd import synthetic as syn
    orc = oracle.load()
    budget = args.cpu_seconds / 16.0
    cores = orc.max_threads()

    def rate(fn, units, share=1.0):
        t, n = 0.0, 0
        while t < budget * share or n == 0:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            n += 1
        return units * n / t, n, t

    legs = {}
    # config 2: layer 0 of the 7B decode step (fused linears, m = 1)
    prepared = []
    for name, w, x in host["decode7b"]:
        packed, scales, zeros, _ = orc.quantize_pack(w, 128)
        prepared.append((packed, scales, zeros, x.view(np.uint16), w.shape))
    step = sum(algorithmic_bytes(s[0], s[1], 1, 128) for *_, s in prepared)
    gbs, n, t = rate(lambda: [orc.linear_from_packed(x, p, s, z, 128) for p, s, z, x, _ in prepared], step / 1e9,
                     share=4.0)
    legs["decode7b_gemv"] = dict(gbs=round(gbs, 3), sample=f"layer 0's four fused GEMVs (m=1) x{n}, {t:.1f} s")
    # config 1: one 4096x4096 linear, quantize+pack and GEMV, all threads and one
    w1 = host["single"]
    gbs, n, t = rate(lambda: orc.quantize_pack(w1, 128), quantize_bytes(4096, 4096, 128) / 1e9)
    legs["single_quantize"] = dict(gbs=round(gbs, 3), sample=f"4096x4096 g=128 x{n}, {t:.1f} s")
    p1, s1, z1, _ = orc.quantize_pack(w1, 128)
    x1 = host["single_x"].view(np.uint16)
    b1 = algorithmic_bytes(4096, 4096, 1, 128) / 1e9
    gbs, n, t = rate(lambda: orc.linear_from_packed(x1, p1, s1, z1, 128), b1)
    legs["single_gemv"] = dict(gbs=round(gbs, 3), sample=f"4096x4096 m=1 x{n}, {t:.1f} s")
    orc.set_threads(1)
    try:
        gbs, n, t = rate(lambda: orc.linear_from_packed(x1, p1, s1, z1, 128), b1)
    finally:
        orc.set_threads(cores)
    legs["single_gemv_1thread"] = dict(gbs=round(gbs, 3), threads=1, sample=f"4096x4096 m=1 x{n}, {t:.1f} s")
    # config 5: the first 512 rows of the 8192x28672 stress matrix per group size
    if "stress" in host:
        xs = host["stress_x"].view(np.uint16)
        for g, wb in sorted(host["stress"].items()):
            for sym in (False, True):
                mode = "sym" if sym else "asym"
                gbs, n, t = rate(lambda: orc.quantize_pack(wb, g, sym), quantize_bytes(wb.shape[0], wb.shape[1], g) / 1e9)
                legs[f"stress_quantize_g{g}_{mode}"] = dict(gbs=round(gbs, 3),
                                                            sample=f"rows 0-511 of 8192x28672 x{n}, {t:.1f} s")
            pb, sb, zb, _ = orc.quantize_pack(wb, g)
            gbs, n, t = rate(lambda: orc.linear_from_packed(xs, pb, sb, zb, g),
                             algorithmic_bytes(wb.shape[0], wb.shape[1], 1, g) / 1e9)
            legs[f"stress_gemv_g{g}"] = dict(gbs=round(gbs, 3), sample=f"rows 0-511 of 8192x28672, m=1, x{n}, {t:.1f} s")
    # config 3: 256 sampled rows of each fused linear of layers 0, 40 and 79 at
    # m = 8, extrapolated to the 80-layer pass by its algorithmic bytes
    if "decode70b" in host:
        items = []
        for layer, j, wr, x in host["decode70b"]:
            p, s, z, _ = orc.quantize_pack(wr, 128)
            items.append((p, s, z, x.view(np.uint16), wr.shape))
        sample_bytes = sum(algorithmic_bytes(sh[0], sh[1], 8, 128) for *_, sh in items)
        gbs, n, t = rate(lambda: [orc.linear_from_packed(x, p, s, z, 128) for p, s, z, x, _ in items],
                         sample_bytes / 1e9)
        pass_bytes = syn.LLAMA70B_LAYERS * sum(algorithmic_bytes(l.n_out, l.n_in, 8, 128)
                                              for l in syn.fused_linears(syn.LLAMA70B_LINEARS))
        legs["decode70b_gemv_extrapolated"] = dict(
            gbs=round(gbs, 3), ms_per_pass_extrapolated=round(pass_bytes / (gbs * 1e9) * 1e3, 1),
            sample=f"256 rows of each fused linear of layers 0, 40, 79 (m=8) x{n}, {t:.1f} s; "
                   f"extrapolated to 80 layers")
    # config 4: 16 rows of x through each prefill shape
    if "prefill" in host:
        flop, tt, nn = 0, 0.0, 0
        for w, x in host["prefill"]:
            p, s, z, _ = orc.quantize_pack(w, 128)
            xr = x.view(np.uint16)
            f = 2 * xr.shape[0] * w.shape[0] * w.shape[1]
            r, n, t = rate(lambda: orc.linear_from_packed(xr, p, s, z, 128), f / 1e9)
            flop += f * n
            tt += t
            nn += n
        legs["prefill_gemm"] = dict(gflops=round(flop / tt / 1e9, 3),
                                    sample=f"16 rows of x (m=2048 workload) through the three 7B shapes, "
                                           f"{nn} products, {tt:.1f} s")
    return dict(value=legs["decode7b_gemv"]["gbs"], unit="GB/s", cores=cores, kind="oracle",
                sample=(f"headline leg: {legs['decode7b_gemv']['sample']} (qkv 12288x4096, o 4096x4096, "
                        f"gate_up 22016x4096, down 4096x11008; g=128) through the C oracle's dequantize + "
                        f"binary64 product; the other legs are listed under `legs`"),
                legs=legs)


def host_samples(dev, full):
    """Host copies of the CPU-baseline samples the GPU legs do not keep (all
    of them with `full`, else only the single linear's)."""
    import numpy as np
    import torch
    from w4a16_dequant_gemv_amd import synthetic as syn
    host = {"single": single_weight(dev).cpu().numpy(), "single_x": single_x(dev).cpu().numpy()}
    if not full:
        return host
    host["stress_x"] = stress_x(dev).cpu().numpy()
    rng = np.random.default_rng(3300)
    host["decode70b"] = []
    for layer in (0, 40, 79):
        for j in range(4):
            wd = decode70b_weight(layer, j, dev)
            rows = np.sort(rng.choice(wd.shape[0], size=256, replace=False))
            host["decode70b"].append((layer, j, wd[torch.from_numpy(rows).to(dev)].cpu().numpy(),
                                      decode70b_x(j, dev).cpu().numpy()))
            del wd
    host["prefill"] = [(prefill_weight(i, dev).cpu().numpy(), prefill_x(i, dev)[:16].cpu().numpy())
                       for i in range(len(syn.PREFILL_LINEARS))]
    return host


# ---------------------------------------------------------------------------
# rocprofv3 kernel-trace summary.
# ---------------------------------------------------------------------------
def kernel_short_name(name):
    """'void (anonymous namespace)::k<1, 2>(int, ...)' -> 'k<1, 2>'."""
    name = re.sub(r"^void |\(anonymous namespace\)::", "", name)
    return re.sub(r"\(.*$", "", name)


def trace_summary(path, last, pattern):
    """Per-kernel statistics of the last `last` dispatches whose kernel name
    matches `pattern` in a rocprofv3 --kernel-trace CSV (the timed replays of a
    run come last)."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            if re.search(pattern, name):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), name))
    rows.sort()
    rows = rows[-last:] if last else rows
    by = collections.defaultdict(list)
    for s, e, name in rows:
        short = kernel_short_name(name)
        by[short].append((e - s) / 1e3)
    out = {"dispatches": len(rows), "total_us": round(sum(sum(v) for v in by.values()), 2), "kernels": {}}
    for k, v in sorted(by.items()):
        out["kernels"][k] = dict(calls=len(v), avg_us=round(sum(v) / len(v), 3), min_us=round(min(v), 3),
                                 max_us=round(max(v), 3), total_us=round(sum(v), 2))
    return out


def counter_summary(path, pattern):
    """Mean of each counter per (kernel, grid size) over the dispatches whose
    kernel name matches `pattern` in a rocprofv3 --pmc CSV."""
    import csv
    acc = collections.defaultdict(lambda: [0.0, 0])
    dur = collections.defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not re.search(pattern, name):
                continue
            short = kernel_short_name(name)
            key = (short, int(r["Grid_Size"]))
            a = acc[key + (r["Counter_Name"],)]
            a[0] += float(r["Counter_Value"])
            a[1] += 1
            dur[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for (short, grid, counter), (tot, n) in sorted(acc.items()):
        d = out.setdefault(f"{short} grid={grid}", {})
        d[counter] = round(tot / n, 1)
        d["dispatches"] = n
        d["avg_us"] = round(sum(dur[(short, grid)]) / len(dur[(short, grid)]) / 1e3, 2)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="decode phase plus a short 70B stack")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline decode phase")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the timed decode graph (no extras, no per-linear reference, no CPU leg); "
                         "used for profiling")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill GEMM phase, printed as its own JSON line; used for profiling")
    ap.add_argument("--decode70b-only", action="store_true",
                    help="only the 70B-shaped m=8 pass (timed replays, no percentile pass), printed as its own "
                         "JSON line; used for profiling")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one elementwise copy of 256 MiB (268435456 bytes read and written), "
                         "the known-size kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU time budget of the oracle baseline, shared by its legs")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarize a rocprofv3 kernel trace (no GPU work) and exit")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="mean of each counter per kernel and grid size in a rocprofv3 --pmc CSV, and exit")
    ap.add_argument("--last", type=int, default=0, help="with --trace-summary: only the last N dispatches")
    ap.add_argument("--kernel", default=r"gemv_|gemm_kernel",
                    help="with --trace-summary / --counter-summary: kernel name regex")
    args = ap.parse_args()

    if args.counter_summary:
        print(json.dumps(counter_summary(args.counter_summary, args.kernel), indent=1))
        return
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary, args.last, args.kernel), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (the library has no CPU path)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        log("copy calibration: torch.neg over 268435456 bytes (read) into 268435456 bytes (written)")
        del a, b
    if args.prefill_only:
        pre = bench_prefill(args, dev)
        check_calls()
        log(f"prefill: {pre}")
        print(json.dumps({
            "metric": "W4A16 prefill GEMM TFLOP/s (m=2048)", "value": pre["tflops"], "unit": "TFLOP/s",
            "n_gpus": 1, "higher_is_better": True, "dtype": "int4 weights x fp16 activations, fp32 accumulate",
            "data": "synthetic", "config": {"workload": "prefill m=2048 on the 7B linear shapes"},
            "prefill": pre, "roofline": {"bound": "mfma", "achieved": pre["tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(pre["tflops"] / MFMA_F16_PEAK_TFLOPS, 4)}}),
              flush=True)
        return
    if args.decode70b_only:
        res = bench_decode70b(args, dev)
        check_calls()
        log(f"decode70b: {res}")
        print(json.dumps({"metric": "W4A16 decode GEMV HBM GB/s, 70B-shaped pass at m=8", "value": res["gbs"],
                          "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": "Llama-2-70B-shaped decode, m=8: 80 layers x 4 fused GEMVs, "
                                                 "INT4 g=128"},
                          "decode70b": res}), flush=True)
        return
    if args.decode_only:
        args.no_extras = True
        args.no_cpu_baseline = True
    host = None if args.no_cpu_baseline else {}
    decode = bench_decode(args, dev, host)
    log(f"decode: {decode['gbs']:.1f} GB/s, {decode['ms_per_step']:.3f} ms/step, "
        f"{decode['per_launch_us']:.2f} us per GEMV launch")
    extras = {}
    if not args.no_extras:
        extras["prefill"] = bench_prefill(args, dev)
        log(f"prefill: {extras['prefill']}")
        extras["decode70b"] = bench_decode70b(args, dev)
        log(f"decode70b: {extras['decode70b']}")
        extras["stress"] = bench_stress_and_quantize(args, dev, host)
        log(f"stress: {extras['stress']}")
        extras["single"] = bench_single(args, dev)
        log(f"single 4096x4096 GEMV: {extras['single']}")
        extras["int8"] = bench_int8(args, dev)
        log(f"int8 (W8A16): {extras['int8']}")
        extras["kv"] = bench_kv(args, dev)
        log(f"kv codec: {extras['kv']}")
        extras["w8a8"] = bench_w8a8(args, dev)
        log(f"w8a8: {extras['w8a8']}")
        extras["producers"] = bench_producers(args, dev)
        log(f"gptq/awq: {extras['producers']}")
    check_calls()
    cpu = None
    if host is not None:
        host.update(host_samples(dev, full=not args.no_extras))
        cpu = cpu_baseline(args, dev, host)
        log(f"cpu baseline: {cpu}")

    achieved = decode["bytes_per_launch"] / (decode["per_launch_us"] * 1e-6) / 1e9
    traffic = counters_traffic(decode["bytes_per_launch"])
    legs = cpu["legs"] if cpu else {}
    record = {
        "metric": "W4A16 decode GEMV HBM GB/s (% peak) + prefill GEMM TFLOPS (% MFMA peak)",
        "value": round(decode["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(decode["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights with 0.1% outlier columns x50, x ~ N(0,1) fp16)",
        "config": {"workload": "Llama-2-7B-shaped decode, m=1: 32 layers x 7 linears "
                               "(q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008), INT4 g=128 asymmetric",
                   "m": 1, "group_size": 128, "layers": 32, "gemvs_per_step": decode["launches"],
                   "bytes_per_step": decode["step_bytes"],
                   "launch": "HIP graph replay; per layer 4 dependent GEMVs: fused qkv, o, fused gate_up, down"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "q4_gemv", "avg_launch_us": round(decode["per_launch_us"], 3),
                     "bytes_per_launch": round(decode["bytes_per_launch"])},
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(decode["wall"], 4),
        "ms_per_step_percentiles": decode["ms_per_step_percentiles"],
        "decode_7_launches_per_layer_gbs": decode["gbs_7_launches_per_layer"],
    }
    if "prefill" in extras:
        tf = extras["prefill"]["tflops"]
        record["prefill"] = dict(extras["prefill"], roofline={
            "bound": "mfma", "achieved": tf, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)})
        record["decode70b"] = dict(extras["decode70b"], frac=round(extras["decode70b"]["gbs"] / HBM_PEAK_GBS, 4))
        record["stress"] = extras["stress"]
        record["single_gemv_4096x4096"] = extras["single"]
        record["w8a16"] = extras["int8"]
        record["kv_codec"] = extras["kv"]
        record["w8a8_smoothquant"] = extras["w8a8"]
        record["gptq_awq"] = extras["producers"]
        # the oracle's figure beside each GPU figure
        if legs:
            record["prefill"]["oracle_gflops"] = legs["prefill_gemm"]["gflops"]
            record["decode70b"]["oracle_gbs_extrapolated"] = legs["decode70b_gemv_extrapolated"]["gbs"]
            record["decode70b"]["oracle_ms_per_pass_extrapolated"] = \
                legs["decode70b_gemv_extrapolated"]["ms_per_pass_extrapolated"]
            for g in (128, 32):
                record["stress"][f"oracle_gemv_g{g}_gbs"] = legs[f"stress_gemv_g{g}"]["gbs"]
                for mode in ("asym", "sym"):
                    record["stress"][f"oracle_quantize_g{g}_{mode}_gbs"] = legs[f"stress_quantize_g{g}_{mode}"]["gbs"]
            record["single_gemv_4096x4096"]["oracle_gbs"] = legs["single_gemv"]["gbs"]
            record["single_gemv_4096x4096"]["oracle_gbs_1thread"] = legs["single_gemv_1thread"]["gbs"]
            record["single_gemv_4096x4096"]["oracle_quantize_gbs"] = legs["single_quantize"]["gbs"]
    if legs:
        record["oracle_decode_gbs"] = legs["decode7b_gemv"]["gbs"]
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
