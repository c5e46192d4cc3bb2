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
  stress   -- q4_gemv at m=1 on 8192x28672 for g=128 and g=32 (GB/s),
  quantize -- q4_quantize_pack and q4_dequant on 8192x28672 (GB/s),
  single_gemv_4096x4096 -- one 4096x4096 linear at m=1 over 64 packed copies,
  w8a16    -- INT8 decode (8 fused 7B layers, per-channel) and prefill (g=128),
  kv_codec -- the KV-cache codec on one 70B-shaped layer cache (GB/s) and the
              decode-time flush of 256 window blocks into a block pool,
  w8a8_smoothquant -- the int8 product at m=2048 on the 7B shapes (TOP/s) and
              the whole smoothed layer (activation quantization + product),
  gptq_awq -- GPTQ and AWQ on one 4096x4096 linear: time per layer and the
              output error relative to plain rounding,
  cpu_baseline -- the CPU oracle (dequantize + binary64 product) timed on
                  this host's cores on a bounded sample of the decode step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
import argparse
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
def build_decode_stack(layers, dev, keep_host_layer0):
    """Quantized 7B-shaped layers stored the way serving engines store them:
    q, k, v concatenated into one [12288, 4096] matrix and gate, up into one
    [22016, 4096] matrix (quantization is per row, so this equals quantizing
    each linear alone).  Each of the four GEMVs of a layer has its own x."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    lin = syn.LLAMA7B_LINEARS
    fused = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
    xs = {name: syn.activations_f16_device(1, lin[idx[0]].n_in, 2100 + j, dev)
          for j, (name, idx) in enumerate(fused)}
    gemvs, host_w = [], []
    for layer in range(layers):
        for name, idx in fused:
            w = torch.cat([syn.normal_weight_device(lin[i].n_out, lin[i].n_in, syn.llama7b_seed(layer, i),
                                                    0.02, syn.n_outliers(lin[i].n_in), dev) for i in idx])
            qw = w4.quantize_pack(w, 128)
            if layer == 0 and keep_host_layer0:
                host_w.append((name, w.cpu().numpy(), xs[name].cpu().numpy()))
            del w
            y = torch.empty((1, qw.n_out), dtype=torch.float16, device=dev)
            gemvs.append((name, qw, xs[name], y))
    torch.cuda.synchronize()
    return gemvs, host_w


def bench_decode(args, dev):
    import w4a16_dequant_gemv_amd as w4
    layers = 32
    t0 = time.perf_counter()
    gemvs, host_w = build_decode_stack(layers, dev, keep_host_layer0=not args.no_cpu_baseline)
    log(f"decode stack: {layers} layers x 7 linears quantized in {time.perf_counter() - t0:.1f} s")

    def step():
        for _, qw, x, y in gemvs:
            w4.gemv(x, qw, y)

    graph = capture(step)
    step_bytes = sum(algorithmic_bytes(qw.n_out, qw.n_in, 1, 128) for _, qw, _, _ in gemvs)
    elapsed, wall = time_graph(graph, args.steps, args.warmup)
    launches = len(gemvs)
    per_launch_s = elapsed / (args.steps * launches)
    res = dict(step_bytes=step_bytes, launches=launches, elapsed=elapsed, wall=wall,
               ms_per_step=elapsed / args.steps * 1e3,
               gbs=step_bytes * args.steps / elapsed / 1e9,
               per_launch_us=per_launch_s * 1e6,
               bytes_per_launch=step_bytes / launches)
    # The same weights with one launch per linear (7 per layer): row slices
    # of the fused matrices are themselves valid packed weights.
    from w4a16_dequant_gemv_amd.api import QuantizedWeight
    split = {"qkv": (4096, 4096, 4096), "gate_up": (11008, 11008)}
    per_linear = []
    for name, qw, x, y in gemvs:
        off = 0
        for n in split.get(name, (qw.n_out,)):
            sl = slice(off, off + n)
            per_linear.append((QuantizedWeight(qw.qweight[sl], qw.scales[sl], qw.zeros[sl], n, qw.n_in, 128),
                               x, y[:, sl]))
            off += n
    res["gbs_7_launches_per_layer"] = None
    if not args.decode_only:
        graph7 = capture(lambda: [w4.gemv(x, q, y) for q, x, y in per_linear])
        el7, _ = time_graph(graph7, max(1, args.steps // 2), 1)
        res["gbs_7_launches_per_layer"] = round(step_bytes * max(1, args.steps // 2) / el7 / 1e9, 1)
        del graph7
    return res, host_w


def cpu_baseline(host_w, budget_s):
    """Oracle GEMV (dequantize, then binary64 product) on layer 0's four
    fused linears, repeated until about `budget_s` seconds of CPU work."""
    import numpy as np
    import oracle
    orc = oracle.load()
    prepared = []
    for name, w, x in host_w:
        packed, scales, zeros, _ = orc.quantize_pack(w, 128)      # untimed preparation
        prepared.append((name, packed, scales, zeros, x.view(np.uint16)))
    done_bytes, t_cpu, n_lin = 0, 0.0, 0
    while t_cpu < budget_s:
        for name, packed, scales, zeros, x in prepared:
            t0 = time.perf_counter()
            orc.linear_from_packed(x, packed, scales, zeros, 128)
            t_cpu += time.perf_counter() - t0
            done_bytes += algorithmic_bytes(packed.shape[0], packed.shape[1] * 8, 1, 128)
            n_lin += 1
            if t_cpu >= budget_s:
                break
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return dict(value=round(done_bytes / t_cpu / 1e9, 3), unit="GB/s", cores=cores, kind="oracle",
                sample=(f"{n_lin} fused decode GEMVs of the 7B layer-0 shapes (qkv 12288x4096, o 4096x4096, "
                        f"gate_up 22016x4096, down 4096x11008; m=1, g=128) through the C oracle's "
                        f"dequantize + binary64 product, {t_cpu:.1f} s of CPU time"))


def bench_prefill(args, dev):
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    out, tot_flop, tot_t = [], 0, 0.0
    for i, lin in enumerate(syn.PREFILL_LINEARS):
        w = syn.normal_weight_device(lin.n_out, lin.n_in, 4000 + i, 0.02, syn.n_outliers(lin.n_in), dev)
        qw = w4.quantize_pack(w, 128)
        del w
        x = syn.activations_f16_device(syn.PREFILL_M, lin.n_in, 4100 + i, dev)
        y = torch.empty((syn.PREFILL_M, lin.n_out), dtype=torch.float16, device=dev)
        reps = 20
        g = capture(lambda: [w4.gemm(x, qw, y) for _ in range(reps)])
        settle(g)
        el, _ = time_graph(g, 5, 3)
        t = el / (5 * reps)
        flop = 2 * syn.PREFILL_M * lin.n_out * lin.n_in
        out.append(dict(shape=f"{syn.PREFILL_M}x{lin.n_out}x{lin.n_in}", us=round(t * 1e6, 2),
                        tflops=round(flop / t / 1e12, 1)))
        tot_flop += flop
        tot_t += t
    return dict(shapes=out, tflops=round(tot_flop / tot_t / 1e12, 1))


def bench_decode70b(args, dev):
    """80 layers of 70B-shaped linears at m=8, stored fused like the 7B stack:
    qkv [10240, 8192], o [8192, 8192], gate_up [57344, 8192], down [8192, 28672]."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    layers = syn.LLAMA70B_LAYERS if not args.quick else 8
    lin = syn.LLAMA70B_LINEARS
    fused = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
    xs = {name: syn.activations_f16_device(8, lin[idx[0]].n_in, 3100 + j, dev)
          for j, (name, idx) in enumerate(fused)}
    gemvs = []
    t0 = time.perf_counter()
    for layer in range(layers):
        for name, idx in fused:
            w = torch.cat([syn.normal_weight_device(lin[i].n_out, lin[i].n_in, syn.llama70b_seed(layer, i),
                                                    0.015, 0, dev) for i in idx])
            qw = w4.quantize_pack(w, 128)
            del w
            gemvs.append((qw, xs[name], torch.empty((8, qw.n_out), dtype=torch.float16, device=dev)))
    torch.cuda.synchronize()
    log(f"70B stack: {layers} layers quantized in {time.perf_counter() - t0:.1f} s")
    g = capture(lambda: [w4.gemv(x, qw, y) for qw, x, y in gemvs])
    el, _ = time_graph(g, 5, 1)
    nbytes = sum(algorithmic_bytes(qw.n_out, qw.n_in, 8, 128) for qw, _, _ in gemvs)
    res = dict(layers=layers, m=8, gemvs_per_pass=len(gemvs), ms_per_pass=round(el / 5 * 1e3, 3),
               gbs=round(nbytes * 5 / el / 1e9, 1), resident_gb=round(nbytes / 1e9, 2))
    del gemvs, g
    torch.cuda.empty_cache()
    return res


def student_t_device(n_out, n_in, seed, dev):
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    z = torch.randn((n_out, n_in), generator=gen, device=dev)
    chi2 = torch.zeros_like(z)
    for _ in range(3):
        chi2.addcmul_(e := torch.randn((n_out, n_in), generator=gen, device=dev), e)
    return z.mul_(torch.rsqrt(chi2.div_(3.0))).mul_(0.02)


def bench_single(args, dev):
    """One 4096x4096 linear at m=1 (g=128), cycled over 64 distinct packed copies
    (about 570 MB, beyond the 256 MB Infinity Cache) inside one graph: the
    latency-dominated single-GEMV case."""
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    n_out = n_in = 4096
    w = syn.normal_weight_device(n_out, n_in, 1, 0.02, 8, dev)
    qws = [w4.quantize_pack(w.mul(1.0 + c * 1e-3) if c else w, 128) for c in range(64)]
    del w
    x = syn.activations_f16_device(1, n_in, 101, dev)
    y = torch.empty((1, n_out), dtype=torch.float16, device=dev)
    gr = capture(lambda: [w4.gemv(x, q, y) for q in qws])
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
    lin = syn.LLAMA7B_LINEARS
    fused = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))
    xs = {name: syn.activations_f16_device(1, lin[idx[0]].n_in, 2200 + j, dev)
          for j, (name, idx) in enumerate(fused)}
    layers, gemvs = 8, []
    for layer in range(layers):
        for name, idx in fused:
            w = torch.cat([syn.normal_weight_device(lin[i].n_out, lin[i].n_in, syn.llama7b_seed(layer, i),
                                                    0.02, syn.n_outliers(lin[i].n_in), dev) for i in idx])
            qw = w4.quantize_pack(w, None, bits=8)
            del w
            gemvs.append((qw, xs[name], torch.empty((1, qw.n_out), dtype=torch.float16, device=dev)))
    g = capture(lambda: [w4.gemv(x, qw, y) for qw, x, y in gemvs])
    el, _ = time_graph(g, 10, 2)
    nbytes = sum(algorithmic_bytes(qw.n_out, qw.n_in, 1, qw.n_in, 8) for qw, _, _ in gemvs)
    res = dict(decode_layers=layers, decode_m=1, decode_group="per-channel",
               decode_gbs=round(nbytes * 10 / el / 1e9, 1),
               decode_us_per_launch=round(el / (10 * len(gemvs)) * 1e6, 2))
    del gemvs, g
    out, tot_flop, tot_t = [], 0, 0.0
    for i, pl in enumerate(syn.PREFILL_LINEARS):
        w = syn.normal_weight_device(pl.n_out, pl.n_in, 4000 + i, 0.02, syn.n_outliers(pl.n_in), dev)
        qw = w4.quantize_pack(w, 128, bits=8)
        del w
        x = syn.activations_f16_device(syn.PREFILL_M, pl.n_in, 4100 + i, dev)
        y = torch.empty((syn.PREFILL_M, pl.n_out), dtype=torch.float16, device=dev)
        reps = 20
        gr = capture(lambda: [w4.gemm(x, qw, y) for _ in range(reps)])
        settle(gr)
        el, _ = time_graph(gr, 5, 3)
        t = el / (5 * reps)
        flop = 2 * syn.PREFILL_M * pl.n_out * pl.n_in
        out.append(dict(shape=f"{syn.PREFILL_M}x{pl.n_out}x{pl.n_in}", tflops=round(flop / t / 1e12, 1)))
        tot_flop += flop
        tot_t += t
    res["prefill_g128_shapes"] = out
    res["prefill_g128_tflops"] = round(tot_flop / tot_t / 1e12, 1)
    torch.cuda.empty_cache()
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
        w = syn.normal_weight_device(lin.n_out, lin.n_in, 4000 + i, 0.02, syn.n_outliers(lin.n_in), dev)
        calib = syn.activations_f16_device(512, lin.n_in, 4200 + i, dev)
        act_max = torch.zeros(lin.n_in, dtype=torch.float32, device=dev)
        w8a8.absmax_update(calib, act_max)
        layer = w8a8.W8A8Linear.from_float(w, act_max)
        del w, calib
        x = syn.activations_f16_device(syn.PREFILL_M, lin.n_in, 4100 + i, dev)
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


def bench_stress_and_quantize(args, dev):
    import torch
    import w4a16_dequant_gemv_amd as w4
    from w4a16_dequant_gemv_amd import synthetic as syn
    n_out, n_in = 8192, 28672
    w = student_t_device(n_out, n_in, 5, dev)
    x = syn.activations_f16_device(1, n_in, 5100, dev)
    res = {}
    for g in (128, 32):
        qws = [w4.quantize_pack(w, g)]
        for c in range(1, 3):          # three copies (3 x 125-147 MB) to defeat the cache
            qws.append(w4.quantize_pack(w.mul(1.0 + c * 1e-3), g))
        y = torch.empty((1, n_out), dtype=torch.float16, device=dev)
        reps = 8
        gr = capture(lambda: [w4.gemv(x, qws[r % 3], y) for r in range(reps * 3)])
        el, _ = time_graph(gr, 3, 1)
        t = el / (3 * reps * 3)
        res[f"gemv_g{g}_gbs"] = round(algorithmic_bytes(n_out, n_in, 1, g) / t / 1e9, 1)
        res[f"gemv_g{g}_us"] = round(t * 1e6, 2)
        del qws, gr
    qw = w4.quantize_pack(w, 128)
    out = torch.empty_like(w)
    gq = capture(lambda: [w4.quantize_pack(w, 128, out=qw) for _ in range(5)])
    el, _ = time_graph(gq, 2, 1)
    qbytes = n_out * n_in * 4 + n_out * n_in // 2 + n_out * (n_in // 128) * 4
    res["quantize_g128_gbs"] = round(qbytes * 10 / el / 1e9, 1)
    gd = capture(lambda: [w4.dequant(qw, out) for _ in range(5)])
    el, _ = time_graph(gd, 2, 1)
    res["dequant_g128_gbs"] = round(qbytes * 10 / el / 1e9, 1)
    del w, out
    torch.cuda.empty_cache()
    return res


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one elementwise copy of 256 MiB (268435456 bytes read and written), "
                         "the known-size kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

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
        log(f"prefill: {pre}")
        print(json.dumps({
            "metric": "W4A16 prefill GEMM TFLOP/s (m=2048)", "value": pre["tflops"], "unit": "TFLOP/s",
            "n_gpus": 1, "higher_is_better": True, "dtype": "int4 weights x fp16 activations, fp32 accumulate",
            "data": "synthetic", "config": {"workload": "prefill m=2048 on the 7B linear shapes"},
            "prefill": pre, "roofline": {"bound": "mfma", "achieved": pre["tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(pre["tflops"] / MFMA_F16_PEAK_TFLOPS, 4)}}),
              flush=True)
        return
    if args.decode_only:
        args.no_extras = True
        args.no_cpu_baseline = True
    decode, host_w = bench_decode(args, dev)
    log(f"decode: {decode['gbs']:.1f} GB/s, {decode['ms_per_step']:.3f} ms/step, "
        f"{decode['per_launch_us']:.2f} us per GEMV launch")
    extras = {}
    if not args.no_extras:
        extras["prefill"] = bench_prefill(args, dev)
        log(f"prefill: {extras['prefill']}")
        extras["decode70b"] = bench_decode70b(args, dev)
        log(f"decode70b: {extras['decode70b']}")
        extras["stress"] = bench_stress_and_quantize(args, dev)
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
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host_w, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    achieved = decode["bytes_per_launch"] / (decode["per_launch_us"] * 1e-6) / 1e9
    traffic = counters_traffic(decode["bytes_per_launch"])
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
                     "kernel": "q4_gemv (gemv_kernel)", "avg_launch_us": round(decode["per_launch_us"], 3),
                     "bytes_per_launch": round(decode["bytes_per_launch"])},
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(decode["wall"], 4),
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
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
