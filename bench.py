#!/usr/bin/env python3
"""Benchmark of the W4A16 routed-expert layer on one MI355X.

Workload: a stack of 30 distinct full-shape layers (T=256 canvas rows, 128
experts, top-8, d=2816, m=704, gate_up groups of 128, down groups of 64),
each with its own seeded weights, activations and routing, run back to back
in rotation so that the 12.4 GB of packed weights stream from HBM rather
than from the 256 MB Infinity Cache. One step = one layer forward
(alignment, gate_up + gated GELU, down, fixed-order combine) through the
C ABI. Inputs are resident in HBM before the timed region starts.

Prints one JSON line: achieved algorithmic HBM throughput (GB/s) over the
timed steps, microseconds per layer, the roofline of the dominant kernel
(the one launch of gate_up and down, timed live with HIP events around it in
a separate pass) and the CPU oracle timed on the host on one layer.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

METRIC = "µs/MoE layer + achieved HBM GB/s (% of 8 TB/s), T=256, 128e top-8 W4A16"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # dense fp16 MFMA, MI355X
# The pages' GB10 figure for one W4 MoE layer at M=256 (Part 2 blog, "Start
# with the measured machine"): 2.366 ms. As GB/s on this layer's algorithmic
# bytes it is context from another machine, not a target.
GB10_LAYER_MS = 2.366
# Steps of the separate pass that splits a step into its stages, and sweeps
# of the rotated stack for the spread and the graph replay (see main()).
STAGE_STEPS = 300
SWEEPS = 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(shape, populated: int) -> dict:
    """Algorithmic HBM bytes of one layer and of its two GEMM kernels."""
    E, d, m, T, k = shape.E, shape.d, shape.m, shape.T, shape.topk
    A = T * k
    gu_w = 2 * m * d // 2 + 2 * (2 * m) * (d // shape.g_gu) * 2     # nibbles + fp16 s, z
    dn_w = d * m // 2 + 2 * d * (m // shape.g_dn) * 2
    x = T * d * 2
    out = T * d * 2
    route = A * 4 * 2                                                 # ids + weights
    # the GEMM launches' algorithmic bytes: the packed weights of the
    # populated experts plus the activations they read from the caller (x);
    # the workspace traffic of H, Y and the sorted ids is implementation
    # overhead and not counted
    return dict(
        layer=populated * (gu_w + dn_w) + x + out + route,
        gate_up=populated * gu_w + x,
        down=populated * dn_w,
        weights=populated * (gu_w + dn_w),
    )


TRAFFIC_PROFILE = "profiles/expert_stages_hbm_traffic_stack_skew_wide.md"
TRAFFIC_SOURCES = ("w4a16_grouped_moe_amd/csrc/moe_gemm.hip",
                   "w4a16_grouped_moe_amd/csrc/gemm_common.hpp",
                   "w4a16_grouped_moe_amd/csrc/dgw4_internal.hpp",
                   "w4a16_grouped_moe_amd/csrc/wide_gemm.hpp",
                   "w4a16_grouped_moe_amd/csrc/chunk_gate_up.hip",
                   "w4a16_grouped_moe_amd/csrc/chunk_down.hip",
                   "w4a16_grouped_moe_amd/csrc/align.hip")


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_key(shape, layout: str, row_block: int) -> dict:
    """What a counter record must have been taken on to describe this run."""
    return {"T": shape.T, "E": shape.E, "topk": shape.topk, "d": shape.d, "m": shape.m,
            "g_gu": shape.g_gu, "g_dn": shape.g_dn,
            "routing": f"zipf({shape.zipf})" if shape.zipf else "uniform", "layout": layout,
            "row_block": row_block}


def measured_traffic(key: dict) -> dict | None:
    """HBM bytes per launch of the GEMM kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads
    for a plain copy of known size), or None when no record was taken on this
    workload (token count, routing, weight layout) or the GEMM sources
    changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), TRAFFIC_PROFILE)
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    recs = json.loads(m.group(1))
    for rec in recs if isinstance(recs, list) else [recs]:
        if rec.get("source_sha256") == gemm_source_hash() and rec.get("workload") == key:
            return rec
    return None


def make_layer(torch, dg, shape, l: int, dev, layout: str = "tiled", keep_masters: bool = False) -> dict:
    """Layer l of a workload as the benchmark runs it: fp32 master weights
    drawn on the device (seeded), packed there by dgw4_quantize_rtn, the
    tiled copies made by dgw4_pack_tiled (a load-time conversion, outside
    every timed region), activations from the host generator, and the
    routing from the seeded router logits through the library's router
    (dgw4_router) on the device.
    ``gu``/``dn`` are the packs in ``layout``, ``gu_other``/``dn_other`` the
    other layout's. keep_masters also returns the fp32 masters (on the
    device), for auditing a layer against the oracle."""
    from synth import activations, expert_weights_device, router_logits
    gw, dw = expert_weights_device(shape, l, dev)
    gu_c = (*dg.quantize_rtn(gw, shape.g_gu), shape.g_gu)
    dn_c = (*dg.quantize_rtn(dw, shape.g_dn), shape.g_dn)
    masters = (gw, dw) if keep_masters else None
    del gw, dw
    gu_t, dn_t = dg.pack_tiled(gu_c), dg.pack_tiled(dn_c)
    tiled = layout == "tiled"
    x = activations(shape, l)
    logits = router_logits(shape, l)
    ids_d, w_d = dg.router(torch.from_numpy(logits).to(dev), shape.topk)
    ids = ids_d.cpu().numpy()
    populated = int(np.unique(ids).size)
    return dict(
        gu=gu_t if tiled else gu_c, dn=dn_t if tiled else dn_c,
        gu_other=gu_c if tiled else gu_t, dn_other=dn_c if tiled else dn_t,
        x=torch.from_numpy(x).to(dev), ids=ids_d, w=w_d, bytes=layer_bytes(shape, populated),
        populated=populated, masters=masters, x_host=x, logits_host=logits)


def graph_replay(torch, dg, step, L, R, out, last, ws, dev, rows: str = "auto") -> dict:
    """Capture one sweep of L layer forwards into a HIP graph, replay it R
    times, and compare the last layer's output with an eager forward."""
    stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)              # default priority
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(L):
            step(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    ev[0].record(stream)
    for r in range(R):
        g.replay()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[r].elapsed_time(ev[r + 1]) * 1e3 / L for r in range(R)])
    replayed = out.clone()
    eager = dg.moe_forward(last["x"], last["ids"], last["w"], last["gu"], last["dn"], workspace=ws,
                           rows=rows)
    torch.cuda.synchronize()
    same = bool(torch.equal(replayed.view(torch.int16), eager.view(torch.int16)))
    del g
    return {"replays": R, "layers_per_replay": L,
            "median_us_per_layer": round(float(np.median(us)), 2),
            "p10_us_per_layer": round(float(np.percentile(us, 10)), 2),
            "p90_us_per_layer": round(float(np.percentile(us, 90)), 2),
            "bitwise_equal_to_eager": same}


def read_probe(torch, dg, dev, gib: int = 2, reps: int = 10) -> dict:
    """On-box HBM read ceiling: the library's whole-chip read of a `gib` GiB
    buffer (8x the 256 MB Infinity Cache, so it streams from HBM)."""
    n = gib << 30
    buf = torch.ones(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        dg.hbm_read_probe(buf, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dg.hbm_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    return {"kind": f"whole-chip read of a {gib} GiB buffer (dgw4_hbm_read_probe)",
            "gbps": round(gbps, 1)}


def mfma_probe(torch, dg, dev, iters: int = 20000, reps: int = 5) -> dict:
    """On-box dense fp16 MFMA ceiling: the library's whole-chip MFMA probe
    (register operands, no memory traffic)."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    dg.mfma_probe(iters // 10, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    flops = sum(dg.mfma_probe(iters, sink) for _ in range(reps))
    e1.record()
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"kind": "whole-chip v_mfma_f32_16x16x32_f16 on register operands (dgw4_mfma_probe)",
            "tflops": round(tflops, 1)}


def _time_calls(torch, fn, calls: int) -> float:
    """us per call of fn over `calls` back-to-back calls (after two warm-ups)."""
    fn()
    fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(calls):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def dense_comparison(torch, dg, dev, xd, w4, w4_us: float, calls: int) -> dict:
    """The pages compare their dense W4A16 kernels with the dense 16-bit GEMM
    at 256 rows (an LM-head tile, QKV). Here: torch's F.linear (hipBLASLt) in
    bf16 and fp16 on the same x and a random [N, K] weight of the same size,
    at the LM-head shape, and at 256 x 2816 x N for N = 4096 .. 16384 against
    this library's linear (the pages give no QKV width, so a range of widths
    stands in for one)."""
    import torch.nn.functional as F
    T, K = xd.shape
    N = 262144
    out = {"lmhead": {"w4a16_us": round(w4_us, 1)}}
    for name, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        wd = torch.randn((N, K), device=dev, dtype=dt)
        xt = xd.to(dt)
        us = _time_calls(torch, lambda: F.linear(xt, wd), calls)
        out["lmhead"][f"{name}_us"] = round(us, 1)
        out["lmhead"][f"w4a16_speedup_vs_{name}"] = round(us / w4_us, 3)
        del wd, xt
    log(f"[linear] F.linear at the LM-head shape: bf16 {out['lmhead']['bf16_us']} us, "
        f"f16 {out['lmhead']['f16_us']} us; W4A16 {w4_us:.1f} us")
    rows = []
    if w4 is not None:
        for n in (4096, 8192, 16384):
            wq = tuple(t[:n] for t in w4[:3]) + (w4[3],)      # the first n rows of the tiled matrix
            w4us = _time_calls(torch, lambda: dg.w4a16_linear(xd, wq), 50)
            wd = torch.randn((n, K), device=dev, dtype=torch.bfloat16)
            xt = xd.to(torch.bfloat16)
            bus = _time_calls(torch, lambda: F.linear(xt, wd), 50)
            rows.append({"N": n, "w4a16_us": round(w4us, 1), "bf16_us": round(bus, 1),
                         "w4a16_speedup_vs_bf16": round(bus / w4us, 3),
                         "row_block": dg.linear_row_block(T, K, n, w4[3])})
            log(f"[linear] T={T} K={K} N={n}: W4A16 {w4us:.1f} us, bf16 F.linear {bus:.1f} us")
            del wd, xt
        out["narrow"] = rows
    return out


def bench_linear(torch, dg, dev, args) -> int:
    """The dense W4A16 linear at an LM-head shape: x fp16 [256, 2816] against
    one packed [262144, 2816] matrix (392 MB of nibbles, scales and zeros:
    more than the 256 MB Infinity Cache, so it streams from HBM on every
    call). Prints one JSON line of its own."""
    from synth import linear_inputs
    T, K, N, g = 256, 2816, 262144, 128
    x, _ = linear_inputs(5, T, K, 16)
    xd = torch.from_numpy(x).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    wd = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32).mul_(0.02)
    q, s_, z = dg.quantize_rtn(wd, g)
    del wd
    y = torch.empty((T, N), dtype=torch.float16, device=dev)
    w = (q, s_, z, g)
    if args.weight_layout == "tiled":
        w = dg.pack_tiled(w)
        del q
    stream = torch.cuda.current_stream(dev)
    for _ in range(max(1, args.warmup // 30)):
        dg.w4a16_linear(xd, w, out=y)
    steps = max(1, args.steps // 30)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        dg.w4a16_linear(xd, w, out=y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    wbytes = N * K // 2 + 2 * N * (K // g) * 2
    nbytes = wbytes + T * K * 2 + T * N * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    flops = 2 * T * K * N
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[linear] {steps} calls: {ms * 1e3:.1f} us each, {gbps:.1f} GB/s, {tflops:.1f} TFLOP/s")
    del y
    dense = dense_comparison(torch, dg, dev, xd, w if args.weight_layout == "tiled" else None,
                             ms * 1e3, steps)
    probe = mfma_probe(torch, dg, dev)
    probe["pct_of_probe"] = round(100 * tflops / probe["tflops"], 2)
    log(f"[linear] MFMA probe {probe['tflops']} TFLOP/s; the linear at {probe['pct_of_probe']}% of it")
    print(json.dumps({
        "metric": "us per dense W4A16 linear + achieved HBM GB/s (% of 8 TB/s)",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": max(1, args.warmup // 30), "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"dense W4A16 linear (LM-head shape): T={T}, K={K}, N={N}, g={g}",
                   "weight_layout": args.weight_layout},
        "us_per_call": round(ms * 1e3, 2), "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_call": nbytes,
        "mfma_probe": probe,
        "dense_f16_bf16": dense,
        # 2 T K N FLOP over 392 MB of weights is 4 T = 1024 FLOP per byte,
        # far past the fp16 ridge (2.5 PFLOP/s over 8 TB/s = 312): MFMA-bound
        "roofline": {"kernel": (f"linear_wide_kernel<128, 22, {str(args.weight_layout == 'tiled').lower()}, "
                                f"{str(args.weight_layout == 'tiled').lower()}> (256-row blocks, each "
                                f"weight formed once per block)"),
                     "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "flops_per_call": flops, "traffic": None},
    }), flush=True)
    return 0


def bench_sampler(torch, dg, dev, args) -> int:
    """The sampler of a denoising step on the pages' tensor: fp32 logits
    [256, 262144] (268 MB, more than the Infinity Cache, rotated over 4
    copies), one pass for entropy, Gumbel-max sample and argmax; also the
    entropy-only pass. Prints one JSON line of its own."""
    from synth import sampler_logits
    R, V = 256, 262144
    copies = [torch.from_numpy(sampler_logits(31 + c, R, V, 2.0)).to(dev) for c in range(4)]
    n = R * V * 4
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(entropy: bool, draw: bool) -> float:
        for i in range(8):
            dg.sample(copies[i % 4], i, entropy=entropy, draw=draw, workspace=ws)
        steps = max(20, args.steps // 30)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            dg.sample(copies[i % 4], i, entropy=entropy, draw=draw, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    ms_all = timed(True, True)
    ms_ent = timed(True, False)
    probe = read_probe(torch, dg, dev)
    gbps = n / (ms_all * 1e-3) / 1e9
    gbps_ent = n / (ms_ent * 1e-3) / 1e9
    log(f"[sampler] entropy+sample+argmax {ms_all * 1e3:.1f} us ({gbps:.1f} GB/s); "
        f"entropy+argmax {ms_ent * 1e3:.1f} us ({gbps_ent:.1f} GB/s); read probe {probe['gbps']} GB/s")
    print(json.dumps({
        "metric": "us per sampler pass (entropy + Gumbel-max sample + argmax) + achieved HBM GB/s",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": max(20, args.steps // 30),
        "warmup": 8, "ms_per_step": round(ms_all, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"sampler: fp32 logits [{R}, {V}] ~ N(0, 2), 4 copies in rotation"},
        "us_per_call": round(ms_all * 1e3, 2), "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "entropy_only": {"us_per_call": round(ms_ent * 1e3, 2), "gbps": round(gbps_ent, 1),
                         "pct_of_8TBps": round(100 * gbps_ent / HBM_PEAK_GBPS, 2)},
        "hbm_probe": probe,
        # time source: HIP events around the timed passes, each the partial
        # kernel plus the small merge, so `achieved` is a lower bound on the
        # partial kernel's own rate
        "roofline": {"kernel": "sample_partial_kernel<true> + sample_merge_kernel (one pass)", "bound": "hbm",
                     "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None},
    }), flush=True)
    return 0


CPU_SAMPLE_TOKENS = 16


def cpu_baseline(shape, runs: int = 3):
    """The CPU oracle, as it stands, on a bounded sample of the workload: the
    first CPU_SAMPLE_TOKENS tokens of one full layer drawn on the host (all
    their top-k assignments through the full-size experts), timed as the
    median of `runs` runs at one thread and at every core this process may
    use. The rate is scaled to the whole layer (the oracle's work is linear
    in the tokens): layer bytes / (sample seconds x T / sample tokens)."""
    import oracle
    from synth import activations, expert_weights, router_logits
    t0 = time.time()
    gw, dw = expert_weights(shape, 0)
    gu = (*oracle.quantize_rtn(gw, shape.g_gu), shape.g_gu)
    del gw
    dn = (*oracle.quantize_rtn(dw, shape.g_dn), shape.g_dn)
    del dw
    x = activations(shape, 0)
    ids, w = oracle.router(router_logits(shape, 0), shape.topk)
    w = w.astype(np.float32)
    toks = np.arange(CPU_SAMPLE_TOKENS, dtype=np.int32)
    populated = int(np.unique(ids).size)
    nbytes = layer_bytes(shape, populated)["layer"]
    log(f"[cpu] inputs ready in {time.time() - t0:.1f}s; timing the oracle forward")
    all_cores = len(os.sched_getaffinity(0))
    legs = {}
    for n in (1, all_cores):
        used = oracle.set_threads(n)
        secs = []
        for _ in range(runs):
            t1 = time.perf_counter()
            oracle.moe_forward(x, ids, w, gu, dn, shape.E, tokens=toks)
            secs.append(time.perf_counter() - t1)
        sec = float(np.median(secs))
        layer_sec = sec * shape.T / CPU_SAMPLE_TOKENS
        legs[n] = dict(value=round(nbytes / layer_sec / 1e9, 4), cores=used,
                       sample_seconds=[round(v, 3) for v in secs],
                       seconds_per_layer=round(layer_sec, 3))
        log(f"[cpu] oracle on {used} threads: {sec:.2f} s per {CPU_SAMPLE_TOKENS}-token sample "
            f"(median of {runs}), {layer_sec:.2f} s per layer, {legs[n]['value']} GB/s")
    top = legs[all_cores]
    return {"value": top["value"], "unit": "GB/s", "cores": top["cores"], "kind": "oracle",
            "sample": (f"the first {CPU_SAMPLE_TOKENS} of {shape.T} tokens of one full layer "
                       f"(E={shape.E}, top-{shape.topk}, d={shape.d}, m={shape.m}) drawn on the "
                       f"host; median of {runs} runs, scaled to the whole layer"),
            "seconds_per_layer": top["seconds_per_layer"],
            "sample_seconds": top["sample_seconds"],
            "one_thread": legs[1]}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000, help="timed layer forwards")
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--layers", type=int, default=30, help="distinct weight sets in rotation")
    ap.add_argument("--workload", default="stack", choices=["stack", "full", "skew", "wide", "down_g64", "down_g128", "lmhead",
                             "sampler"],
                    help="lmhead: the dense W4A16 linear at T=256, K=2816, N=262144; sampler: "
                         "entropy + Gumbel-max sample + argmax over [256, 262144] fp32 logits "
                         "(neither is the layer)")
    ap.add_argument("--weight-layout", default="tiled", choices=["tiled", "canonical"],
                    help="layout of the packed weights the timed steps read (both give "
                         "identical results; the other one is timed in a short pass too)")
    ap.add_argument("--rows", default="auto", choices=["auto", "tiles", "chunks"],
                    help="row blocks of the expert GEMMs: the library's choice (default), "
                         "32-row tiles or 128-row chunks (see DGW4_ROWS_* in include/dgw4.h)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB 5 times (the counter "
                         "calibration kernel for HBM traffic) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this layer "
              "has no multi-GPU path; see the sharding paragraph in DESIGN.md.", file=sys.stderr)
        return 2

    import torch
    import w4a16_grouped_moe_amd as dg
    from synth import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm device", file=sys.stderr)
        return 2
    dg.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[copy] 5 copies of {n} bytes")
        return 0
    if args.workload == "lmhead":
        return bench_linear(torch, dg, dev, args)
    if args.workload == "sampler":
        return bench_sampler(torch, dg, dev, args)
    shape = CONFIGS[args.workload]
    L = args.layers if args.workload == "stack" else 1
    if args.workload != "stack":
        L = max(1, args.layers)          # rotate weight sets for single-layer workloads too

    t0 = time.time()
    layers = [make_layer(torch, dg, shape, l, dev, args.weight_layout) for l in range(L)]
    torch.cuda.synchronize()
    log(f"[bench] {L} layers packed on the device in {time.time() - t0:.1f}s "
        f"({sum(x['bytes']['weights'] for x in layers) / 1e9:.2f} GB of packed weights touched)")

    # (the workspace depends on the row blocks the library picks, which
    # depend on the weight layout: size it for both layouts the steps use)
    ws = torch.empty(max(dg.workspace_bytes(shape.T, shape.topk, shape.E, shape.d, shape.m,
                                            layers[0][k][3], layers[0][j][3],
                                            rows=args.rows if k == "gu" else "auto")
                         for k, j in (("gu", "dn"), ("gu_other", "dn_other"))),
                     dtype=torch.uint8, device=dev)
    row_block = dg.row_block(shape.T, shape.topk, shape.E, shape.d, shape.m,
                             layers[0]["gu"][3], layers[0]["dn"][3], rows=args.rows)
    log(f"[bench] expert GEMMs on {'128-row chunks' if row_block == 128 else '32-row tiles'}")
    out = torch.empty((shape.T, shape.d), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, events=None, other=False):
        ly = layers[i % L]
        gu, dn = (ly["gu_other"], ly["dn_other"]) if other else (ly["gu"], ly["dn"])
        # (the other layout's pass takes the library's choice: chunks need
        # tiled weights)
        dg.moe_forward(ly["x"], ly["ids"], ly["w"], gu, dn, workspace=ws, out=out,
                       events=events, rows="auto" if other else args.rows)

    for i in range(args.warmup):
        step(i)
    K = args.steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    # Spread: R sweeps of the rotated stack, each bracketed by events (a pass
    # of its own, so the timed steps above carry no events).
    R = SWEEPS
    sw = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    torch.cuda.synchronize()
    sw[0].record(stream)
    for r in range(R):
        for i in range(L):
            step(i)
        sw[r + 1].record(stream)
    torch.cuda.synchronize()
    sweep_us = np.array([sw[r].elapsed_time(sw[r + 1]) * 1e3 / L for r in range(R)])
    spread = {"sweeps": R, "layers_per_sweep": L,
              "median_us_per_layer": round(float(np.median(sweep_us)), 2),
              "p10_us_per_layer": round(float(np.percentile(sweep_us, 10)), 2),
              "p90_us_per_layer": round(float(np.percentile(sweep_us, 90)), 2)}

    # The same sweeps on the other weight layout (same results, other load
    # addresses), for comparison.
    torch.cuda.synchronize()
    sw[0].record(stream)
    for r in range(R):
        for i in range(L):
            step(i, other=True)
        sw[r + 1].record(stream)
    torch.cuda.synchronize()
    other_us = np.array([sw[r].elapsed_time(sw[r + 1]) * 1e3 / L for r in range(R)])
    other_layout = "canonical" if args.weight_layout == "tiled" else "tiled"
    spread[f"{other_layout}_layout_median_us_per_layer"] = round(float(np.median(other_us)), 2)

    # The same sweep replayed as one HIP graph (captured once; every replay
    # re-runs alignment and both GEMMs on the device), checked bitwise
    # against the eager result of its last layer.
    graph = graph_replay(torch, dg, step, L, R, out, layers[L - 1], ws, dev, args.rows)

    # Stage split, in a pass of its own after the timed region: each recorded
    # event adds a few microseconds of dispatch gap, so they stay out of the
    # steps that give the throughput. At the layer's shape alignment, gate_up
    # and down are one launch: events 0 -> 1 bracket it, 1 -> 2 and 2 -> 3 no
    # kernel.
    S = min(K, STAGE_STEPS)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(S)]
    for e in evs:                       # create the HIP events before the pass
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    for i in range(S):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])

    # The dominant kernel alone: S launches of the expert stages (no combine)
    # back to back over the rotated layers, HIP events on the launch stream at
    # the two ends only, so the average includes no event's dispatch gap.
    def experts(i):
        ly = layers[i % L]
        dg.moe_experts(ly["x"], ly["ids"], ly["gu"], ly["dn"], ws, rows=args.rows)
    for i in range(L):
        experts(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(S):
        experts(i)
    e1.record(stream)
    torch.cuda.synchronize()
    kern_us = e0.elapsed_time(e1) * 1e3 / S
    kern_bytes = sum(layers[i % L]["bytes"]["gate_up"] + layers[i % L]["bytes"]["down"]
                     for i in range(S)) / S

    # The layer from router logits (dgw4_moe_forward_routed: the router
    # kernel, then the layer) over the same steps, and the router alone.
    logits_d = [torch.from_numpy(layers[i]["logits_host"]).to(dev) for i in range(L)]
    rids = torch.empty((shape.T, shape.topk), dtype=torch.int32, device=dev)
    rw = torch.empty((shape.T, shape.topk), dtype=torch.float32, device=dev)

    def routed(i):
        ly = layers[i % L]
        dg.moe_forward_routed(ly["x"], logits_d[i % L], shape.topk, ly["gu"], ly["dn"],
                              workspace=ws, out=out, rows=args.rows)

    def router_only(i):
        dg.router(logits_d[i % L], shape.topk, rids, rw)

    routed_us = {}
    for name, fn, n in (("routed_forward", routed, K), ("router_alone", router_only, S)):
        for i in range(L):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        routed_us[name] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
    log(f"[bench] from router logits: {routed_us['routed_forward']} us per layer; "
        f"router alone {routed_us['router_alone']} us back to back")

    moved = sum(layers[i % L]["bytes"]["layer"] for i in range(K))
    ms_per_step = total_ms / K
    gbps = moved / (total_ms * 1e-3) / 1e9
    fused = row_block == 32 and (shape.d, shape.m, shape.g_gu, shape.g_dn) == (2816, 704, 128, 64)
    names = ("layer_kernel", "gap", "gap2", "combine") if fused else \
        ("align", "gate_up", "down", "combine")
    stage_us = {n: round(float(stage_ms[:, j].mean() * 1e3), 2) for j, n in enumerate(names)}
    kern_gbps = kern_bytes / (kern_us * 1e-6) / 1e9
    log(f"[bench] {K} steps in {total_ms:.2f} ms: {ms_per_step * 1e3:.2f} us/layer, "
        f"{gbps:.1f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")
    log(f"[bench] stages over {S} steps (us): {stage_us}")
    log(f"[bench] expert kernel(s) alone, {S} back to back: {kern_us:.2f} us per launch, "
        f"{kern_gbps:.1f} GB/s")

    probe = read_probe(torch, dg, dev)
    probe["pct_of_probe"] = round(100 * gbps / probe["gbps"], 2)
    traffic = measured_traffic(traffic_key(shape, args.weight_layout, row_block))
    pages_gbps = layers[0]["bytes"]["layer"] / (GB10_LAYER_MS * 1e-3) / 1e9
    kern_flops = 2 * shape.T * shape.topk * (2 * shape.m * shape.d + shape.d * shape.m)
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(gbps / pages_gbps, 2),
        "vs_baseline_note": (f"ratio to the pages' GB10 figure for one layer at M=256 "
                             f"(2.366 ms = {pages_gbps:.1f} GB/s on the same algorithmic "
                             f"bytes); another machine, context only"),
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"{'rotated ' + str(L) + '-layer stack' if L > 1 else 'one layer'}: "
                         f"T={shape.T}, E={shape.E}, top-{shape.topk}, d={shape.d}, "
                         f"m={shape.m}, gate_up g={shape.g_gu}, down g={shape.g_dn}"
                         + (f", Zipf({shape.zipf}) routing" if shape.zipf else "")),
            "layers": L,
            "tokens": shape.T,
            "experts": shape.E,
            "topk": shape.topk,
            "d": shape.d,
            "m": shape.m,
            "weight_layout": args.weight_layout,
            "row_block": row_block,
        },
        "us_per_layer": round(ms_per_step * 1e3, 2),
        "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_layer": layers[0]["bytes"]["layer"],
        "stage_us": stage_us,
        "from_router_logits": {
            "us_per_layer": routed_us["routed_forward"],
            "router_alone_us": routed_us["router_alone"],
            "note": ("dgw4_moe_forward_routed over the same steps: the router kernel "
                     "(top-8 of fp32 logits [T, E] and weights) before the layer"),
        },
        "eager_sweeps": spread,
        "graph_replay": graph,
        "hbm_probe": probe,
        "roofline": {
            "kernel": (f"layer_kernel<{str(args.weight_layout == 'tiled').lower()}> (alignment, "
                       f"gate_up + GELU(tanh) gate and down in one launch, layer shape, "
                       f"{args.weight_layout} weights)" if fused else
                       (f"align (128-row chunks), chunk_gate_up_kernel and chunk_down_kernel "
                        f"together ({args.weight_layout} weights)" if row_block == 128 else
                        f"align, gate_up and down launches together ({args.weight_layout} weights)")),
            "bound": "hbm",
            "achieved": round(kern_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kern_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic["bytes_per_launch"] if traffic else None,
            "bytes_per_launch": round(kern_bytes),
            "us_per_launch": round(kern_us, 2),
            "time_source": (f"HIP events on the launch stream around {S} back-to-back launches "
                            f"of the expert stages (dgw4_moe_experts) over the rotated layers"),
            "bytes_source": ("packed q + s + z of the populated experts plus x, per launch; "
                             "H, Y and alignment workspace traffic not counted"),
        },
        # the same launches against the fp16 MFMA peak: every assignment row
        # through gate_up (2m x d) and down (d x m), padding rows not counted
        "mfma": {
            "achieved": round(kern_flops / (kern_us * 1e-6) / 1e12, 1),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_flops / (kern_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "flops_per_launch": kern_flops,
            "note": "MfmaUtil per kernel (rocprofv3) is in profiles/expert_stages_workloads_utilisation_stack_skew_wide.md",
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(CONFIGS["full"])
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
