#!/usr/bin/env python3
"""Benchmark of the Q4_0 W4A8 MoE expert matmul on one MI355X.

Headline (the JSON `value`): decode weight bandwidth, in GB/s of expert weight
bytes touched, for one MoE layer at decode (T = 1 token, hidden 2048, 128
experts with gate/up 512x2048 and down 2048x512, top-8).  A step is one pass
of the whole path on fresh inputs: Q8_0 quantisation of the token, routing
(softmax, top-8, renormalisation, counting sort) and the decode layer.  The
expert weights rotate through R distinct resident copies (>= 1 GiB in total)
so that no step finds its weights in the 256 MB last-level cache.

The timed steps are captured into a HIP graph and replayed (the way a serving
loop issues a decode step), so the clock sees GPU work, not Python overhead.
`roofline` covers decode_fused_kernel, the one launch of a step, timed live
with HIP events on the launch stream around a graph of steps; `achievable`
holds the ceilings measured on the same GPU by the library's three probes (a
plain streaming read, an int8-MFMA-only loop, and the W4A8 prefill step on
registers: two int8 MFMAs and the fp32 scale FMAs of their outputs); `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.  `extra` reports the prefill grouped GEMM
(int8 TOPS on the 947-token and the skewed 4096-token workloads, and its W4A16
variant on the same routing), the router
projection in front of the routing, and the 40-layer decode stack.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, TOP/s
FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, TFLOP/s (the published figure counts packed fp32, not used here)
CAL_COPY_BYTES = 64 << 20  # counter calibration copy
METRIC = "W4A8 MoE decode weight GB/s (% of HBM peak); prefill grouped-GEMM int8 TOPS"


# HBM traffic per launch of a kernel, from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of this
# bench, each scaled by what the same counter reads for the plain 64 MiB copy that main() runs first (the
# summary and its commands are in profiles/).  A figure is valid only for the sources it was measured on
# (their SHA-256, in order), so a kernel edited since then reports null.
TRAFFIC = {
    # kernel: (source files, sha256 over their bytes, HBM bytes per launch)
    "decode_fused_kernel": (
        ['quantized_moe_q4_amd/csrc/fused.hip', 'quantized_moe_q4_amd/csrc/fused.h', 'quantized_moe_q4_amd/csrc/rows.h', 'quantized_moe_q4_amd/csrc/topk.h', 'quantized_moe_q4_amd/csrc/device.h'],
        "146cfc871f7bdb5c74bf7d158fed90e314577bc16de5a35533575005a5532e2f",
        14920459,
    ),
    "decode_stack_kernel": (  # one launch = the 40-layer stack at batch 1
        ['quantized_moe_q4_amd/csrc/stack.hip', 'quantized_moe_q4_amd/csrc/fused.h', 'quantized_moe_q4_amd/csrc/rows.h', 'quantized_moe_q4_amd/csrc/topk.h', 'quantized_moe_q4_amd/csrc/device.h'],
        "4bfa37a2c36cda5fd8453264a248197c381c2d06ee5a6b0903e3f55d0b251296",
        607516950,
    ),
}


def traffic_of(kernel: str):
    ent = TRAFFIC.get(kernel)
    if ent is None:
        return None
    import hashlib
    srcs, digest, nbytes = ent
    h = hashlib.sha256()
    try:
        for src in srcs:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    return nbytes if h.hexdigest() == digest else None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the expert matmul runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_moe_q4_amd as mq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def experts_dev(es):
        return mq.Experts(to_dev(es.gate_qs), to_dev(es.up_qs), to_dev(es.down_qs), to_dev(es.gate_d),
                          to_dev(es.up_d), to_dev(es.down_d))

    def clone(ex):
        return mq.Experts(*(t.clone() for t in (ex.gate_qs, ex.up_qs, ex.down_qs, ex.gate_d, ex.up_d, ex.down_d)))

    # A plain device copy of known size (64 MiB read + 64 MiB written), run first: in a rocprofv3 --pmc run
    # of this script, its FETCH_SIZE / WRITE_SIZE calibrate the counters for the kernels measured after it.
    cal_src = torch.ones(CAL_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    for _ in range(3):
        cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    ach = achievable(torch, mq, dev)
    log(f"achievable: HBM read {ach['hbm_read_gbs']:.0f} GB/s, int8 MFMA {ach['int8_mfma_tops']:.0f} TOPS, "
        f"W4A8 step {ach['w4a8_step_tops']:.0f} TOPS")

    # ---------------------------------------------------------------- headline: decode, workload 1
    w1 = synth.WORKLOADS[1]
    t0 = time.time()
    es = synth.expert_set(w1.seed, 0, w1.E, w1.H, w1.I)
    base = experts_dev(es)
    layer_bytes = base.nbytes
    expert_bytes = base.expert_bytes()
    R = args.copies or max(2, math.ceil((1 << 30) / layer_bytes) + 1)
    copies = [base] + [clone(base) for _ in range(R - 1)]
    S = args.warmup + args.steps
    X = to_dev(synth.normal(w1.seed, synth.x_tid(1) + (1 << 48), (S, 1, w1.H)))
    L = to_dev(synth.normal(w1.seed, synth.logits_tid(0, 1) + (1 << 48), (S, 1, w1.E)))
    k = w1.k
    xq = torch.empty((1, w1.H), dtype=torch.int8, device=dev)
    xd = torch.empty((1, w1.H // 32), dtype=torch.float32, device=dev)
    ids_all = torch.empty((S, 1, k), dtype=torch.int32, device=dev)
    w_all = torch.empty((S, 1, k), dtype=torch.float32, device=dev)
    off = torch.empty(w1.E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(k, dtype=torch.int32, device=dev)
    y = torch.empty((1, w1.H), dtype=torch.float32, device=dev)
    ws = mq.new_workspace(1, w1.E, k, w1.H, w1.I, dev)
    torch.cuda.synchronize()
    log(f"decode setup: {R} weight copies x {layer_bytes / 1e6:.1f} MB, {time.time() - t0:.1f} s")

    # One step = the whole hot path on one token: Q8_0 quantisation, routing,
    # gate/up + SwiGLU + re-quantisation, down and the weighted combine, as the
    # library's one-launch decode (moe_q4_decode_fused).
    def step(s):
        mq.decode_fused(copies[s % R], X[s], L[s], k, out=(ids_all[s], w_all[s], off, sp), y=y, ws=ws)

    # The same work as three calls (quantize_act, route, decode: four kernels), for comparison.
    def step3(s):
        mq.quantize_act(X[s], xq=xq, xd=xd)
        mq.route(L[s], k, out=(ids_all[s], w_all[s], off, sp))
        mq.decode(copies[s % R], xq, xd, ids_all[s], w_all[s], off, sp, y=y, ws=ws)

    for s in range(args.warmup):
        step(s)
        step3(s)
    torch.cuda.synchronize()
    # The timed steps are captured once into a HIP graph and replayed, so the
    # clock sees the GPU work of the steps rather than Python launch overhead.
    g_steps, g_three = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_steps):
        for i in range(args.steps):
            step(args.warmup + i)
    with torch.cuda.graph(g_three):
        for i in range(args.steps):
            step3(args.warmup + i)
    g_steps.replay()
    g_three.replay()
    torch.cuda.synchronize()
    if mq.workspace_error(ws):
        raise RuntimeError("fused decode: a bounded wait gave up (workspace error word set)")
    # events on the stream the graphs replay on (the current stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    ev[0].record()
    g_steps.replay()
    ev[1].record()
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[1])
    ev[2].record()
    g_three.replay()
    ev[3].record()
    torch.cuda.synchronize()
    three_ms = ev[2].elapsed_time(ev[3]) / args.steps
    ids_np = ids_all[args.warmup:].cpu().numpy()
    touched = np.array([len(np.unique(ids_np[i])) for i in range(args.steps)])
    bytes_steps = touched * expert_bytes
    ms_per_step = total_ms / args.steps
    value = float(bytes_steps.sum() / (total_ms * 1e-3) / 1e9)
    # one launch of decode_fused_kernel per step: its average duration is the step time
    achieved = float(bytes_steps.mean() / (ms_per_step * 1e-3) / 1e9)
    log(f"decode: {ms_per_step * 1e3:.2f} us/step fused ({value:.0f} GB/s); three calls "
        f"{three_ms * 1e3:.2f} us/step")
    del g_steps, g_three

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w1.name, "tokens": 1, "hidden": w1.H, "inter": w1.I, "experts": w1.E, "top_k": k,
                   "weight_copies_rotated": R, "bytes_per_expert": expert_bytes,
                   "step": "moe_q4_decode_fused (quantize + route + gate/up + SwiGLU + requant + down + combine)"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 3),
        "three_call_us_per_step": round(three_ms * 1e3, 3),
        "roofline": {
            "kernel": "decode_fused_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5),
            "traffic": traffic_of("decode_fused_kernel"),
            "avg_launch_us": round(ms_per_step * 1e3, 3),
            "algorithmic_bytes_per_launch": float(bytes_steps.mean()),
            "achievable": ach["hbm_read_gbs"],
            "frac_of_achievable": round(achieved / ach["hbm_read_gbs"], 5),
        },
        "achievable": ach,
    }
    del copies, base

    # ---------------------------------------------------------------- extras
    if not args.no_extra:
        result["extra"] = extras(args, np, torch, mq, synth, to_dev, experts_dev, clone, ach)

    # ---------------------------------------------------------------- CPU oracle beside it
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, np, synth, es, expert_bytes)

    print(json.dumps(result), flush=True)


def achievable(torch, mq, dev, read_bytes=1 << 30, reps=5):
    """Ceilings measured on this GPU: a plain streaming read of a buffer larger
    than every cache (best of `reps` calls) and back-to-back int8 MFMA on
    registers, eight workgroups of four waves per CU (best of `reps`)."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best_ms(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            t.append(ev[0].elapsed_time(ev[1]))
        return min(t)

    ms_read = best_ms(lambda: mq.probe_read(buf, sink))
    iters, wgs = 256, 8 * cus
    ops = 262144 * iters * 4 * wgs
    ms_mfma = best_ms(lambda: mq.probe_mfma_i8(iters, wgs, sink))
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    st_iters, st_wgs = 2048, 2 * cus
    st_ops = 131072 * st_iters * 4 * st_wgs
    ms_step = best_ms(lambda: mq.probe_w4a8_step(st_iters, st_wgs, fsink))
    del buf
    return {"hbm_read_gbs": round(read_bytes / (ms_read * 1e-3) / 1e9, 1),
            "int8_mfma_tops": round(ops / (ms_mfma * 1e-3) / 1e12, 1),
            "w4a8_step_tops": round(st_ops / (ms_step * 1e-3) / 1e12, 1),
            "probe": f"moe_q4_probe_read over {read_bytes >> 20} MiB; moe_q4_probe_mfma_i8 {iters} x 4 MFMA "
                     f"32x32x32 per wave, {wgs} workgroups of 4 waves; moe_q4_probe_w4a8_step {st_iters} steps "
                     f"(2 MFMA + 2 scale FMAs per output) per wave, {st_wgs} workgroups of 4 waves; best of {reps}"}


def extras(args, np, torch, mq, synth, to_dev, experts_dev, clone, ach):
    out = {}
    dev = torch.device("cuda:0")
    reps = 20
    for wi in (2, 3):
        w = synth.WORKLOADS[wi]
        t0 = time.time()
        es = synth.expert_set(w.seed, 0, w.E, w.H, w.I)
        base = experts_dev(es)
        R = max(2, math.ceil((1 << 30) / base.nbytes) + 1)
        copies = [base] + [clone(base) for _ in range(R - 1)]
        x = to_dev(synth.activations(w))
        lg = to_dev(synth.logits(w))
        xq, xd = mq.quantize_act(x)
        ids, wts, off, sp = mq.route(lg, w.k)
        y = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
        ws = torch.empty(mq.workspace_size(w.T, w.E, w.k, w.H, w.I), dtype=torch.uint8, device=dev)
        for i in range(3):
            mq.prefill(copies[i % R], xq, xd, ids, wts, off, sp, y=y, ws=ws)
        torch.cuda.synchronize()
        g_pf, g_st = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pf):
            for i in range(reps):
                mq.prefill(copies[i % R], xq, xd, ids, wts, off, sp, y=y, ws=ws)
        with torch.cuda.graph(g_st):
            for i in range(reps):
                mq.quantize_act(x, xq=xq, xd=xd)
                mq.route(lg, w.k, out=(ids, wts, off, sp))
                mq.prefill(copies[i % R], xq, xd, ids, wts, off, sp, y=y, ws=ws)
        g_pf.replay()
        g_st.replay()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        g_pf.replay()
        e[1].record()
        g_st.replay()
        e[2].record()
        torch.cuda.synchronize()
        pf_ms = e[0].elapsed_time(e[1]) / reps
        step_ms = e[1].elapsed_time(e[2]) / reps
        # the W4A16 variant of the same layer (fp16 activations, fp16 MFMA) on the same routing
        ws16 = torch.empty(mq.prefill_a16_workspace_size(w.T, w.k, w.H, w.I), dtype=torch.uint8, device=dev)
        for i in range(3):
            mq.prefill_a16(copies[i % R], x, ids, wts, off, sp, y=y, ws=ws16)
        torch.cuda.synchronize()
        g16 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g16):
            for i in range(reps):
                mq.prefill_a16(copies[i % R], x, ids, wts, off, sp, y=y, ws=ws16)
        g16.replay()
        torch.cuda.synchronize()
        e[0].record()
        g16.replay()
        e[1].record()
        torch.cuda.synchronize()
        a16_ms = e[0].elapsed_time(e[1]) / reps
        del g_pf, g_st, g16, ws16
        cnt = np.diff(off.cpu().numpy())
        ops = 2.0 * float(cnt.sum()) * 3 * w.H * w.I
        # what the MFMA tiles execute: every touched expert's rows padded to whole 32-row m-tiles (a row tile
        # runs as many m-tiles as its live rows need)
        padded_ops = 2.0 * float(((cnt + 31) // 32 * 32).sum()) * 3 * w.H * w.I
        touched = int((cnt > 0).sum())
        wbytes = touched * base.expert_bytes()
        tops = ops / (pf_ms * 1e-3) / 1e12
        out[w.name] = {"prefill_call_us": round(pf_ms * 1e3, 2), "step_us": round(step_ms * 1e3, 2),
                       "int8_tops": round(tops, 2), "pct_of_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
                       "pct_of_achievable_int8": round(100 * tops / ach["int8_mfma_tops"], 2),
                       "pct_of_w4a8_step_ceiling": round(100 * tops / ach["w4a8_step_tops"], 2),
                       "weight_gbs": round(wbytes / (pf_ms * 1e-3) / 1e9, 1),
                       "pct_of_hbm_peak": round(100 * wbytes / (pf_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                       "algorithmic_ops": ops, "padded_ops": padded_ops,
                       "w4a16": {"prefill_call_us": round(a16_ms * 1e3, 2),
                                 "fp16_tflops": round(ops / (a16_ms * 1e-3) / 1e12, 2),
                                 "pct_of_fp16_peak": round(100 * ops / (a16_ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 2),
                                 "weight_gbs": round(wbytes / (a16_ms * 1e-3) / 1e9, 1),
                                 "pct_of_hbm_peak": round(100 * wbytes / (a16_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
                       "experts_touched": touched, "max_tokens_per_expert": int(cnt.max()),
                       "weight_copies_rotated": R}
        log(f"prefill {w.name}: {pf_ms * 1e3:.1f} us, {tops:.1f} TOPS; W4A16 {a16_ms * 1e3:.1f} us; "
            f"setup {time.time() - t0:.1f} s")
        del copies, base

    # router projection (the step in front of the routing) at the decode and prefill shapes
    rl = {}
    for T, E in ((1, 128), (947, 128), (4096, 256)):
        H = 2048
        xr = to_dev(synth.normal(3, synth.x_tid(T), (T, H)))
        wrs = [to_dev(synth.router_weights(3, l, E, H)) for l in range(8)]  # 8 layers' weights rotate
        lo = torch.empty((T, E), dtype=torch.float32, device=dev)
        for i in range(3):
            mq.router_logits(xr, wrs[i % 8], flags=mq.QUANT_RMSNORM, out=lo)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        n = 40
        with torch.cuda.graph(g):
            for i in range(n):
                mq.router_logits(xr, wrs[i % 8], flags=mq.QUANT_RMSNORM, out=lo)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        flops = 2.0 * T * E * H
        nbytes = 4.0 * (E * H + T * H + T * E)
        rl[f"T{T}_E{E}_H{H}"] = {"us": round(us, 2), "gflops": round(flops / (us * 1e-6) / 1e9, 1),
                                 "pct_of_fp32_vector_peak": round(100 * flops / (us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS, 2),
                                 "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log(f"router logits T={T} E={E}: {us:.2f} us")
        del g, wrs
    out["router_logits_fp32"] = rl

    # 40-layer decode stack at batch 1, 4, 16
    w4 = synth.WORKLOADS[4]
    t0 = time.time()
    layers = [experts_dev(synth.expert_set(w4.seed, l, w4.E, w4.H, w4.I)) for l in range(w4.layers)]
    log(f"stack setup {time.time() - t0:.1f} s")
    eb = layers[0].expert_bytes()
    stack = {}
    for T in synth.STACK_BATCHES:
        h0 = to_dev(synth.normal(w4.seed, synth.x_tid(T), (T, w4.H)))
        lgs = [to_dev(synth.normal(w4.seed, synth.logits_tid(l, T), (T, w4.E))) for l in range(w4.layers)]
        k = w4.k
        xq = torch.empty((T, w4.H), dtype=torch.int8, device=dev)
        xd = torch.empty((T, w4.H // 32), dtype=torch.float32, device=dev)
        routes = [(torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32,
                                                                                   device=dev),
                   torch.empty(w4.E + 1, dtype=torch.int32, device=dev),
                   torch.empty(T * k, dtype=torch.int32, device=dev)) for _ in range(w4.layers)]
        ws = mq.new_workspace(T, w4.E, k, w4.H, w4.I, dev)
        h = h0.clone()

        def run_stack(fused):
            h.copy_(h0)
            for l in range(w4.layers):
                if fused:  # one launch per layer, residual stream updated in place
                    mq.decode_fused(layers[l], h, lgs[l], k, flags=mq.QUANT_RMSNORM | mq.ACCUMULATE,
                                    out=routes[l], y=h, ws=ws)
                    continue
                mq.quantize_act(h, flags=mq.QUANT_RMSNORM, xq=xq, xd=xd)
                r = mq.route(lgs[l], k, out=routes[l])
                mq.decode(layers[l], xq, xd, *r, flags=mq.ACCUMULATE, y=h, ws=ws)

        timed, eager = {}, {}
        one_launch_traffic = None
        for fused in ([True, False] if T <= mq.MAX_FUSED_TOKENS else [False]):
            name = "decode_fused" if fused else "quantize_act + route + decode"
            run_stack(fused)
            torch.cuda.synchronize()
            # eager: the same step issued call by call from Python (launch overhead included)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run_stack(fused)
            b.record()
            torch.cuda.synchronize()
            eager[name] = a.elapsed_time(b)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_stack(fused)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 5
            a.record()
            for _ in range(n):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            timed[name] = a.elapsed_time(b) / n
            del g
        if T == 1:
            # the whole stack in one launch (moe_q4_decode_stack): one call per step, timed by events around
            # n calls (a cooperative launch, not captured in a graph)
            lg_all = torch.stack([t.reshape(-1) for t in lgs])
            sws = mq.new_stack_workspace(w4.H, dev)
            hs = h0.clone().reshape(-1)
            stl = mq.StackLayers(layers)  # pointers checked and packed once

            def run_one_launch():
                hs.copy_(h0.reshape(-1))
                mq.decode_stack(stl, hs, lg_all, k, flags=mq.QUANT_RMSNORM | mq.ACCUMULATE, ws=sws)

            run_one_launch()
            torch.cuda.synchronize()
            name = "decode_stack (one launch)"
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 10
            a.record()
            for _ in range(n):
                run_one_launch()
            b.record()
            torch.cuda.synchronize()
            timed[name] = eager[name] = a.elapsed_time(b) / n
            if mq.workspace_error(sws) != 0:
                raise RuntimeError("decode_stack: a bounded wait gave up")
            one_launch_traffic = traffic_of("decode_stack_kernel")
        path = min(timed, key=timed.get)
        ms = timed[path]
        touched = sum(int((np.diff(r[2].cpu().numpy()) > 0).sum()) for r in routes)
        gbs = touched * eb / (ms * 1e-3) / 1e9
        stack[f"T{T}"] = {"step_ms": round(ms, 4), "weight_gbs": round(gbs, 1),
                          "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                          "pct_of_achievable_hbm": round(100 * gbs / ach["hbm_read_gbs"], 2), "experts_touched": touched,
                          "path": path, "step_ms_by_path": {p: round(v, 4) for p, v in timed.items()},
                          "eager_step_ms_by_path": {p: round(v, 4) for p, v in eager.items()}}
        if T == 1:  # HBM bytes per launch of the one-launch stack from the counter runs (null when stale)
            stack[f"T{T}"]["one_launch_hbm_bytes"] = one_launch_traffic
        log(f"stack T={T}: {ms:.3f} ms/step, {gbs:.0f} GB/s")
    out[w4.name] = stack
    return out


def cpu_baseline(args, np, synth, es, expert_bytes):
    """The CPU oracle, as it stands, on a bounded sample of the decode workload (one host thread)."""
    import oracle

    w1 = synth.WORKLOADS[1]
    n = 0
    nbytes = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.cpu_seconds:
        x = synth.normal(w1.seed, synth.x_tid(1) + (1 << 48), (1, w1.H), start=n * w1.H)
        lg = synth.normal(w1.seed, synth.logits_tid(0, 1) + (1 << 48), (1, w1.E), start=n * w1.E)
        xq, xd = oracle.q8_quantize(x)
        ids, w, off, sp = oracle.route(lg, w1.k)
        oracle.moe_layer(es, xq, xd, ids, w)
        nbytes += len(np.unique(ids)) * expert_bytes
        n += 1
    dt = time.perf_counter() - t0
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} decode steps of {w1.name} (quantize + route + layer, one token each), {dt:.1f} s",
            "host_cpu": cpu, "host_logical_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
